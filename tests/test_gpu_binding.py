"""The Python binding's checks: mismatched shapes, head dimensions, dtypes
and devices raise ValueError before anything is launched (the C ABI sees
only pointers and sizes, so these are the checks that keep a wrong tensor
from being read or written out of bounds)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def dev_tensor(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype, device="cuda")


def test_fwd_rejects_bad_outputs():
    q, k, v = dev_tensor(1, 64, 4, 64), dev_tensor(1, 64, 2, 64), dev_tensor(1, 64, 2, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, out=dev_tensor(1, 64, 4, 32))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, lse=dev_tensor(1, 64, 4))  # not float32
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, lse=torch.zeros(1, 64, 4, dtype=torch.float32))  # on the host
    with pytest.raises(ValueError):
        fa.fwd(q, dev_tensor(1, 64, 2, 128), dev_tensor(1, 64, 2, 128))  # head dim


def test_varlen_and_paged_reject_head_dim_mismatch():
    cu = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_varlen(dev_tensor(64, 4, 64), dev_tensor(64, 2, 128), dev_tensor(64, 2, 128),
                      cu, cu, 64, 64)
    pool = dev_tensor(8, 16, 2, 128)
    pt = torch.zeros(1, 8, dtype=torch.int32, device="cuda")
    sl = torch.tensor([100], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_paged(dev_tensor(4, 4, 64), pool, pool, torch.tensor([0, 4], dtype=torch.int32,
                                                                      device="cuda"), pt, sl, 4)
    with pytest.raises(ValueError):
        fa.decode_paged(dev_tensor(1, 4, 64), pool, pool, pt, sl)
    with pytest.raises(ValueError):
        fa.decode_cascade(dev_tensor(1, 4, 64), pool, pool, None, 0, pt, sl)


def test_decode_rejects_host_workspace_and_bad_lse():
    pool = dev_tensor(8, 16, 2, 128)
    pt = torch.zeros(1, 8, dtype=torch.int32, device="cuda")
    sl = torch.tensor([100], dtype=torch.int32, device="cuda")
    q = dev_tensor(1, 4, 128)
    with pytest.raises(ValueError):
        fa.decode_paged(q, pool, pool, pt, sl, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fa.decode_paged(q, pool, pool, pt, sl, lse=torch.zeros(1, 3, dtype=torch.float32,
                                                               device="cuda"))
