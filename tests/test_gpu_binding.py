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


# ---- empty tensors: a zero-element torch tensor has a NULL data pointer ----
def test_empty_tensors_through_the_binding():
    # kv_append with no new tokens leaves the pools as they were
    pool = torch.randn(4, 16, 2, 64, device="cuda").to(torch.bfloat16)
    before = pool.clone()
    empty = dev_tensor(0, 2, 64)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    pt = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    lb = torch.zeros(2, dtype=torch.int32, device="cuda")
    fa.kv_append(empty, empty, pool, pool, cu, pt, lb)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    # ragged call with no query row: nothing to do, empty outputs
    cq = torch.zeros(3, dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, 5, 9], dtype=torch.int32, device="cuda")
    o, l = fa.fwd_varlen(dev_tensor(0, 4, 64), dev_tensor(9, 2, 64), dev_tensor(9, 2, 64),
                         cq, ck, 0, 5, causal=True)
    assert o.shape == (0, 4, 64) and l.shape == (0, 4)
    # ragged call with no key at all: every row O = 0, LSE = -inf
    cq = torch.tensor([0, 3, 7], dtype=torch.int32, device="cuda")
    ck = torch.zeros(3, dtype=torch.int32, device="cuda")
    q = torch.randn(7, 4, 64, device="cuda").to(torch.bfloat16)
    for causal in (False, True):
        o, l = fa.fwd_varlen(q, dev_tensor(0, 2, 64), dev_tensor(0, 2, 64), cq, ck, 4, 0,
                             causal=causal)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(l == float("-inf"))


# ---- FA_DEBUG_VALIDATE: bad device index arrays rejected before launch ----
@pytest.fixture
def debug_validate(monkeypatch):
    monkeypatch.setenv("FA_DEBUG_VALIDATE", "1")


def test_debug_validate_rejects_bad_index_arrays(debug_validate):
    dev = "cuda"
    q = torch.randn(10, 4, 64, device=dev).to(torch.bfloat16)
    k = torch.randn(10, 2, 64, device=dev).to(torch.bfloat16)
    good = torch.tensor([0, 3, 10], dtype=torch.int32, device=dev)
    o_ok, l_ok = fa.fwd_varlen(q, k, k, good, good, 7, 7, causal=True)
    for bad in ([0, 5, 4], [1, 3, 10], [0, 3, 9]):
        cu = torch.tensor(bad, dtype=torch.int32, device=dev)
        out = torch.full_like(q, 7.0)
        with pytest.raises(fa.FaError) as e:
            fa.fwd_varlen(q, k, k, cu, good, 7, 7, causal=True, out=out)
        assert e.value.status == 1
        assert torch.all(out == 7.0)  # nothing was launched
    # a run longer than max_seqlen_q
    with pytest.raises(fa.FaError):
        fa.fwd_varlen(q, k, k, good, good, 6, 7, causal=True)
    # paged decode: a page entry outside the pool, a length past the table row
    pool = torch.randn(5, 16, 2, 64, device=dev).to(torch.bfloat16)
    qd = torch.randn(2, 4, 64, device=dev).to(torch.bfloat16)
    pt = torch.tensor([[4, 0, -1], [2, -1, -1]], dtype=torch.int32, device=dev)
    sl = torch.tensor([17, 16], dtype=torch.int32, device=dev)
    o1, l1 = fa.decode_paged(qd, pool, pool, pt, sl)
    with pytest.raises(fa.FaError):
        fa.decode_paged(qd, pool, pool, torch.tensor([[5, 0, -1], [2, -1, -1]], dtype=torch.int32,
                                                     device=dev), sl)
    with pytest.raises(fa.FaError):
        fa.decode_paged(qd, pool, pool, pt, torch.tensor([49, 1], dtype=torch.int32, device=dev))
    with pytest.raises(fa.FaError):
        fa.decode_paged(qd, pool, pool, pt, torch.tensor([33, 1], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    # the check changes nothing for valid arrays
    o2, l2 = fa.fwd_varlen(q, k, k, good, good, 7, 7, causal=True)
    assert torch.equal(o_ok, o2) and torch.equal(l_ok, l2)
