"""fa_decode_paged_noalloc, the decode entry point that allocates nothing:
two calls in a row through the C ABI (the second on a smaller batch, with
another head dimension and dtype) give bitwise the outputs of
fa_decode_paged with a caller workspace, and both match the fp64 oracle.
The second call reuses the device buffer the first one filled."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.util import assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def check_against_workspace_call(x: fi.Paged, num_splits, what):
    print(f"[case] {what}: B={len(x.seq_lens)} max_pages={x.max_pages} splits={num_splits}",
          flush=True)
    q, kp, vp = to_dev(x.q, x.dtype), to_dev(x.k_pool, x.dtype), to_dev(x.v_pool, x.dtype)
    pt, sl = to_dev(x.page_table, "i32"), to_dev(x.seq_lens, "i32")
    B, Hq, d = x.q.shape
    need = fa.decode_workspace_size(B, Hq, d, x.max_pages, 16, num_splits)
    assert 0 < need <= fa._lib.DECODE_NOALLOC_MAX_WORKSPACE
    o_n = torch.full_like(q, float("nan"))
    l_n = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    fa.decode_paged_noalloc(q, kp, vp, pt, sl, num_splits=num_splits, scale=x.scale, out=o_n,
                            lse=l_n)
    o_w, l_w = fa.decode_paged(q, kp, vp, pt, sl, num_splits=num_splits, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), f"{what}: differs from fa_decode_paged"
    O, L = oracle.decode(fi.to_f64(x.q, x.dtype), fi.to_f64(x.k_seq, x.dtype),
                         fi.to_f64(x.v_seq, x.dtype), x.cu_k, x.scale)
    assert_parity(to_f64(o_n), to_f64(l_n), O, L, fi.to_f64(x.v_seq, x.dtype), x.dtype, what)


def test_noalloc_decode_two_calls_second_smaller():
    rng = np.random.default_rng(90)
    lens = rng.integers(1, 12000, 24, endpoint=True)
    lens[3] = 0
    big = fi.paged(lens, 32, 8, 128, "bf16", seed=90)
    check_against_workspace_call(big, 0, "noalloc call 1 (bf16 d128, 24 sequences)")
    small = fi.paged([5, 0, 300, 17], 8, 2, 64, "f16", seed=91)
    check_against_workspace_call(small, 2, "noalloc call 2 (f16 d64, 4 sequences)")


def test_noalloc_decode_rejects_requests_beyond_its_buffer():
    pool = torch.zeros(4, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(128, 64, 128, dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros(128, 2017, dtype=torch.int32, device="cuda")
    sl = torch.ones(128, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(fa.FaError) as e:
        fa.decode_paged_noalloc(q, pool, pool, pt, sl, out=o)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
