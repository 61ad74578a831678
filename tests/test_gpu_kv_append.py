"""GPU tests of appending tokens to the paged cache (fa_kv_append): bit-exact
against the plain oracle, and end to end with the paged decode."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def split_case(full_lens, before, dtype, seed, Hkv=2, d=128):
    """Full sequences in a pool; the last full-before tokens of each are the
    new ones, and their slots start as NaN (not yet written)."""
    full_lens, before = np.asarray(full_lens), np.asarray(before)
    x = fi.paged(full_lens, 4 * Hkv, Hkv, d, dtype, seed, permute=True, tail_fill="nan")
    new_k = np.concatenate([x.k_seq[x.cu_k[s] + before[s]:x.cu_k[s + 1]] for s in range(len(full_lens))])
    new_v = np.concatenate([x.v_seq[x.cu_k[s] + before[s]:x.cu_k[s + 1]] for s in range(len(full_lens))])
    cu_new = np.concatenate([[0], np.cumsum(full_lens - before)]).astype(np.int32)
    nan = fi.paged([1], 1, 1, 8, dtype, 0, tail_fill="nan").k_pool.reshape(-1)[-1]
    k_before, v_before = x.k_pool.copy(), x.v_pool.copy()
    for s in range(len(full_lens)):
        for t in range(before[s], full_lens[s]):
            pg, sl = x.page_table[s, t // 16], t % 16
            k_before[pg, sl] = nan
            v_before[pg, sl] = nan
    return x, new_k, new_v, cu_new, before.astype(np.int32), k_before, v_before


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if a.dtype.itemsize == 2 else np.uint32)


def dev_bits(t):
    return bits(t.cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy())


@pytest.mark.parametrize("dtype,Hkv,d,n", [("bf16", 2, 128, 6), ("f16", 2, 128, 6),
                                          ("f32", 2, 128, 6), ("bf16", 1, 64, 41),
                                          ("f32", 8, 128, 41)])
def test_append_bit_exact_against_oracle(dtype, Hkv, d, n):
    """Rows of 128 B to 4 KB (one 16-byte piece per lane for up to 64 pieces,
    more pieces per lane beyond); 6 or 41 sequences, and a token count that
    is not a multiple of the four tokens a workgroup takes."""
    if n == 6:
        full = [1, 17, 16, 300, 45, 0]
        before = [0, 16, 3, 299, 0, 0]
    else:
        rng = np.random.default_rng(71)
        full = rng.integers(0, 120, n)
        before = np.minimum(full, rng.integers(0, 60, n))
    x, nk, nv, cu, lb, kb, vb = split_case(full, before, dtype, seed=70, Hkv=Hkv, d=d)
    print(f"[case] kv append {dtype} T_new={len(nk)}", flush=True)
    kp, vp = to_dev(kb, dtype), to_dev(vb, dtype)
    fa.kv_append(to_dev(nk, dtype), to_dev(nv, dtype), kp, vp, to_dev(cu, "i32"),
                 to_dev(x.page_table, "i32"), to_dev(lb, "i32"))
    torch.cuda.synchronize()
    want_k = oracle.cache_append(kb, nk, cu, x.page_table, lb)
    want_v = oracle.cache_append(vb, nv, cu, x.page_table, lb)
    assert np.array_equal(dev_bits(kp), bits(want_k))
    assert np.array_equal(dev_bits(vp), bits(want_v))
    # and the result is the generator's full pool (unwritten tail slots stay NaN)
    assert np.array_equal(dev_bits(kp), bits(x.k_pool)) and np.array_equal(dev_bits(vp), bits(x.v_pool))


def test_append_then_decode_equals_full_pool_decode():
    full = [513, 40, 1, 2000]
    before = [500, 0, 0, 1999]
    x, nk, nv, cu, lb, kb, vb = split_case(full, before, "bf16", seed=71, Hkv=2, d=128)
    q = to_dev(x.q, "bf16")
    pt, sl = to_dev(x.page_table, "i32"), to_dev(x.seq_lens, "i32")
    kp, vp = to_dev(kb, "bf16"), to_dev(vb, "bf16")
    fa.kv_append(to_dev(nk, "bf16"), to_dev(nv, "bf16"), kp, vp, to_dev(cu, "i32"), pt, to_dev(lb, "i32"))
    o1, l1 = fa.decode_paged(q, kp, vp, pt, sl, scale=x.scale)
    o2, l2 = fa.decode_paged(q, to_dev(x.k_pool, "bf16"), to_dev(x.v_pool, "bf16"), pt, sl, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_append_skips_positions_outside_the_table():
    """Tokens whose page-table entry is -1 or past the pool, or whose position
    is past max_pages*16, are not written; nothing else changes."""
    x = fi.paged([32, 16], 4, 2, 64, "bf16", seed=72, permute=False)
    pt = x.page_table.copy()          # [[0, 1], [2, -1]] -> make entries invalid
    pt[0, 1] = -1                     # sequence 0, positions 16..31
    pt[1, 0] = x.k_pool.shape[0] + 5  # sequence 1, positions 0..15: page past the pool
    new = fi.round_to(np.ones((3, 2, 64), np.float32) * 7.0, "bf16")
    cu = np.array([0, 2, 3], np.int32)       # seq 0 gets 2 tokens, seq 1 gets 1
    lb = np.array([16, 0], np.int32)         # seq 0 at positions 16, 17; seq 1 at 0
    kp, vp = to_dev(x.k_pool, "bf16"), to_dev(x.v_pool, "bf16")
    fa.kv_append(to_dev(new, "bf16"), to_dev(new, "bf16"), kp, vp, to_dev(cu, "i32"),
                 to_dev(pt, "i32"), to_dev(lb, "i32"))
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(kp), bits(x.k_pool)) and np.array_equal(dev_bits(vp), bits(x.v_pool))
    # a position past max_pages * 16 = 32
    lb2 = np.array([40, 0], np.int32)
    cu2 = np.array([0, 1, 1], np.int32)
    fa.kv_append(to_dev(new[:1], "bf16"), to_dev(new[:1], "bf16"), kp, vp, to_dev(cu2, "i32"),
                 to_dev(x.page_table, "i32"), to_dev(lb2, "i32"))
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(kp), bits(x.k_pool))
