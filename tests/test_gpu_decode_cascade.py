"""GPU parity of the shared-prefix (cascade) decode, fa_decode_cascade: the
fp64 oracle decodes each sequence over its contiguous prefix + suffix keys."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests import full_oracle
from tests.util import assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def run(x: fi.Cascade):
    p = x.pool
    pp = to_dev(x.prefix_pages, "i32") if x.prefix_len > 0 else None
    o, l = fa.decode_cascade(to_dev(x.q, p.dtype), to_dev(p.k_pool, p.dtype), to_dev(p.v_pool, p.dtype),
                             pp, x.prefix_len, to_dev(x.page_table, "i32"), to_dev(x.seq_lens, "i32"),
                             scale=p.scale)
    torch.cuda.synchronize()
    return o, l


def oracle_for(x: fi.Cascade, seqs):
    dt = x.pool.dtype
    ks = [fi.to_f64(x.keys(b, "k"), dt) for b in seqs]
    vs = [fi.to_f64(x.keys(b, "v"), dt) for b in seqs]
    cu = np.concatenate([[0], np.cumsum([len(a) for a in ks])]).astype(np.int64)
    O, L = oracle.decode(fi.to_f64(x.q[seqs], dt), np.concatenate(ks), np.concatenate(vs), cu,
                         x.pool.scale)
    return O, L, np.concatenate([v.ravel() for v in vs] + [np.zeros(1)])


def check(x: fi.Cascade, what, seqs=None):
    print(f"[case] {what} B={len(x.seq_lens)} prefix={x.prefix_len}", flush=True)
    o, l = run(x)
    o, l = to_f64(o), to_f64(l)
    seqs = list(range(len(x.seq_lens))) if seqs is None else list(seqs)
    O, L, v_read = oracle_for(x, seqs)
    return assert_parity(o[seqs], l[seqs], O, L, v_read, x.pool.dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("prefix", [1, 100, 1024])
def test_cascade_small(dtype, d, G, prefix):
    x = fi.cascade(prefix, [0, 1, 17, 300, 64, 1000, 5], 2 * G, 2, d, dtype, seed=80 + G + prefix)
    check(x, f"cascade {dtype} d{d} G{G} prefix{prefix}")


def test_cascade_without_prefix_equals_paged_decode_bitwise():
    """With an empty prefix the cascade is the paged decode with the same
    split layout: its suffix splits are 8 pages, so the paged decode is asked
    for splits of 8 pages too."""
    x = fi.cascade(0, [40, 3000, 1, 0, 700], 16, 4, 128, "bf16", seed=81)
    o1, l1 = run(x)
    p = x.pool
    max_pages = x.page_table.shape[1]
    ns = -(-max_pages // 8)
    assert -(-max_pages // ns) == 8
    o2, l2 = fa.decode_paged(to_dev(x.q, "bf16"), to_dev(p.k_pool, "bf16"), to_dev(p.v_pool, "bf16"),
                             to_dev(x.page_table, "i32"), to_dev(x.seq_lens, "i32"), num_splits=ns,
                             scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cascade_matches_decode_over_aliased_page_tables():
    """Sequences whose page tables begin with the same prefix pages, decoded
    the plain way, agree with the cascade (different split structure: equal
    within the bf16 bound of each other and of the oracle)."""
    x = fi.cascade(512, [1, 200, 33], 32, 8, 128, "bf16", seed=82)
    o_c, l_c = run(x)
    pre = x.prefix_pages
    B = len(x.seq_lens)
    mp = len(pre) + x.page_table.shape[1]
    pt = np.full((B, mp), -1, np.int32)
    for b in range(B):
        pt[b, :len(pre)] = pre
        pt[b, len(pre):] = x.page_table[b]
    sl = (x.seq_lens + x.prefix_len).astype(np.int32)
    p = x.pool
    o_d, l_d = fa.decode_paged(to_dev(x.q, "bf16"), to_dev(p.k_pool, "bf16"), to_dev(p.v_pool, "bf16"),
                               to_dev(pt, "i32"), to_dev(sl, "i32"), scale=p.scale)
    torch.cuda.synchronize()
    vmax = np.abs(fi.to_f64(p.v_seq, "bf16")).max()
    assert np.abs(to_f64(o_c) - to_f64(o_d)).max() / vmax <= 1e-2
    assert np.abs(to_f64(l_c) - to_f64(l_d)).max() <= 1e-4 * max(1.0, np.abs(to_f64(l_d)).max())
    check(x, "cascade vs aliased tables")


def test_cascade_shared_prompt_batch_full():
    """64 sequences sharing a 16384-token prefix, suffixes U[1, 2048]: every
    sequence and query head against the fp64 oracle over prefix + suffix."""
    rng = np.random.default_rng(83)
    suf = rng.integers(1, 2048, 64, endpoint=True)
    x = fi.cascade(16384, suf, 32, 8, 128, "bf16", seed=83)
    print("[case] cascade shared prompt full", flush=True)
    o, l = run(x)
    o, l = to_f64(o), to_f64(l)
    O, L = full_oracle.decode_all(x.q, lambda b: x.keys(b, "k"), lambda b: x.keys(b, "v"), "bf16",
                                  x.pool.scale)
    vmax = np.abs(fi.to_f64(x.pool.v_seq, "bf16")).max()
    assert_parity(o, l, O, L, np.array([vmax]), "bf16", "cascade shared prompt full")
