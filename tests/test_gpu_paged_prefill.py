"""GPU parity of the chunked prefill over a paged cache (fa_fwd_paged):
the fp64 oracle sees each sequence's contiguous K/V (no page table), and
bitwise checks tie the paged path to the contiguous ragged path."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests import full_oracle
from tests.util import assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def dev_inputs(x: fi.PagedPrefill):
    kv = x.kv
    return (to_dev(x.q, kv.dtype), to_dev(kv.k_pool, kv.dtype), to_dev(kv.v_pool, kv.dtype),
            to_dev(x.cu_q, "i32"), to_dev(kv.page_table, "i32"), to_dev(kv.seq_lens, "i32"))


def run(x: fi.PagedPrefill, causal=True):
    q, kp, vp, cq, pt, sl = dev_inputs(x)
    o, l = fa.fwd_paged(q, kp, vp, cq, pt, sl, x.max_q, causal=causal, scale=x.kv.scale)
    torch.cuda.synchronize()
    return o, l


def oracle_all(x: fi.PagedPrefill, causal=True):
    kv = x.kv
    return oracle.attention_varlen(fi.to_f64(x.q, kv.dtype), fi.to_f64(kv.k_seq, kv.dtype),
                                   fi.to_f64(kv.v_seq, kv.dtype), x.cu_q, kv.cu_k, kv.scale, causal)


def check(x: fi.PagedPrefill, what, causal=True):
    print(f"[case] {what} B={len(x.kv.seq_lens)} causal={causal}", flush=True)
    o, l = run(x, causal)
    o, l = to_f64(o), to_f64(l)
    assert np.all(np.isfinite(o))
    O, L = oracle_all(x, causal)
    return assert_parity(o, l, O, L, fi.to_f64(x.kv.v_seq, x.kv.dtype), x.kv.dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_paged_prefill_small(dtype, d, G):
    # chunk = whole sequence, chunk after a prefix, one-token chunk, empty
    # chunk, lengths off page and tile boundaries, several query tiles
    lq = [37, 0, 1, 300, 16, 5]
    lk = [37, 9, 700, 611, 16, 1029]
    x = fi.paged_prefill(lq, lk, 2 * G, 2, d, dtype, seed=60 + G + d)
    check(x, f"paged prefill small {dtype} d{d} G{G}")


def test_paged_prefill_non_causal():
    x = fi.paged_prefill([70, 200, 3], [70, 513, 1000], 8, 2, 128, "bf16", seed=61)
    check(x, "paged prefill non-causal", causal=False)


def test_chunked_prefill_batch_full():
    """16 sequences: cached prefix U[0,8192] + chunk U[1,2048]; every row of
    every query head of every chunk against the fp64 oracle on the
    contiguous keys."""
    lq, lk = fi.chunked_prefill_lengths()
    x = fi.paged_prefill(lq, lk, 32, 8, 128, "bf16", seed=5)
    print(f"[case] chunked prefill batch full Tq={len(x.q)} keys={int(lk.sum())}", flush=True)
    o, l = run(x)
    o, l = to_f64(o), to_f64(l)
    assert np.all(np.isfinite(o))
    kv = x.kv
    O, L = full_oracle.varlen_all(x.q, kv.k_seq, kv.v_seq, x.cu_q, kv.cu_k, "bf16", kv.scale, True)
    vmax = np.abs(fi.to_f64(kv.v_seq, "bf16")).max()
    assert_parity(o, l, O, L, np.array([vmax]), "bf16", "chunked prefill batch full")


def test_paged_equals_contiguous_varlen_bitwise():
    """Same queries and keys through the page table and as contiguous ragged
    K/V: the kernel does the same arithmetic, so the outputs are identical."""
    lq = [300, 1, 77, 0, 512]
    lk = [900, 40, 77, 16, 2000]
    x = fi.paged_prefill(lq, lk, 16, 4, 128, "bf16", seed=62)
    o_p, l_p = run(x)
    kv = x.kv
    o_v, l_v = fa.fwd_varlen(to_dev(x.q, "bf16"), to_dev(kv.k_seq, "bf16"), to_dev(kv.v_seq, "bf16"),
                             to_dev(x.cu_q, "i32"), to_dev(kv.cu_k, "i32"), x.max_q,
                             int(np.max(kv.seq_lens)), causal=True, scale=kv.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_v) and torch.equal(l_p, l_v)


def test_page_permutation_and_poison_bitwise():
    lq, lk = [20, 130, 1], [50, 130, 333]
    a = fi.paged_prefill(lq, lk, 8, 2, 64, "bf16", seed=63, permute=False)
    b = fi.paged_prefill(lq, lk, 8, 2, 64, "bf16", seed=63, permute=True)
    c = fi.paged_prefill(lq, lk, 8, 2, 64, "bf16", seed=63, permute=True, tail_fill="nan")
    oa, la = run(a)
    ob, lb = run(b)
    oc, lc = run(c)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(ob, oc) and torch.equal(lb, lc)
    assert not torch.isnan(oc).any()


def test_paged_prefill_at_the_page_table_limit():
    """A sequence of 8192 pages (131072 keys), the most one page-table row
    staged in LDS may hold, beside a short one; the chunk is the last 64
    tokens. max_pages = 8193 is refused before any launch."""
    x = fi.paged_prefill([64, 300], [131072, 300], 2, 1, 128, "bf16", seed=64)
    assert x.kv.page_table.shape[1] == 8192
    check(x, "paged prefill at 8192 pages per sequence")
    q, kp, vp, cq, pt, sl = dev_inputs(x)
    wide = torch.full((2, 8193), -1, dtype=torch.int32, device="cuda")
    wide[:, :8192] = pt
    with pytest.raises(RuntimeError):
        fa.fwd_paged(q, kp, vp, cq, wide, sl, x.max_q, causal=True, scale=x.kv.scale)
