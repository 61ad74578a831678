"""GPU parity of the paged split-KV decode (fa_decode_paged) against the
fp64 CPU oracle, which sees each sequence's contiguous K/V and no page
table, plus bitwise checks of the page-table handling."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests import full_oracle
from tests.util import assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")


def dev_paged(x: fi.Paged):
    return (to_dev(x.q, x.dtype), to_dev(x.k_pool, x.dtype), to_dev(x.v_pool, x.dtype),
            to_dev(x.page_table, "i32"), to_dev(x.seq_lens, "i32"))


def run(x: fi.Paged, num_splits=0, dev=None):
    q, kp, vp, pt, sl = dev if dev is not None else dev_paged(x)
    o, l = fa.decode_paged(q, kp, vp, pt, sl, num_splits=num_splits, scale=x.scale)
    torch.cuda.synchronize()
    return o, l


def oracle_for(x: fi.Paged, seqs):
    """fp64 oracle of the sampled sequences, fed their contiguous K/V."""
    k = [fi.to_f64(x.k_seq[x.cu_k[b]:x.cu_k[b + 1]], x.dtype) for b in seqs]
    v = [fi.to_f64(x.v_seq[x.cu_k[b]:x.cu_k[b + 1]], x.dtype) for b in seqs]
    cu = np.concatenate([[0], np.cumsum([len(a) for a in k])]).astype(np.int64)
    shape = (0,) + x.k_seq.shape[1:]
    k = np.concatenate(k) if k else np.zeros(shape)
    v = np.concatenate(v) if v else np.zeros(shape)
    O, L = oracle.decode(fi.to_f64(x.q[seqs], x.dtype), k, v, cu, x.scale)
    return O, L, v


def check(x: fi.Paged, what, seqs=None, num_splits=0, dev=None):
    print(f"[case] {what} B={len(x.seq_lens)} splits={num_splits}", flush=True)
    o, l = run(x, num_splits, dev)
    o, l = to_f64(o), to_f64(l)
    seqs = list(range(len(x.seq_lens))) if seqs is None else list(seqs)
    O, L, v_read = oracle_for(x, seqs)
    return assert_parity(o[seqs], l[seqs], O, L, np.concatenate([v_read.ravel(), [0.0]]),
                         x.dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 6])
def test_decode_small(dtype, d, G):
    lens = [1, 15, 16, 17, 33, 512, 700, 1025]
    x = fi.paged(lens, 2 * G, 2, d, dtype, seed=40 + G + d)
    check(x, f"decode small {dtype} d{d} G{G}")


@pytest.mark.parametrize("num_splits", [1, 2, 7, 0])
def test_decode_split_counts(num_splits):
    lens = [100, 3000, 4096, 1]
    x = fi.paged(lens, 32, 8, 128, "bf16", seed=41)
    check(x, f"decode splits={num_splits}", num_splits=num_splits)


def test_decode_many_sequences():
    """300 sequences of 0..699 tokens, about 15% of them empty: a grid of
    many short split items, empty sequences giving O = 0 and LSE = -inf, and
    the split merge of every non-empty one."""
    rng = np.random.default_rng(46)
    lens = rng.integers(0, 700, 300)
    lens[rng.random(300) < 0.15] = 0
    x = fi.paged(lens, 8, 2, 128, "bf16", seed=46)
    o, l = run(x)
    empty = np.flatnonzero(lens == 0)
    assert np.all(to_f64(o)[empty] == 0) and np.all(to_f64(l)[empty] == -np.inf)
    check(x, "decode 300 sequences", seqs=np.flatnonzero(lens > 0))


def test_decode_zero_length_sequence():
    lens = [0, 20, 0, 300]
    x = fi.paged(lens, 8, 2, 128, "bf16", seed=42)
    o, l = run(x)
    o, l = to_f64(o), to_f64(l)
    assert np.all(o[[0, 2]] == 0) and np.all(l[[0, 2]] == -np.inf)
    check(x, "decode with empty sequences", seqs=[1, 3])


def test_cfg4_paged_gqa_decode_full():
    """Full size: 64 sequences, 1.2M tokens in 75219 permuted pages; every
    sequence and all 32 query heads against the fp64 oracle, which reads each
    sequence's contiguous K/V."""
    x = fi.cfg4()
    print("[case] cfg4 paged GQA decode full", flush=True)
    o, l = run(x)
    o, l = to_f64(o), to_f64(l)
    seq = lambda src: (lambda b: src[x.cu_k[b]:x.cu_k[b + 1]])
    O, L = full_oracle.decode_all(x.q, seq(x.k_seq), seq(x.v_seq), x.dtype, x.scale)
    vmax = np.abs(fi.to_f64(x.v_seq, x.dtype)).max()
    assert_parity(o, l, O, L, np.array([vmax]), x.dtype, "cfg4 paged GQA decode full")


def test_page_table_permutation_and_poison_bitwise():
    """Same sequences under identity and permuted page tables, and with NaN
    in every slot past a sequence end: outputs are bit-identical."""
    lens = [5, 16, 31, 200, 1000, 2049]
    a = fi.paged(lens, 16, 4, 128, "bf16", seed=43, permute=False)
    b = fi.paged(lens, 16, 4, 128, "bf16", seed=43, permute=True)
    c = fi.paged(lens, 16, 4, 128, "bf16", seed=43, permute=True, tail_fill="nan")
    oa, la = run(a)
    ob, lb = run(b)
    oc, lc = run(c)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(ob, oc) and torch.equal(lb, lc)
    assert not torch.isnan(oc).any()


def test_decode_matches_last_prefill_row():
    """A decode query equals the last row of a causal prefill over the
    sequence with that query appended (both within tolerance of the oracle,
    and of each other)."""
    lens = [777]
    x = fi.paged(lens, 8, 2, 128, "bf16", seed=44, permute=True)
    od, ld = run(x)
    n = lens[0]
    rng = np.random.default_rng(1)
    qpre = fi.round_to(rng.standard_normal((1, n, 8, 128)).astype(np.float32), "bf16")
    qpre[0, -1] = x.q[0]
    o, l = fa.fwd(to_dev(qpre, "bf16"), to_dev(x.k_seq[None], "bf16"), to_dev(x.v_seq[None], "bf16"),
                  causal=True)
    err = (to_f64(o)[0, -1] - to_f64(od)[0]).__abs__().max() / np.abs(fi.to_f64(x.v_seq, "bf16")).max()
    assert err <= 1e-2
    assert np.abs(to_f64(l)[0, -1] - to_f64(ld)[0]).max() <= 1e-4 * 10


def test_deterministic():
    x = fi.paged([3000, 40, 999], 32, 8, 128, "bf16", seed=45)
    dev = dev_paged(x)
    o1, l1 = run(x, dev=dev)
    o2, l2 = run(x, dev=dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
