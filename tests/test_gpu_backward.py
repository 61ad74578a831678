"""GPU parity of the backward pass (fa_bwd) against the fp64 backward
oracle, which differentiates the forward definition directly (S, P, dP, dS
formed whole). The GPU takes the O and LSE of its own forward call, as a
training step does.

Tolerance: max |dX_gpu - dX_ref| / max |dX_ref| per gradient, at ten times
the half-unit roundoff of the input type (bf16: 10 * 2^-9 -> 2e-2; fp16:
10 * 2^-12 -> 5e-3). The kernels round P and dS to the input type before
three of their products, take D from the rounded forward output and round
the gradients on output: about five roundings of half a unit each, with room
for the cancellation in dP - D and in the key-gradient sums."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.util import dense_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")

G_TOL = {"bf16": 2e-2, "f16": 5e-3}


def grad_error(g, ref):
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(g - ref))) / m if m > 0 else float(np.max(np.abs(g)))


def run_bwd(x: fi.Dense, do):
    q, k, v = dense_dev(x)
    o, lse = fa.fwd(q, k, v, causal=x.causal, scale=x.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, to_dev(do, x.dtype), causal=x.causal, scale=x.scale)
    torch.cuda.synchronize()
    return to_f64(dq), to_f64(dk), to_f64(dv)


def check_grads(got, want, dtype, what):
    errs = [grad_error(g, w) for g, w in zip(got, want)]
    print(f"[parity] {what}: err_dQ={errs[0]:.3e} err_dK={errs[1]:.3e} err_dV={errs[2]:.3e} "
          f"(tol {G_TOL[dtype]:.0e})", flush=True)
    for name, e in zip(("dQ", "dK", "dV"), errs):
        assert e <= G_TOL[dtype], f"{what}: {name} error {e:.3e} > {G_TOL[dtype]:.0e}"
    for g in got:
        assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    return errs


def check_dense(x: fi.Dense, what, seed):
    print(f"[case] {what} shape={x.shape} dtype={x.dtype} causal={x.causal}", flush=True)
    B, Nq, Nk, Hq, Hkv, d = x.shape
    do = fi.grad_out((B, Nq, Hq, d), x.dtype, seed)
    got = run_bwd(x, do)
    want = oracle.attention_grad(fi.to_f64(x.q, x.dtype), fi.to_f64(x.k, x.dtype),
                                 fi.to_f64(x.v, x.dtype), fi.to_f64(do, x.dtype), x.scale, x.causal)
    return check_grads(got, want, x.dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(300, 300), (200, 333), (333, 200), (1, 77), (64, 64), (129, 5)])
def test_backward_small_ragged(dtype, d, causal, nq, nk):
    """Several query and key tiles with ragged tails, Nq != Nk both ways
    (bottom-right causal, rows that see no key), grouped-query heads."""
    seed = 500 + nq + nk + d
    x = fi.dense(2, nq, nk, 4, 2, d, dtype, seed=seed, causal=causal)
    check_dense(x, f"bwd {dtype} d{d} causal={causal} nq={nq} nk={nk}", seed)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_causal_multihead_n2048(dtype):
    """Causal multi-head B=4 H=16 N=2048 d=64 (the causal multi-head
    prefill workload), every gradient element."""
    x = fi.cfg1(dtype=dtype)
    check_dense(x, f"bwd causal B4 H16 N2048 d64 {dtype}", 1)


def test_backward_gqa_group_of_eight():
    x = fi.dense(1, 700, 700, 16, 2, 128, "bf16", seed=520, causal=True)
    check_dense(x, "bwd GQA 16 query heads on 2 KV heads", 520)


def test_backward_long_context_heads():
    """B=1 H=32 N=16384 d=128 causal bf16 (the long-context prefill
    workload): every element of the gradients of heads 0, 13 and 31 (dK and
    dV of a head depend only on its own query head here, Hq = Hkv)."""
    x = fi.cfg2()
    B, Nq, Nk, Hq, Hkv, d = x.shape
    do = fi.grad_out((B, Nq, Hq, d), "bf16", 2)
    print("[case] bwd long context: GPU call", flush=True)
    dq, dk, dv = run_bwd(x, do)
    from tests import full_oracle

    def one(h):
        return oracle.attention_head_grad(fi.to_f64(x.q[0, :, h], "bf16"),
                                          fi.to_f64(x.k[0, :, h], "bf16"),
                                          fi.to_f64(x.v[0, :, h], "bf16"),
                                          fi.to_f64(do[0, :, h], "bf16"), x.scale, True)
    heads = [0, 13, 31]
    res = full_oracle._map(one, heads)
    for h, (gq, gk, gv) in zip(heads, res):
        check_grads((dq[0, :, h], dk[0, :, h], dv[0, :, h]), (gq, gk, gv), "bf16",
                    f"bwd long context head {h}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,hq,hkv", [(5, 300, 2, 2), (64, 64, 1, 1), (65, 200, 1, 1),
                                          (130, 130, 1, 1), (150, 500, 3, 3), (40, 40, 2, 1)])
def test_backward_few_query_tiles(causal, nq, nk, hq, hkv):
    """d=128 calls in which a key workgroup streams only one to four 64-row
    Q/dO tiles (the prologue and the tail of the dK/dV tile pipeline carry
    all the work), including a single row tile shared by two query heads."""
    seed = 530 + nq + nk + hq
    x = fi.dense(2, nq, nk, hq, hkv, 128, "bf16", seed=seed, causal=causal)
    check_dense(x, f"bwd few tiles causal={causal} nq={nq} nk={nk} hq={hq} hkv={hkv}", seed)


def test_backward_deterministic():
    x = fi.dense(1, 500, 500, 8, 2, 128, "bf16", seed=521, causal=True)
    q, k, v = dense_dev(x)
    o, lse = fa.fwd(q, k, v, causal=True)
    do = to_dev(fi.grad_out((1, 500, 8, 128), "bf16", 521), "bf16")
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_backward_gqa_equals_repeated_heads_summed():
    """dK, dV of a shared key/value head equal the sums over its query heads
    of the gradients with the head repeated (up to the output rounding)."""
    x = fi.dense(1, 256, 256, 8, 2, 64, "bf16", seed=522, causal=False)
    q, k, v = dense_dev(x)
    do = to_dev(fi.grad_out((1, 256, 8, 64), "bf16", 522), "bf16")
    o, lse = fa.fwd(q, k, v)
    dq1, dk1, dv1 = fa.bwd(q, k, v, o, lse, do)
    kr, vr = k.repeat_interleave(4, dim=2).contiguous(), v.repeat_interleave(4, dim=2).contiguous()
    o2, lse2 = fa.fwd(q, kr, vr)
    dq2, dk2, dv2 = fa.bwd(q, kr, vr, o2, lse2, do)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    for g1, g2 in ((dk1, dk2), (dv1, dv2)):
        s = to_f64(g2).reshape(1, 256, 2, 4, 64).sum(axis=3)
        assert grad_error(to_f64(g1), s) <= G_TOL["bf16"]
