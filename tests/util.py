"""Helpers shared by the GPU tests: host arrays <-> device tensors and the
parity metrics (normalised max-abs error of O, relative error of LSE)."""
from __future__ import annotations

import numpy as np

import fa_inputs as fi

# error bars on max|O_gpu - O_ref| / max|V read|, by input dtype
O_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
# error bars on |lse_gpu - lse_ref| / max(1, |lse_ref|), by input dtype
LSE_TOL = {"f32": 1e-5, "f16": 1e-4, "bf16": 1e-4}


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    raise ValueError(dtype)


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def o_error(o_gpu, o_ref, v_read) -> float:
    """max |O_gpu - O_ref| / max |V| over the values the call reads."""
    vmax = float(np.max(np.abs(v_read))) if np.size(v_read) else 1.0
    if o_ref.size == 0:
        return 0.0
    return float(np.max(np.abs(o_gpu - o_ref))) / max(vmax, 1e-30)


def lse_error(l_gpu, l_ref) -> float:
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_gpu), fin), "LSE finiteness differs from the oracle"
    assert np.array_equal(l_gpu[~fin], l_ref[~fin]), "LSE infinities differ from the oracle"
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(l_gpu[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))))


# (case, dtype, err_O, err_LSE) of every parity check of the session, printed
# by the terminal summary in tests/conftest.py
PARITY_LOG = []


def assert_parity(o_gpu, l_gpu, o_ref, l_ref, v_read, dtype, what=""):
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    eo = o_error(o_gpu, o_ref, v_read)
    el = lse_error(l_gpu, l_ref)
    PARITY_LOG.append((what, dtype, eo, el))
    print(f"[parity] {what}: err_O={eo:.3e} (tol {O_TOL[dtype]:.0e}) err_LSE={el:.3e} "
          f"(tol {LSE_TOL[dtype]:.0e})", flush=True)
    assert eo <= O_TOL[dtype], f"{what}: O error {eo:.3e} > {O_TOL[dtype]:.0e}"
    assert el <= LSE_TOL[dtype], f"{what}: LSE error {el:.3e} > {LSE_TOL[dtype]:.0e}"
    return eo, el


def dense_dev(x: fi.Dense):
    return to_dev(x.q, x.dtype), to_dev(x.k, x.dtype), to_dev(x.v, x.dtype)
