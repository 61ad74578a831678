"""The fp64 oracle over whole full-size workloads, one (sequence, head) unit
per task on a thread pool. NumPy releases the GIL inside its matrix products
and element-wise passes, so independent heads run side by side on the host
cores; every unit is still one plain call of the oracle on one sequence and
one head, exactly as the serial loops of ``oracle`` would make it.

Test infrastructure: used by the GPU parity tests and by the benchmark's
check of the outputs it timed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import fa_inputs as fi
import oracle


def workers() -> int:
    """Host threads for independent oracle units (half the cores: each unit's
    matrix products use BLAS threads of their own)."""
    return max(1, min(8, (os.cpu_count() or 2) // 2))


def _map(fn, items, n=None):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with cf.ThreadPoolExecutor(n or workers()) as ex:
        return list(ex.map(fn, items))


def dense_heads(x: fi.Dense, heads, rows=None, b=0):
    """Oracle of query rows ``rows`` (all when None) of heads ``heads`` in
    batch entry b of a dense workload -> O [R, len(heads), d], LSE [R, len(heads)]."""
    B, Nq, Nk, Hq, Hkv, d = x.shape
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    heads = list(heads)

    def one(h):
        g = oracle.kv_head_of(h, Hq, Hkv)
        return oracle.attention_rows(fi.to_f64(x.q[b, rows, h], x.dtype), rows, Nq,
                                     fi.to_f64(x.k[b, :, g], x.dtype),
                                     fi.to_f64(x.v[b, :, g], x.dtype), x.scale, x.causal)

    res = _map(one, heads)
    O = np.stack([r[0] for r in res], axis=1)
    L = np.stack([r[1] for r in res], axis=1)
    return O, L


def varlen_all(q, k, v, cu_q, cu_k, dtype, scale, causal):
    """Oracle of every row of every head of a packed ragged batch (q [Tq, Hq,
    d], k/v [Tk, Hkv, d] in storage form) -> O [Tq, Hq, d], LSE [Tq, Hq]."""
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((Tq, Hq, v.shape[2]))
    L = np.full((Tq, Hq), -np.inf)
    units = [(s, h) for s in range(len(cu_q) - 1) for h in range(Hq)
             if cu_q[s + 1] > cu_q[s]]

    def one(u):
        s, h = u
        a, b, c, e = (int(t) for t in (cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]))
        g = oracle.kv_head_of(h, Hq, Hkv)
        o, lse = oracle.attention_head(fi.to_f64(q[a:b, h], dtype), fi.to_f64(k[c:e, g], dtype),
                                       fi.to_f64(v[c:e, g], dtype), scale, causal)
        O[a:b, h] = o
        L[a:b, h] = lse

    _map(one, units)
    return O, L


def decode_all(q, keys, values, dtype, scale):
    """Oracle of one query per sequence against its contiguous keys:
    q [B, Hq, d]; keys(b) / values(b) give sequence b's [L_b, Hkv, d] in
    storage form -> O [B, Hq, d], LSE [B, Hq]."""
    B, Hq, d = q.shape

    def one(b):
        kb = fi.to_f64(keys(b), dtype)
        vb = fi.to_f64(values(b), dtype)
        cu = np.array([0, len(kb)])
        return oracle.decode(fi.to_f64(q[b:b + 1], dtype), kb, vb, cu, scale)

    res = _map(one, range(B))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
