"""Plain fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY. Imported by the test suite and nothing on the
product path; it shares no code with the GPU library.

What it computes
----------------
The pages describe only the forward pass. Its definition ("I/O-Aware
Kernels", section "Naive attention: materializing the k x k score matrix")
is S = scale * Q K^T, P = the softmax of every row of S, O = P V. Given the
gradient dO of a loss with respect to O, the chain rule through those three
steps gives, for one head:

    dV = P^T dO                        (O = P V, differentiated in V)
    dP = dO V^T                        (O = P V, differentiated in P)
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
                                       (row softmax: dP_i -> dS_i)
    dQ = scale * dS K                  (S = scale Q K^T, in Q)
    dK = scale * dS^T Q                (S = scale Q K^T, in K)

Masked scores are -inf, so their P is 0 and they receive no gradient; a row
that sees no key has P = 0 throughout. The log-sum-exp output is not
differentiated (it is saved state, not a loss term). Grouped-query heads:
a key/value head's gradient is the sum over the query heads that read it.
The oracle forms S, P, dP and dS whole for blocks of full rows, as the
forward oracle does, with no online recurrence.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 2048


def _values(a):
    a = np.asarray(a)
    if not np.issubdtype(a.dtype, np.floating):
        raise TypeError(f"oracle inputs must be floating point values, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def attention_head_grad(q, k, v, do, scale, causal):
    """One head. q [Nq, d], k [Nk, d], v [Nk, dv], do [Nq, dv]
    -> (dQ [Nq, d], dK [Nk, d], dV [Nk, dv]), float64. Causal masking is
    bottom-right aligned: query i sees key j iff j <= i + (Nk - Nq)."""
    q, k, v, do = _values(q), _values(k), _values(v), _values(do)
    Nq, Nk = q.shape[0], k.shape[0]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    if Nq == 0 or Nk == 0:
        return dq, dk, dv
    scale = np.float64(scale)
    for r0 in range(0, Nq, ROW_BLOCK):
        r1 = min(Nq, r0 + ROW_BLOCK)
        S = (q[r0:r1] @ k.T) * scale                              # scores
        if causal:
            last = np.arange(r0, r1) + (Nk - Nq)                  # last visible key
            S[np.arange(Nk)[None, :] > last[:, None]] = -np.inf
        m = S.max(axis=1)
        live = np.isfinite(m)
        E = np.exp(S - np.where(live, m, 0.0)[:, None])
        P = E / np.where(live, E.sum(axis=1), 1.0)[:, None]      # row softmax (0 if empty)
        dv += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v.T
        dS = P * (dP - (P * dP).sum(axis=1)[:, None])
        dq[r0:r1] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv


def kv_head_of(h, Hq, Hkv):
    """Key/value head read by query head h (consecutive groups of Hq/Hkv)."""
    return h // (Hq // Hkv)


def attention_grad(q, k, v, do, scale, causal):
    """Dense batch: q, do [B, Nq, Hq, d], k, v [B, Nk, Hkv, d] -> (dQ like q,
    dK like k, dV like v), float64. Query head h reads key/value head
    h // (Hq / Hkv); dK and dV of a key/value head sum the contributions of
    every query head that reads it."""
    q, k, v, do = _values(q), _values(k), _values(v), _values(do)
    B, Nq, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            gq, gk, gv = attention_head_grad(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h],
                                             scale, causal)
            dq[b, :, h] = gq
            dk[b, :, g] += gk
            dv[b, :, g] += gv
    return dq, dk, dv
