"""Plain fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY. This module is imported by the test suite, by the
smoke check and by the CPU-baseline leg of the benchmark, and by nothing on
the product path. It shares no code with the GPU library.

What it computes
----------------
The definition of attention that the pages contrast with the fused kernel
("I/O-Aware Kernels", section "Naive attention: materializing the k x k score
matrix"): the score matrix S = Q K^T is formed whole, a softmax is taken over
every full row, and the result multiplies V. The section "FlashAttention:
tiling + online softmax" states that the fused kernel reaches exactly these
numbers, so this definition is the parity target. Following that, this
oracle materialises S (in blocks of whole rows, purely to bound memory) and
uses the two-pass textbook softmax - no running max, no online rescaling.

Readings taken where the pages are silent (all of them documented with the
design notes):
* the logits are scaled: S = (Q K^T) * scale, scale passed in (1/sqrt(d) by
  default, as a float32 value);
* causal masking is bottom-right aligned: query i may see key j iff
  j <= i + (Nk - Nq); with Nq == Nk this is j <= i, and a single decode query
  sees every key;
* the per-row log-sum-exp is natural-log, of the scaled logits over the
  allowed keys: lse_i = ln sum_j exp(S_ij);
* a row with no allowed key has O = 0 and lse = -inf;
* grouped-query heads: query head h reads key/value head h // (Hq / Hkv)
  ("FlashInfer: I/O-aware attention for serving" names grouped-query
  attention; the consecutive grouping is the reading taken).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 2048


def _values(a):
    """float64 view of values. Integer arrays are refused: 16-bit storage
    (e.g. bfloat16 bit patterns) must be decoded by the caller first."""
    a = np.asarray(a)
    if not np.issubdtype(a.dtype, np.floating):
        raise TypeError(f"oracle inputs must be floating point values, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def attention_head(q, k, v, scale, causal):
    """One head. q [Nq, d], k [Nk, d], v [Nk, dv] (float64) -> (O [Nq, dv], lse [Nq])."""
    q, k, v = _values(q), _values(k), _values(v)
    Nq, Nk = q.shape[0], k.shape[0]
    return attention_rows(q, np.arange(Nq), Nq, k, v, scale, causal)


def attention_rows(q_rows, rows, Nq, k, v, scale, causal):
    """Selected query rows of one head.

    q_rows [R, d] are the query vectors of rows ``rows`` (indices into a query
    sequence of length ``Nq``); k [Nk, d], v [Nk, dv]. Each row's full score
    row is formed, so any subset of rows gives the same values as the whole.

    Follows "I/O-Aware Kernels", section "Naive attention: materializing the
    k x k score matrix": S = Q K^T for the rows, a softmax over each complete
    row (max, exponentials, sum), then the weighted sum of the value rows.
    """
    q_rows, k, v = _values(q_rows), _values(k), _values(v)
    rows = np.asarray(rows, dtype=np.int64)
    R, Nk, dv = q_rows.shape[0], k.shape[0], v.shape[1]
    O = np.zeros((R, dv), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    if R == 0 or Nk == 0:
        return O, lse
    scale = np.float64(scale)
    for r0 in range(0, R, ROW_BLOCK):
        r1 = min(R, r0 + ROW_BLOCK)
        S = (q_rows[r0:r1] @ k.T) * scale                      # [r, Nk] scores
        if causal:
            last = rows[r0:r1] + (Nk - Nq)                      # last visible key
            S[np.arange(Nk)[None, :] > last[:, None]] = -np.inf
        m = S.max(axis=1)                                       # row max
        live = np.isfinite(m)
        P = np.exp(S - np.where(live, m, 0.0)[:, None])         # masked -> 0
        l = P.sum(axis=1)                                       # row sum
        safe_l = np.where(live, l, 1.0)
        O[r0:r1] = np.where(live[:, None], (P @ v) / safe_l[:, None], 0.0)
        lse[r0:r1] = np.where(live, m + np.log(safe_l), -np.inf)
    return O, lse


def kv_head_of(h, Hq, Hkv):
    """Key/value head read by query head h (consecutive groups of Hq/Hkv)."""
    return h // (Hq // Hkv)


def attention(q, k, v, scale, causal):
    """Dense batch. q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] float64
    -> O [B, Nq, Hq, d], lse [B, Nq, Hq].

    Multi-head and grouped-query attention as listed in "I/O-Aware Kernels",
    section "FlashInfer: I/O-aware attention for serving": each query head is
    an independent instance of the definition on its key/value head."""
    q, k, v = _values(q), _values(k), _values(v)
    B, Nq, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    O = np.zeros(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.zeros((B, Nq, Hq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[b, :, h], lse[b, :, h] = attention_head(q[b, :, h], k[b, :, g], v[b, :, g],
                                                      scale, causal)
    return O, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale, causal):
    """Packed ragged batch. q [Tq, Hq, d], k/v [Tk, Hkv, d]; sequence s owns
    rows cu_q[s]:cu_q[s+1] of q and cu_k[s]:cu_k[s+1] of k/v. The definition
    is applied to each sequence on its own ("I/O-Aware Kernels", section
    "FlashInfer: I/O-aware attention for serving": ragged, variable-length
    batches)."""
    q, k, v = _values(q), _values(k), _values(v)
    Hq, Hkv = q.shape[1], k.shape[1]
    O = np.zeros(q.shape[:2] + (v.shape[2],), dtype=np.float64)
    lse = np.zeros(q.shape[:2], dtype=np.float64)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[q0:q1, h], lse[q0:q1, h] = attention_head(q[q0:q1, h], k[k0:k1, g],
                                                        v[k0:k1, g], scale, causal)
    return O, lse


def decode(q, k_seq, v_seq, cu_k, scale, seqs=None):
    """One query token per sequence against that sequence's whole K/V.

    q [B, Hq, d]; k_seq/v_seq [T, Hkv, d] hold the sequences' keys/values
    contiguously (cu_k offsets) - the oracle never sees a page table. A lone
    query is the last row of its sequence, so every key is visible.
    ``seqs`` restricts the work to some sequences (others are left zero).
    The paged cache of "I/O-Aware Kernels", section "FlashInfer: I/O-aware
    attention for serving", only changes where K/V live, not the result.
    Returns O [B, Hq, d], lse [B, Hq].
    """
    q = _values(q)
    B, Hq, _ = q.shape
    Hkv = k_seq.shape[1]
    O = np.zeros(q.shape[:2] + (v_seq.shape[2],), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        kb = _values(k_seq[k0:k1])
        vb = _values(v_seq[k0:k1])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, l = attention_head(q[b, h][None, :], kb[:, g], vb[:, g], scale, causal=False)
            O[b, h], lse[b, h] = o[0], l[0]
    return O, lse
