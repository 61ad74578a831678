"""Pins of the CPU oracle: checks against facts that the pages and the
mathematics fix, independent of the oracle's own code.

Each ``pin_*`` function takes an oracle module (``attention_head``,
``attention``, ``attention_varlen``, ``decode``) and raises AssertionError
when it disagrees. ``tests/test_oracle.py`` runs them against the real
oracle (all must pass) and against mutated copies of it (each mutant must
fail at least one), so a dropped term, a wrong sign or index or a
transposed operand in the oracle is caught.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
TIGHT = 1e-12


def _parse(s: str) -> float:
    s = s.strip()
    if s == "-inf":
        return -math.inf
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    return float(Fraction(s))


def _grid(rows):
    return np.array([[_parse(x) for x in r] for r in rows], dtype=np.float64)


def hand_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        yield (c["name"], _grid(c["q"]), _grid(c["k"]), _grid(c["v"]), _parse(c["scale"]),
               bool(c["causal"]), _grid(c["o"]), np.array([_parse(x) for x in c["lse"]]))


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), (what, "finiteness differs")
    assert np.array_equal(a[~fin], b[~fin]), (what, "infinite entries differ")
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin])))
        assert err <= tol, (what, err)


# ------------------------------------------------------------------ pins --
def pin_hand_cases(orc):
    for name, q, k, v, scale, causal, o, lse in hand_cases():
        O, L = orc.attention_head(q, k, v, scale, causal)
        _close(O, o, 1e-13, name + " O")
        _close(L, lse, 1e-13, name + " lse")


def _tiny_cases(seed):
    rng = np.random.default_rng(seed)
    for _ in range(12):
        nq = int(rng.integers(1, 7))
        nk = int(rng.integers(1, 7))
        d = int(rng.integers(1, 5))
        dv = int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        q = rng.standard_normal((nq, d)) * 2
        k = rng.standard_normal((nk, d)) * 2
        v = rng.standard_normal((nk, dv))
        scale = float(rng.uniform(0.2, 1.5))
        yield q, k, v, scale, causal


def pin_brute_force(orc, seed=11):
    for q, k, v, scale, causal in _tiny_cases(seed):
        O, L = orc.attention_head(q, k, v, scale, causal)
        o2, l2 = scalar.attention_head(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        _close(O, np.array(o2).reshape(O.shape), 1e-12, "brute O")
        _close(L, np.array(l2), 1e-12, "brute lse")


def pin_rows_normalised(orc, seed=12):
    """exp(scale*q.k_j - lse) summed over visible keys is 1 for each row."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q = rng.standard_normal((37, 16))
        k = rng.standard_normal((53, 16))
        v = rng.standard_normal((53, 8))
        _, L = orc.attention_head(q, k, v, 0.25, causal)
        S = q @ k.T * 0.25
        for i in range(37):
            vis = np.arange(53) <= i + 16 if causal else np.ones(53, bool)
            assert abs(np.exp(S[i, vis] - L[i]).sum() - 1.0) <= 1e-12


def pin_constant_v(orc, seed=13):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q = rng.standard_normal((20, 8)) * 3
        k = rng.standard_normal((20, 8)) * 3
        row = rng.standard_normal(5)
        v = np.tile(row, (20, 1))
        O, _ = orc.attention_head(q, k, v, 0.35, causal)
        _close(O, np.tile(row, (20, 1)), 1e-12, "constant V")


def pin_dominant_logit(orc, seed=14):
    """One logit 300 above every other: the output is that key's value row."""
    rng = np.random.default_rng(seed)
    n = 24
    v = rng.standard_normal((n, 6))
    target = rng.permutation(n)
    k = np.eye(n) * 30.0
    q = np.zeros((n, n))
    q[np.arange(n), target] = 10.0
    O, L = orc.attention_head(q, k, v, 1.0, False)
    _close(O, v[target], 1e-12, "dominant O")
    _close(L, np.full(n, 300.0), 1e-12, "dominant lse")


def pin_permutation(orc, seed=15):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((19, 8))
    k = rng.standard_normal((23, 8))
    v = rng.standard_normal((23, 4))
    p = rng.permutation(23)
    O1, L1 = orc.attention_head(q, k, v, 0.4, False)
    O2, L2 = orc.attention_head(q, k[p], v[p], 0.4, False)
    _close(O1, O2, 1e-12, "perm O")
    _close(L1, L2, 1e-12, "perm lse")


def pin_shift(orc, seed=16):
    """K + u for every key: O unchanged, lse moves by scale*q.u. Large u
    exercises the max subtraction (logits near +-900 overflow exp)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((17, 8))
    k = rng.standard_normal((17, 8))
    v = rng.standard_normal((17, 5))
    u = rng.standard_normal(8) * 150
    for causal in (False, True):
        O1, L1 = orc.attention_head(q, k, v, 0.7, causal)
        O2, L2 = orc.attention_head(q, k + u, v, 0.7, causal)
        _close(O2, O1, 1e-10, "shift O")
        _close(L2, L1 + 0.7 * (q @ u), 1e-12, "shift lse")


def pin_zero_q(orc, seed=17):
    """Q = 0: non-causal rows are the mean of V and lse = ln Nk; causal row
    i is the mean of V[0..i] and lse = ln(i+1)."""
    rng = np.random.default_rng(seed)
    n, d = 41, 8
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, 3))
    O, L = orc.attention_head(q, k, v, 0.3, False)
    _close(O, np.tile(v.mean(axis=0), (n, 1)), 1e-12, "zero-q O")
    _close(L, np.full(n, math.log(n)), 1e-12, "zero-q lse")
    O, L = orc.attention_head(q, k, v, 0.3, True)
    pref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    _close(O, pref, 1e-12, "zero-q causal O")
    _close(L, np.log(np.arange(1, n + 1)), 1e-12, "zero-q causal lse")


def pin_causal_row0(orc, seed=18):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((9, 8))
    k = rng.standard_normal((9, 8))
    v = rng.standard_normal((9, 4))
    O, L = orc.attention_head(q, k, v, 0.5, True)
    _close(O[0], v[0], 1e-12, "row0 O")
    _close(L[0], 0.5 * q[0] @ k[0], 1e-12, "row0 lse")


def pin_split_combine(orc, seed=19):
    """Attention over keys A u B equals the log-sum-exp merge of attention
    over A and over B (the algebra a split-KV decode relies on)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((6, 8))
    k = rng.standard_normal((30, 8))
    v = rng.standard_normal((30, 4))
    O, L = orc.attention_head(q, k, v, 0.6, False)
    Oa, La = orc.attention_head(q, k[:11], v[:11], 0.6, False)
    Ob, Lb = orc.attention_head(q, k[11:], v[11:], 0.6, False)
    Lm = np.logaddexp(La, Lb)
    Om = np.exp(La - Lm)[:, None] * Oa + np.exp(Lb - Lm)[:, None] * Ob
    _close(Om, O, 1e-12, "combine O")
    _close(Lm, L, 1e-12, "combine lse")


def pin_torch_composition(orc, seed=20):
    """A library special case: torch CPU fp64 matmul + softmax + logsumexp."""
    import torch
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((33, 16))
    k = rng.standard_normal((40, 16))
    v = rng.standard_normal((40, 16))
    for causal in (False, True):
        O, L = orc.attention_head(q, k, v, 0.25, causal)
        S = torch.from_numpy(q) @ torch.from_numpy(k).T * 0.25
        if causal:
            mask = torch.arange(40)[None, :] > torch.arange(33)[:, None] + 7
            S = S.masked_fill(mask, float("-inf"))
        ref_o = torch.softmax(S, dim=1) @ torch.from_numpy(v)
        ref_l = torch.logsumexp(S, dim=1)
        _close(O, ref_o.numpy(), 1e-12, "torch O")
        _close(L, ref_l.numpy(), 1e-12, "torch lse")


def pin_gqa(orc, seed=21):
    """Grouped heads equal multi-head attention with each K/V head repeated
    Hq/Hkv times consecutively."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, d = 2, 13, 6, 2, 8
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    for causal in (False, True):
        O1, L1 = orc.attention(q, k, v, 0.3, causal)
        O2, L2 = orc.attention(q, np.repeat(k, Hq // Hkv, axis=2),
                               np.repeat(v, Hq // Hkv, axis=2), 0.3, causal)
        _close(O1, O2, 1e-12, "gqa O")
        _close(L1, L2, 1e-12, "gqa lse")
        # head h of the grouped call equals a single-head call on head h // 3
        for h in range(Hq):
            o, l = orc.attention_head(q[1, :, h], k[1, :, h // 3], v[1, :, h // 3], 0.3, causal)
            _close(O1[1, :, h], o, 1e-12, "gqa head O")
            _close(L1[1, :, h], l, 1e-12, "gqa head lse")


def pin_varlen(orc, seed=22):
    """A ragged batch equals separate single-sequence calls, including an
    empty sequence and sequences with fewer queries than keys."""
    rng = np.random.default_rng(seed)
    lq, lk = [3, 0, 9, 1, 0], [5, 2, 9, 4, 0]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hq, Hkv, d = 4, 2, 8
    q = rng.standard_normal((int(cq[-1]), Hq, d))
    k = rng.standard_normal((int(ck[-1]), Hkv, d))
    v = rng.standard_normal((int(ck[-1]), Hkv, d))
    for causal in (False, True):
        O, L = orc.attention_varlen(q, k, v, cq, ck, 0.3, causal)
        for s in range(len(lq)):
            a, b, c, e = cq[s], cq[s + 1], ck[s], ck[s + 1]
            o1, l1 = orc.attention(q[None, a:b], k[None, c:e], v[None, c:e], 0.3, causal)
            _close(O[a:b], o1[0], 1e-12, "varlen O")
            _close(L[a:b], l1[0], 1e-12, "varlen lse")


def pin_decode(orc, seed=23):
    """A decode query equals the last row of a causal call on the sequence
    with that query appended, and its lse matches."""
    rng = np.random.default_rng(seed)
    lens = np.array([7, 1, 12])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Hq, Hkv, d = 4, 2, 8
    ks = rng.standard_normal((int(cu[-1]), Hkv, d))
    vs = rng.standard_normal((int(cu[-1]), Hkv, d))
    q = rng.standard_normal((3, Hq, d))
    O, L = orc.decode(q, ks, vs, cu, 0.4)
    for b in range(3):
        kb, vb = ks[cu[b]:cu[b + 1]], vs[cu[b]:cu[b + 1]]
        n = lens[b]
        qq = np.concatenate([rng.standard_normal((n - 1, Hq, d)), q[b][None]], axis=0)
        o1, l1 = orc.attention(qq[None], kb[None], vb[None], 0.4, True)
        _close(O[b], o1[0, -1], 1e-12, "decode O")
        _close(L[b], l1[0, -1], 1e-12, "decode lse")


ALL_PINS = [pin_hand_cases, pin_brute_force, pin_rows_normalised, pin_constant_v,
            pin_dominant_logit, pin_permutation, pin_shift, pin_zero_q, pin_causal_row0,
            pin_split_combine, pin_torch_composition, pin_gqa, pin_varlen, pin_decode]
