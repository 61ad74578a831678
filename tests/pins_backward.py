"""Pins of the backward oracle (oracle/backward.py): checks against facts
that the mathematics fixes, independent of that oracle's own code.

Each ``pin_*`` takes a backward-oracle module (``attention_head_grad``,
``attention_grad``) and raises AssertionError when it disagrees.
``tests/test_oracle_backward.py`` runs them against the real module (all
must pass) and against copies with a planted mistake (each must fail one).

* hand cases: exact gradients derived by hand (tests/golden/bwd_hand_cases.json);
* central finite differences of the forward oracle (itself pinned by
  tests/pins.py) on random small heads: causal and not, fewer and more
  queries than keys, grouped-query heads, a non-default scale;
* invariants: key gradients of a head sum to zero (adding one vector to
  every key adds a per-row constant to the logits, which the softmax
  ignores); constant values give zero query and key gradients; value
  gradients sum to the sum of dO over rows that see a key; a row that sees
  no key gets a zero query gradient; grouped-query heads equal repeated
  heads with the repeated key/value gradients summed.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bwd_hand_cases.json")


def _parse(s: str) -> float:
    s = s.strip()
    if "*ln " in s:
        c, x = s.split("*ln ")
        return float(Fraction(c)) * math.log(float(Fraction(x)))
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    return float(Fraction(s))


def _grid(rows):
    return np.array([[_parse(x) for x in r] for r in rows], dtype=np.float64)


def hand_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        yield (c["name"], _grid(c["q"]), _grid(c["k"]), _grid(c["v"]), _grid(c["do"]),
               _parse(c["scale"]), bool(c["causal"]), _grid(c["dq"]), _grid(c["dk"]),
               _grid(c["dv"]))


def _close(a, b, tol, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b))) if b.size else 0.0
    assert err <= tol, (what, err)


def pin_bwd_hand_cases(bwd):
    for name, q, k, v, do, scale, causal, dq, dk, dv in hand_cases():
        gq, gk, gv = bwd.attention_head_grad(q, k, v, do, scale, causal)
        _close(gq, dq, 1e-14, name + " dq")
        _close(gk, dk, 1e-14, name + " dk")
        _close(gv, dv, 1e-14, name + " dv")


def _fd_case(bwd, B, Nq, Nk, Hq, Hkv, d, scale, causal, seed):
    """Central differences of L = sum(W * O) through the forward oracle
    against the backward oracle's gradients with dO = W."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    w = rng.standard_normal((B, Nq, Hq, d))

    def loss(q_, k_, v_):
        O, _ = oracle.attention(q_, k_, v_, scale, causal)
        return float(np.sum(w * O))

    gq, gk, gv = bwd.attention_grad(q, k, v, w, scale, causal)
    h = 1e-6
    for name, x, g in (("dq", q, gq), ("dk", k, gk), ("dv", v, gv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(q, k, v)
            x[idx] = x0 - h
            lm = loss(q, k, v)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        _close(g, fd, 1e-7, f"finite differences {name} Nq={Nq} Nk={Nk} causal={causal}")


def pin_bwd_finite_differences(bwd):
    _fd_case(bwd, 1, 5, 7, 4, 2, 3, 0.7, False, 1)
    _fd_case(bwd, 1, 5, 7, 4, 2, 3, 0.7, True, 2)    # fewer queries than keys
    _fd_case(bwd, 2, 6, 4, 2, 1, 2, 1.3, True, 3)    # more queries: rows 0, 1 see no key
    _fd_case(bwd, 1, 4, 4, 2, 2, 3, 0.5, True, 4)    # square causal, plain multi-head


def pin_bwd_key_gradients_sum_to_zero(bwd):
    rng = np.random.default_rng(11)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal(s) for s in ((30, 8), (40, 8), (40, 8), (30, 8)))
        _, gk, _ = bwd.attention_head_grad(q, k, v, do, 0.4, causal)
        assert np.max(np.abs(gk.sum(axis=0))) <= 1e-12 * max(1.0, np.abs(gk).max()), causal


def pin_bwd_constant_values(bwd):
    rng = np.random.default_rng(12)
    q, k, do = (rng.standard_normal(s) for s in ((20, 4), (25, 4), (20, 4)))
    v = np.tile(rng.standard_normal((1, 4)), (25, 1))
    for causal in (False, True):
        gq, gk, gv = bwd.attention_head_grad(q, k, v, do, 0.6, causal)
        assert np.max(np.abs(gq)) <= 1e-12 and np.max(np.abs(gk)) <= 1e-12, causal


def pin_bwd_value_gradient_sums(bwd):
    rng = np.random.default_rng(13)
    # Nq > Nk causal: rows 0..4 see no key and contribute nothing
    q, k, v, do = (rng.standard_normal(s) for s in ((12, 4), (7, 4), (7, 4), (12, 4)))
    gq, _, gv = bwd.attention_head_grad(q, k, v, do, 0.8, True)
    _close(gv.sum(axis=0), do[5:].sum(axis=0), 1e-12, "sum of dV")
    assert np.all(gq[:5] == 0), "rows without keys must get no query gradient"
    gq, _, gv = bwd.attention_head_grad(q, k, v, do, 0.8, False)
    _close(gv.sum(axis=0), do.sum(axis=0), 1e-12, "sum of dV, no mask")


def pin_bwd_gqa_equals_repeated_heads(bwd):
    rng = np.random.default_rng(14)
    q, do = rng.standard_normal((2, 9, 6, 4)), rng.standard_normal((2, 9, 6, 4))
    k, v = rng.standard_normal((2, 11, 2, 4)), rng.standard_normal((2, 11, 2, 4))
    gq, gk, gv = bwd.attention_grad(q, k, v, do, 0.5, True)
    rq, rk, rv = bwd.attention_grad(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), do, 0.5,
                                    True)
    _close(gq, rq, 1e-13, "GQA dq")
    _close(gk, rk.reshape(2, 11, 2, 3, 4).sum(axis=3), 1e-13, "GQA dk")
    _close(gv, rv.reshape(2, 11, 2, 3, 4).sum(axis=3), 1e-13, "GQA dv")


ALL_PINS = [pin_bwd_hand_cases, pin_bwd_finite_differences, pin_bwd_key_gradients_sum_to_zero,
            pin_bwd_constant_values, pin_bwd_value_gradient_sums,
            pin_bwd_gqa_equals_repeated_heads]
