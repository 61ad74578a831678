"""CPU tests: the oracle against its pins, and planted mistakes in copies of
the oracle caught by those pins."""
import importlib
import types

import numpy as np
import pytest

import oracle
oracle_attention = importlib.import_module("oracle.attention")
from tests import pins

ORACLE_SRC = oracle_attention.__file__


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _mutant(old: str, new: str) -> types.ModuleType:
    """A copy of the oracle module with one planted mistake."""
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = ORACLE_SRC
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = {
    "scale dropped": ("* scale  ", "* 1.0  "),
    "scale squared": ("* scale  ", "* scale * scale  "),
    "causal offset dropped": ("rows[r0:r1] + (Nk - Nq)", "rows[r0:r1]"),
    "causal offset sign": ("rows[r0:r1] + (Nk - Nq)", "rows[r0:r1] - (Nk - Nq)"),
    "causal strictly below": ("> last[:, None]", ">= last[:, None]"),
    "values from keys": ("(P @ v)", "(P @ k[:, :v.shape[1]])"),
    "no normalisation": ("(P @ v) / safe_l[:, None]", "(P @ v)"),
    "lse in base 2": ("m + np.log(safe_l)", "m + np.log2(safe_l)"),
    "lse without max": ("m + np.log(safe_l)", "np.log(safe_l)"),
    "max not subtracted": ("np.exp(S - np.where(live, m, 0.0)[:, None])", "np.exp(S)"),
    "min instead of max": ("m = S.max(axis=1)", "m = S.min(axis=1)"),
    "kv head modulo": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "query transposed against keys": ("(q_rows[r0:r1] @ k.T)", "(k[:q_rows.shape[0]][r0:r1] @ q_rows.T[:, :k.shape[0]])"),
    "empty row lse zero": ("m + np.log(safe_l), -np.inf)", "m + np.log(safe_l), 0.0)"),
    "decode drops last key": ("k0, k1 = int(cu_k[b]), int(cu_k[b + 1])\n", "k0, k1 = int(cu_k[b]), int(cu_k[b + 1]) - 1\n"),
    "varlen key offsets from queries": ("k[k0:k1, g],\n", "k[q0:q1, g],\n"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    mut = _mutant(old, new)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"no pin catches the planted mistake {name!r}"


def test_scalar_twin_hand_cases():
    """The brute-force twin also reproduces the hand-worked values."""
    for name, q, k, v, scale, causal, o, lse in pins.hand_cases():
        o2, l2 = pins.scalar.attention_head(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        pins._close(np.array(o2).reshape(o.shape), o, 1e-13, name)
        pins._close(np.array(l2), lse, 1e-13, name)


def test_rows_subset_equals_whole():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((50, 8))
    k = rng.standard_normal((60, 8))
    v = rng.standard_normal((60, 8))
    O, L = oracle.attention_head(q, k, v, 0.3, True)
    rows = np.array([0, 3, 17, 49])
    o, l = oracle.attention_rows(q[rows], rows, 50, k, v, 0.3, True)
    np.testing.assert_array_equal(o, O[rows])
    np.testing.assert_array_equal(l, L[rows])


def test_oracle_refuses_integer_storage():
    """16-bit storage must be decoded to values before reaching the oracle."""
    bits = np.zeros((4, 8), dtype=np.uint16)
    with pytest.raises(TypeError):
        oracle.attention_head(bits, bits, bits, 0.5, False)
