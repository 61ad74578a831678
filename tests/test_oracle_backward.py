"""CPU tests: the backward oracle against its pins, and planted mistakes in
copies of it caught by those pins."""
import importlib
import types

import numpy as np
import pytest

from tests import pins_backward as pins

backward = importlib.import_module("oracle.backward")
SRC = backward.__file__


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(backward)


def _mutant(old: str, new: str) -> types.ModuleType:
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("backward_mutant")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = {
    "softmax term dropped": ("dS = P * (dP - (P * dP).sum(axis=1)[:, None])", "dS = P * dP"),
    "softmax term sign": ("dS = P * (dP - (P * dP).sum(axis=1)[:, None])",
                          "dS = P * (dP + (P * dP).sum(axis=1)[:, None])"),
    "row term summed over keys": ("(P * dP).sum(axis=1)[:, None]", "(P * dP).sum(axis=0)[None, :]"),
    "dq without scale": ("dq[r0:r1] = scale * (dS @ k)", "dq[r0:r1] = (dS @ k)"),
    "dk without scale": ("dk += scale * (dS.T @ q[r0:r1])", "dk += (dS.T @ q[r0:r1])"),
    "dk from dP": ("dk += scale * (dS.T @ q[r0:r1])", "dk += scale * (dP.T @ q[r0:r1])"),
    "dv from unnormalised weights": ("dv += P.T @ do[r0:r1]", "dv += E.T @ do[r0:r1]"),
    "dP against keys": ("dP = do[r0:r1] @ v.T", "dP = do[r0:r1] @ k.T"),
    "dq against values": ("dq[r0:r1] = scale * (dS @ k)", "dq[r0:r1] = scale * (dS @ v)"),
    "causal offset dropped": ("last = np.arange(r0, r1) + (Nk - Nq)", "last = np.arange(r0, r1)"),
    "causal mask dropped": ("if causal:\n            last", "if False:\n            last"),
    "gqa gradients overwritten": ("dk[b, :, g] += gk", "dk[b, :, g] = gk"),
    "gqa map modulo": ("return h // (Hq // Hkv)", "return h % Hkv"),
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
