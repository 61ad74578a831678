"""Seeded random sweep of shapes against the fp64 oracles (forward and
backward): ragged batches,
query-head groups of every size the kernels specialise for (and odd ones),
head dims 64/128, bf16/fp16, causal or not, lengths on and off the 16-token
page, 32-row wave and 128/256-row tile boundaries, more queries than keys.
Each case draws its own shape from its seed; the fixed-shape tests cover the
configurations of the benchmark."""
import numpy as np
import pytest

import fa_inputs as fi
from tests import test_gpu_backward as tbwd
from tests import test_gpu_decode as tdec
from tests import test_gpu_paged_prefill as tpp
from tests import test_gpu_prefill as tpre

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("io_aware_exact_flashattention_amd")

# lengths that sit on, just below and just above the boundaries the kernels
# care about (page 16, wave 32 rows, key tile 128, query tile 256)
EDGES = [0, 1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 300, 511, 513]


def draw_len(rng, hi):
    return int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, hi + 1))


def draw_heads(rng):
    hkv = int(rng.choice([1, 2, 3, 4]))
    group = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
    while hkv * group > 32:
        hkv = max(1, hkv // 2)
    return hkv * group, hkv


@pytest.mark.parametrize("case", range(24))
def test_sweep_varlen(case):
    rng = np.random.default_rng(7000 + case)
    B = int(rng.integers(1, 5))
    Hq, Hkv = draw_heads(rng)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.random() < 0.6)
    lq = [draw_len(rng, 600) for _ in range(B)]
    mode = rng.random()
    if mode < 0.5:
        lk = list(lq)                                          # self-attention
    elif mode < 0.8:
        lk = [q + int(rng.integers(0, 400)) for q in lq]       # cached keys before the queries
    else:
        lk = [max(0, q - int(rng.integers(0, 300))) for q in lq]  # more queries than keys
    x = fi.varlen(lq, lk, Hq, Hkv, d, dtype, seed=7000 + case, causal=causal)
    tpre.check_varlen(x, f"sweep varlen #{case}: B={B} Hq={Hq} Hkv={Hkv} d={d} {dtype} "
                         f"causal={causal} lq={lq} lk={lk}")


@pytest.mark.parametrize("case", range(12))
def test_sweep_paged_prefill(case):
    rng = np.random.default_rng(8000 + case)
    B = int(rng.integers(1, 5))
    Hq, Hkv = draw_heads(rng)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.random() < 0.7)
    lq = [draw_len(rng, 500) for _ in range(B)]
    lk = [q + (int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(0, 900)))
          for q in lq]
    x = fi.paged_prefill(lq, lk, Hq, Hkv, d, dtype, seed=8000 + case)
    tpp.check(x, f"sweep paged prefill #{case}: B={B} Hq={Hq} Hkv={Hkv} d={d} {dtype} "
                 f"lq={lq} lk={lk}", causal=causal)


@pytest.mark.parametrize("case", range(12))
def test_sweep_decode(case):
    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 9))
    Hq, Hkv = draw_heads(rng)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    lens = [draw_len(rng, 3000) if rng.random() < 0.8 else int(rng.integers(1000, 5000))
            for _ in range(B)]
    num_splits = int(rng.choice([0, 0, 1, 3, 9]))
    x = fi.paged(lens, Hq, Hkv, d, dtype, seed=9000 + case)
    tdec.check(x, f"sweep decode #{case}: B={B} Hq={Hq} Hkv={Hkv} d={d} {dtype} lens={lens}",
               num_splits=num_splits)


@pytest.mark.parametrize("case", range(20))
def test_sweep_backward(case):
    rng = np.random.default_rng(9500 + case)
    B = int(rng.integers(1, 3))
    Hq, Hkv = draw_heads(rng)
    Hq, Hkv = min(Hq, 12), min(Hkv, 12)
    while Hq % Hkv:
        Hkv -= 1
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.random() < 0.6)
    nq = max(1, draw_len(rng, 400))
    nk = nq if rng.random() < 0.5 else max(1, draw_len(rng, 400))
    x = fi.dense(B, nq, nk, Hq, Hkv, d, dtype, seed=9500 + case, causal=causal)
    tbwd.check_dense(x, f"sweep bwd #{case}: B={B} Hq={Hq} Hkv={Hkv} d={d} {dtype} "
                        f"causal={causal} nq={nq} nk={nk}", 9500 + case)
