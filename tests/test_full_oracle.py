"""The thread-pool driver of the oracle (tests/full_oracle.py), used by the
full-size GPU parity tests and the benchmark's output check, returns exactly
what the oracle's own serial calls return."""
import numpy as np

import fa_inputs as fi
import oracle
from tests import full_oracle


def test_dense_heads_equals_serial_oracle():
    x = fi.dense(2, 40, 70, 4, 2, 8, "bf16", seed=3, causal=True)
    O, L = oracle.attention(fi.to_f64(x.q, "bf16"), fi.to_f64(x.k, "bf16"), fi.to_f64(x.v, "bf16"),
                            x.scale, True)
    for b in range(2):
        o, l = full_oracle.dense_heads(x, [3, 0, 2], b=b)
        np.testing.assert_array_equal(o, O[b][:, [3, 0, 2]])
        np.testing.assert_array_equal(l, L[b][:, [3, 0, 2]])
    rows = np.array([0, 17, 39])
    o, l = full_oracle.dense_heads(x, [1], rows=rows, b=1)
    np.testing.assert_array_equal(o[:, 0], O[1, rows, 1])
    np.testing.assert_array_equal(l[:, 0], L[1, rows, 1])


def test_varlen_all_equals_serial_oracle():
    x = fi.varlen([5, 0, 33, 1], [9, 4, 33, 0], 6, 3, 8, "f16", seed=4, causal=True)
    O, L = oracle.attention_varlen(fi.to_f64(x.q, "f16"), fi.to_f64(x.k, "f16"),
                                   fi.to_f64(x.v, "f16"), x.cu_q, x.cu_k, x.scale, True)
    o, l = full_oracle.varlen_all(x.q, x.k, x.v, x.cu_q, x.cu_k, "f16", x.scale, True)
    np.testing.assert_array_equal(o, O)
    np.testing.assert_array_equal(l, L)


def test_decode_all_equals_serial_oracle():
    x = fi.paged([1, 20, 0, 47], 8, 2, 16, "bf16", seed=5)
    O, L = oracle.decode(fi.to_f64(x.q, "bf16"), fi.to_f64(x.k_seq, "bf16"),
                         fi.to_f64(x.v_seq, "bf16"), x.cu_k, x.scale)
    seq = lambda src: (lambda b: src[x.cu_k[b]:x.cu_k[b + 1]])
    o, l = full_oracle.decode_all(x.q, seq(x.k_seq), seq(x.v_seq), "bf16", x.scale)
    np.testing.assert_array_equal(o, O)
    np.testing.assert_array_equal(l, L)
