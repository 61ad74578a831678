"""Brute-force scalar twin of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle.attention``). Pure Python loops and
``math.exp``/``math.log`` on nested lists: every logit, weight and output
element is written out one at a time, with no array library. It serves as an
independent pin of the vectorised oracle on sizes of a few rows.

The definition followed is the one of "I/O-Aware Kernels", section "Naive
attention": softmax over each row of the scaled score matrix, then the
weighted sum of value rows; bottom-right causal masking, natural-log
log-sum-exp, and O = 0 / lse = -inf for a row that sees no key.
"""
from __future__ import annotations

import math


def attention_head(q, k, v, scale, causal):
    nq, nk = len(q), len(k)
    dv = len(v[0]) if nk else 0
    out, lses = [], []
    for i in range(nq):
        visible = [j for j in range(nk) if (not causal) or j <= i + (nk - nq)]
        if not visible:
            out.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        logits = []
        for j in visible:
            dot = 0.0
            for t in range(len(q[i])):
                dot += q[i][t] * k[j][t]
            logits.append(dot * scale)
        top = max(logits)
        weights = [math.exp(x - top) for x in logits]
        total = sum(weights)
        row = []
        for c in range(dv):
            acc = 0.0
            for w, j in zip(weights, visible):
                acc += w * v[j][c]
            row.append(acc / total)
        out.append(row)
        lses.append(top + math.log(total))
    return out, lses
