"""Plain CPU oracle for appending tokens to a paged K/V cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the
tests and nothing on the product path; it shares no code with the GPU
library.

What it computes
----------------
The paged cache of "I/O-Aware Kernels", section "FlashInfer: I/O-aware
attention for serving" (keys and values gathered from paged KV layouts),
read as: a pool of pages of 16 token slots, each slot holding the K (or V)
row of one token for every KV head, and a page table that lists, for every
sequence, the physical page of its tokens 16*i .. 16*i+15. Appending n new
tokens to a sequence that holds L tokens writes token i of the batch to
position L + i of that sequence: page page_table[s][(L+i) // 16], slot
(L+i) % 16. Nothing else in the pool changes. The operation moves bits, so
the result is exact.

The loop below is that definition, one token at a time.
"""
from __future__ import annotations

import numpy as np

PAGE_SIZE = 16


def append(pool, new_rows, cu_new, page_table, seq_lens_before):
    """Return a copy of `pool` ([P, 16, Hkv, d]) with the token rows of
    `new_rows` ([T_new, Hkv, d], sequence s owning rows cu_new[s] ..
    cu_new[s+1]-1) written after the seq_lens_before[s] tokens each sequence
    already holds."""
    out = np.array(pool, copy=True)
    B = len(cu_new) - 1
    for s in range(B):
        base = int(seq_lens_before[s])
        for i in range(int(cu_new[s]), int(cu_new[s + 1])):
            pos = base + (i - int(cu_new[s]))
            page = int(page_table[s][pos // PAGE_SIZE])
            out[page, pos % PAGE_SIZE] = new_rows[i]
    return out


def gather(pool, page_table, seq_len, s):
    """The contiguous [seq_len, Hkv, d] rows of sequence s read back through
    the page table (the inverse view of `append`)."""
    rows = [pool[int(page_table[s][t // PAGE_SIZE]), t % PAGE_SIZE] for t in range(int(seq_len))]
    return np.stack(rows) if rows else np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
