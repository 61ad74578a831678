"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the CPU oracle and the GPU path. It holds random
number generation, rounding of float32 draws to the storage dtype, and the
layout of the generated tensors (dense rows, packed ragged batches, a paged
key/value pool). It holds no attention arithmetic.

Storage conventions
-------------------
* ``"f32"`` tensors are ``np.float32``.
* ``"f16"`` tensors are ``np.float16`` (numpy's cast is round-to-nearest-even).
* ``"bf16"`` tensors are ``np.uint16`` arrays holding bfloat16 bit patterns,
  rounded from float32 with round-to-nearest-even (``f32_to_bf16_bits``).

Random streams
--------------
Every tensor comes from its own PCG64 stream, so that large tensors can be
drawn on several threads without changing any value:

* ``default_rng(seed)``          - structure: lengths, then the page permutation;
* ``default_rng([seed, 1])``      - Q;
* ``default_rng([seed, 2, c])``   - K, chunk c;
* ``default_rng([seed, 3, c])``   - V, chunk c;
* ``default_rng([seed, 4])``      - the output gradient dO of the backward pass.

Dense tensors are drawn in chunks of whole leading rows (``_CHUNK_ROWS``
rows of the flattened ``[rows, H, d]`` view); ragged and paged K/V are drawn
one sequence per chunk. Every draw is ``standard_normal(dtype=float32)``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
PAGE_SIZE = 16
_CHUNK_ROWS = 2048


# ---------------------------------------------------------------- rounding --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the upper 16 bits of the rounded float32 pattern as uint16.
    NaN inputs map to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + (np.uint32(0x7FFF) + lsb)
    out = (r >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage representation of ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def element_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


# ----------------------------------------------------------------- drawing --
def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_chunks(seed: int, tag: int, shapes, dtype: str, out: np.ndarray):
    """Fill ``out`` (first axis split as ``shapes``) from per-chunk streams."""
    offs = np.concatenate([[0], np.cumsum([s[0] for s in shapes])]).astype(np.int64)

    def work(c):
        rng = np.random.default_rng([seed, tag, c])
        x = rng.standard_normal(shapes[c], dtype=np.float32)
        out[offs[c]:offs[c + 1]] = round_to(x, dtype)

    if len(shapes) == 1:
        work(0)
        return
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(shapes))))


def _draw_rows(seed: int, tag: int, rows: int, tail: tuple, dtype: str) -> np.ndarray:
    out = np.empty((rows,) + tail, dtype=storage_dtype(dtype))
    if rows == 0:
        return out
    shapes = []
    r = 0
    while r < rows:
        n = min(_CHUNK_ROWS, rows - r)
        shapes.append((n,) + tail)
        r += n
    _draw_chunks(seed, tag, shapes, dtype, out)
    return out


def _draw_q(seed: int, shape: tuple, dtype: str) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


def default_scale(d: int) -> float:
    """1/sqrt(d) as the float32 value passed to every implementation."""
    return float(np.float32(1.0 / math.sqrt(d)))


# ------------------------------------------------------------------ dense --
@dataclass
class Dense:
    q: np.ndarray          # [B, Nq, Hq, d]
    k: np.ndarray          # [B, Nk, Hkv, d]
    v: np.ndarray          # [B, Nk, Hkv, d]
    dtype: str
    causal: bool
    scale: float
    name: str = ""

    @property
    def shape(self):
        B, Nq, Hq, d = self.q.shape
        return B, Nq, self.k.shape[1], Hq, self.k.shape[2], d


def dense(B, Nq, Nk, Hq, Hkv, d, dtype, seed, causal, q_mult=1.0, name="") -> Dense:
    """i.i.d. N(0,1) Q/K/V in [B, N, H, d] layout; Q optionally multiplied
    by ``q_mult`` in float32 before rounding."""
    q = np.random.default_rng([seed, 1]).standard_normal((B, Nq, Hq, d), dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    q = round_to(q, dtype)
    k = _draw_rows(seed, 2, B * Nk, (Hkv, d), dtype).reshape(B, Nk, Hkv, d)
    v = _draw_rows(seed, 3, B * Nk, (Hkv, d), dtype).reshape(B, Nk, Hkv, d)
    return Dense(q, k, v, dtype, causal, default_scale(d), name)


def grad_out(shape, dtype, seed) -> np.ndarray:
    """An output gradient dO for the backward pass: i.i.d. N(0,1) of the
    given shape from its own stream ``default_rng([seed, 4])``, rounded to
    the storage type."""
    rng = np.random.default_rng([seed, 4])
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


# ----------------------------------------------------------------- varlen --
@dataclass
class Varlen:
    q: np.ndarray          # [Tq, Hq, d]
    k: np.ndarray          # [Tk, Hkv, d]
    v: np.ndarray          # [Tk, Hkv, d]
    cu_q: np.ndarray       # int32 [B+1]
    cu_k: np.ndarray       # int32 [B+1]
    dtype: str
    causal: bool
    scale: float
    name: str = ""

    @property
    def max_q(self):
        return int(np.diff(self.cu_q).max()) if len(self.cu_q) > 1 else 0

    @property
    def max_k(self):
        return int(np.diff(self.cu_k).max()) if len(self.cu_k) > 1 else 0


def varlen(lens_q, lens_k, Hq, Hkv, d, dtype, seed, causal, name="") -> Varlen:
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = _draw_q(seed, (int(cu_q[-1]), Hq, d), dtype)
    k = _draw_rows(seed, 2, int(cu_k[-1]), (Hkv, d), dtype)
    v = _draw_rows(seed, 3, int(cu_k[-1]), (Hkv, d), dtype)
    return Varlen(q, k, v, cu_q, cu_k, dtype, causal, default_scale(d), name)


# ------------------------------------------------------------------ paged --
@dataclass
class Paged:
    q: np.ndarray              # [B, Hq, d]   one query token per sequence
    k_seq: np.ndarray          # [T, Hkv, d]  contiguous K of all sequences
    v_seq: np.ndarray          # [T, Hkv, d]
    cu_k: np.ndarray           # int32 [B+1]  offsets of each sequence in k_seq
    k_pool: np.ndarray         # [P, PAGE_SIZE, Hkv, d]
    v_pool: np.ndarray
    page_table: np.ndarray     # int32 [B, max_pages], unused entries -1
    seq_lens: np.ndarray       # int32 [B]
    dtype: str
    scale: float
    name: str = ""
    tail_fill: str = "zero"

    @property
    def num_pages(self):
        return self.k_pool.shape[0]

    @property
    def max_pages(self):
        return self.page_table.shape[1]


def _tail_value(dtype, fill):
    if fill == "zero":
        return 0
    if fill == "nan":
        return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]
    raise ValueError(fill)


def paged(lens, Hq, Hkv, d, dtype, seed, permute=True, tail_fill="zero", rng=None,
          name="") -> Paged:
    """Decode inputs: one query token per sequence and K/V scattered into a
    pool of 16-token pages through a page table.

    The pool holds exactly sum(ceil(len/16)) pages. With ``permute`` the
    sequences' logical pages, taken in order, are assigned the physical pages
    of one random permutation of the pool (drawn from ``rng``, default the
    structure stream ``default_rng(seed)``); otherwise the identity. Slots of
    a last page beyond the sequence end hold ``tail_fill``.
    """
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    npg = -(-lens // PAGE_SIZE)
    P = int(npg.sum())
    if rng is None:
        rng = np.random.default_rng(seed)
    perm = rng.permutation(P) if permute else np.arange(P)
    max_pages = max(1, int(npg.max()) if B else 1)
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    off = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    for b in range(B):
        pt[b, :npg[b]] = perm[off[b]:off[b + 1]]
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu_k[-1])
    q = _draw_q(seed, (B, Hq, d), dtype)
    k_seq = np.empty((T, Hkv, d), dtype=storage_dtype(dtype))
    v_seq = np.empty((T, Hkv, d), dtype=storage_dtype(dtype))
    shapes = [(int(n), Hkv, d) for n in lens]
    if T:
        _draw_chunks(seed, 2, shapes, dtype, k_seq)
        _draw_chunks(seed, 3, shapes, dtype, v_seq)
    # physical slot of every token: page_table[b, t // 16] * 16 + t % 16
    seq_of = np.repeat(np.arange(B), lens)
    t_in = np.arange(T) - cu_k[seq_of]
    slot = pt[seq_of, t_in // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + t_in % PAGE_SIZE
    fill = _tail_value(dtype, tail_fill)
    k_pool = np.full((P * PAGE_SIZE, Hkv, d), fill, dtype=storage_dtype(dtype))
    v_pool = np.full((P * PAGE_SIZE, Hkv, d), fill, dtype=storage_dtype(dtype))
    k_pool[slot] = k_seq
    v_pool[slot] = v_seq
    k_pool = k_pool.reshape(P, PAGE_SIZE, Hkv, d)
    v_pool = v_pool.reshape(P, PAGE_SIZE, Hkv, d)
    return Paged(q, k_seq, v_seq, cu_k.astype(np.int32), k_pool, v_pool, pt,
                 lens.astype(np.int32), dtype, default_scale(d), name, tail_fill)


@dataclass
class PagedPrefill:
    """A ragged batch of query chunks plus a paged cache holding every key of
    each sequence (cached prefix and the chunk itself)."""
    q: np.ndarray              # [Tq, Hq, d]
    cu_q: np.ndarray           # int32 [B+1]
    kv: Paged                  # pools, page table, seq_lens and the contiguous K/V

    @property
    def max_q(self):
        return int(np.diff(self.cu_q).max()) if len(self.cu_q) > 1 else 0


def paged_prefill(lens_q, lens_k, Hq, Hkv, d, dtype, seed, permute=True, tail_fill="zero",
                  name="") -> PagedPrefill:
    """Chunked-prefill inputs: chunk s has lens_q[s] query tokens and its
    sequence lens_k[s] >= lens_q[s] keys in the paged pool (same pool layout,
    permutation and K/V streams as `paged`). Queries are drawn on the Q
    stream as one packed [Tq, Hq, d] tensor."""
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    assert np.all(lens_q <= lens_k)
    kv = paged(lens_k, Hq, Hkv, d, dtype, seed, permute=permute, tail_fill=tail_fill, name=name)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    q = _draw_q(seed, (int(cu_q[-1]), Hq, d), dtype)
    return PagedPrefill(q, cu_q, kv)


@dataclass
class Cascade:
    """Decode inputs for sequences that share a cached prefix: one pool holds
    the prefix pages and every sequence's own pages."""
    q: np.ndarray              # [B, Hq, d]
    pool: Paged                # row 0 of its page table: the prefix; rows 1..B: suffixes
    prefix_len: int

    @property
    def prefix_pages(self):
        return self.pool.page_table[0, :(self.prefix_len + PAGE_SIZE - 1) // PAGE_SIZE]

    @property
    def page_table(self):
        return np.ascontiguousarray(self.pool.page_table[1:])

    @property
    def seq_lens(self):
        return self.pool.seq_lens[1:]

    def keys(self, b, which="k"):
        """Contiguous keys (or values) of sequence b: prefix then suffix."""
        src = self.pool.k_seq if which == "k" else self.pool.v_seq
        cu = self.pool.cu_k
        return np.concatenate([src[cu[0]:cu[1]], src[cu[b + 1]:cu[b + 2]]])


def cascade(prefix_len, suffix_lens, Hq, Hkv, d, dtype, seed, permute=True, tail_fill="zero",
            name="") -> Cascade:
    lens = np.concatenate([[prefix_len], np.asarray(suffix_lens, dtype=np.int64)])
    pool = paged(lens, Hq, Hkv, d, dtype, seed, permute=permute, tail_fill=tail_fill, name=name)
    q = _draw_q(seed + 1000, (len(lens) - 1, Hq, d), dtype)
    return Cascade(q, pool, int(prefix_len))


def chunked_prefill_lengths(seed=5, B=16):
    """A chunked-prefill batch: cached prefixes U[0, 8192] and chunks U[1, 2048]
    tokens (keys = prefix + chunk)."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 8192, B, endpoint=True)
    chunk = rng.integers(1, 2048, B, endpoint=True)
    return chunk, prefix + chunk


# ---------------------------------------------------- the five workloads --
CONFIG_TEXT = (
    "single-head exact attention, no mask: B=1 H=1 Nq=Nk=256 d=64 fp32",
    "causal multi-head prefill: B=4 H=16 N=2048 d=64 bf16",
    "long-context causal prefill: B=1 H=32 N=16384 d=128 bf16",
    "ragged varlen GQA causal prefill: 8 sequences, lengths U[128,4096], Hq=32 Hkv=8 d=128 bf16",
    "paged-KV GQA decode: 64 sequences, KV lengths U[512,32768], page 16, Hq=32 Hkv=8 d=128 bf16",
)


def cfg0(seed=0):
    return dense(1, 256, 256, 1, 1, 64, "f32", seed, causal=False, name="cfg0")


def cfg1(seed=1, dtype="bf16", q_mult=1.0):
    return dense(4, 2048, 2048, 16, 16, 64, dtype, seed, causal=True, q_mult=q_mult,
                 name=f"cfg1-{dtype}" + ("" if q_mult == 1.0 else f"-qx{q_mult:g}"))


def cfg2(seed=2):
    return dense(1, 16384, 16384, 32, 32, 128, "bf16", seed, causal=True, name="cfg2")


def cfg3_lengths(seed=3):
    return np.random.default_rng(seed).integers(128, 4096, 8, endpoint=True)


def cfg3(seed=3):
    lens = cfg3_lengths(seed)
    return varlen(lens, lens, 32, 8, 128, "bf16", seed, causal=True, name="cfg3")


def cfg4_lengths(seed=4):
    return np.random.default_rng(seed).integers(512, 32768, 64, endpoint=True)


def cfg4(seed=4, tail_fill="zero", permute=True):
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 32768, 64, endpoint=True)
    return paged(lens, 32, 8, 128, "bf16", seed, permute=permute, tail_fill=tail_fill,
                 rng=rng, name="cfg4")


# --------------------------------------------------- work / byte counts ----
def prefill_flops(lens_q, lens_k, Hq, d, causal) -> float:
    """4*Hq*Nq*Nk*d per sequence, halved when causal."""
    f = sum(4.0 * Hq * int(a) * int(b) * d for a, b in zip(lens_q, lens_k))
    return f / 2 if causal else f


def decode_kv_bytes(lens, Hkv, d, dtype) -> int:
    """K plus V bytes of every valid token: the decode pass must read them all."""
    return int(np.sum(np.asarray(lens, dtype=np.int64))) * Hkv * d * element_bytes(dtype) * 2
