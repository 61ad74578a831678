"""MI355X (gfx950) exact attention forward: Python binding of libfa_amd.so.

Each function is one call into the C ABI (include/fa.h), enqueued on torch's
current HIP stream; the attention calls return (O, LSE):

* ``fwd(q, k, v, causal=False, scale=None)`` - dense [B, N, H, d];
* ``fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, ...)`` -
  packed ragged [T, H, d];
* ``fwd_paged(q, k_pool, v_pool, cu_seqlens_q, page_table, seq_lens, ...)`` -
  chunked prefill against a paged K/V cache;
* ``decode_paged(q, k_pool, v_pool, page_table, seq_lens, ...)`` - one token
  per sequence against a paged K/V cache;
* ``decode_paged_noalloc(...)`` - the same through the entry point that
  allocates nothing (split partials in the library's fixed device buffer);
* ``decode_cascade(q, k_pool, v_pool, prefix_pages, prefix_len, ...)`` - one
  token per sequence, the sequences sharing one cached prefix;
* ``kv_append(k_new, v_new, k_pool, v_pool, cu_new, page_table, ...)`` -
  write new tokens' K/V rows into the paged cache;
* ``bwd(q, k, v, o, lse, dout, causal=False, ...)`` - gradients (dQ, dK, dV)
  of dense attention from the forward pass's O and LSE.

PyTorch only allocates device memory and supplies the stream; the arithmetic
runs in the library's kernels. There is no CPU or PyTorch fallback: on a
machine without the built library every call raises. The device arrays'
contents (cu_seqlens, page tables, lengths) are preconditions the library
does not check; shapes, dtypes, devices and the head dimension of every
tensor are checked here before the call.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import FaError

__all__ = ["fwd", "fwd_varlen", "fwd_paged", "decode_paged", "decode_paged_noalloc",
           "decode_cascade", "kv_append", "bwd", "decode_workspace_size",
           "bwd_workspace_size", "FaError", "default_scale"]

_DT = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32, the value the library receives."""
    import struct
    return struct.unpack("f", struct.pack("f", 1.0 / math.sqrt(d)))[0]


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t: torch.Tensor, name: str):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be on the GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _outputs(q: torch.Tensor, out, lse, lse_shape):
    """O (like q) and LSE (float32, lse_shape): the caller's, checked, or new."""
    o = torch.empty_like(q) if out is None else out
    l = torch.empty(lse_shape, dtype=torch.float32, device=q.device) if lse is None else lse
    _dev_tensor(o, "out")
    _dev_tensor(l, "lse")
    _need(o.shape == q.shape and o.dtype == q.dtype and o.device == q.device, "bad out")
    _need(tuple(l.shape) == tuple(lse_shape) and l.dtype == torch.float32
          and l.device == q.device, "bad lse")
    return o, l


def _workspace(workspace, need: int, device):
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _dev_tensor(workspace, "workspace")
    _need(workspace.device == device, "workspace must be on the device of q")
    return workspace


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None):
    """Dense attention. q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] -> (O like q,
    LSE float32 [B, Nq, Hq])."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, n)
    _need(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "bad shapes")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, dk = k.shape
    _need(k.shape[0] == B and dk == d, "k/v must match q in batch and head dim")
    _need(k.device == q.device and v.device == q.device, "q, k, v must be on one device")
    if scale is None:
        scale = default_scale(d)
    o, l = _outputs(q, out, lse, (B, Nq, Hq))
    _lib.check(lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                          B, Nq, Nk, Hq, Hkv, d, _dtype(q), float(scale), int(bool(causal)),
                          _stream(q)))
    return o, l


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, scale: float | None = None,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Packed ragged batch. q [Tq, Hq, d], k/v [Tk, Hkv, d], cu_seqlens int32
    [B+1] on the GPU -> (O like q, LSE float32 [Tq, Hq])."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                 ("cu_seqlens_k", cu_seqlens_k)):
        _dev_tensor(t, n)
    _need(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape, "bad shapes")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32,
          "cu_seqlens must be int32")
    _need(cu_seqlens_q.shape == cu_seqlens_k.shape and cu_seqlens_q.dim() == 1, "bad cu_seqlens")
    Tq, Hq, d = q.shape
    Tk, Hkv, dk = k.shape
    _need(dk == d, "k/v must match q in head dim")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = default_scale(d)
    o, l = _outputs(q, out, lse, (Tq, Hq))
    _lib.check(lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 l.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                 B, int(max_seqlen_q), int(max_seqlen_k), Tq, Tk, Hq, Hkv, d,
                                 _dtype(q), float(scale), int(bool(causal)), _stream(q)))
    return o, l


def fwd_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
              cu_seqlens_q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
              max_seqlen_q: int, causal: bool = True, scale: float | None = None,
              out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Chunked prefill against a paged cache. q [Tq, Hq, d] packed by
    cu_seqlens_q (int32 [B+1]); pools [num_pages, 16, Hkv, d]; page_table
    int32 [B, max_pages]; seq_lens int32 [B] = keys of each sequence, the
    chunk included -> (O like q, LSE float32 [Tq, Hq])."""
    lib = _lib.load()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("cu_seqlens_q", cu_seqlens_q),
                 ("page_table", page_table), ("seq_lens", seq_lens)):
        _dev_tensor(t, n)
    _need(q.dim() == 3 and k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "bad shapes")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "q and pools must share a dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and page_table.dtype == torch.int32
          and seq_lens.dtype == torch.int32, "indices must be int32")
    Tq, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_pool.shape
    _need(dk == d, "pools must match q in head dim")
    _need(cu_seqlens_q.dim() == 1, "bad cu_seqlens_q")
    B = cu_seqlens_q.shape[0] - 1
    _need(page_table.dim() == 2 and page_table.shape[0] == B and seq_lens.shape == (B,),
          "bad index shapes")
    if scale is None:
        scale = default_scale(d)
    o, l = _outputs(q, out, lse, (Tq, Hq))
    _lib.check(lib.fa_fwd_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), o.data_ptr(),
                                l.data_ptr(), cu_seqlens_q.data_ptr(), page_table.data_ptr(),
                                seq_lens.data_ptr(), B, int(max_seqlen_q), Tq,
                                page_table.shape[1], num_pages, page_size, Hq, Hkv, d, _dtype(q),
                                float(scale), int(bool(causal)), _stream(q)))
    return o, l


def decode_cascade(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   prefix_pages: torch.Tensor | None, prefix_len: int, page_table: torch.Tensor,
                   seq_lens: torch.Tensor, scale: float | None = None,
                   workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None):
    """Decode of sequences sharing one prefix: q [B, Hq, d]; prefix_pages
    int32 [ceil(prefix_len/16)]; page_table int32 [B, max_pages] and seq_lens
    int32 [B] describe each sequence's own suffix -> (O like q, LSE [B, Hq])."""
    lib = _lib.load()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("page_table", page_table),
                 ("seq_lens", seq_lens)):
        _dev_tensor(t, n)
    if prefix_len > 0:
        _dev_tensor(prefix_pages, "prefix_pages")
        _need(prefix_pages.dtype == torch.int32, "prefix_pages must be int32")
    _need(q.dim() == 3 and k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "bad shapes")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "q and pools must share a dtype")
    _need(page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "indices must be int32")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_pool.shape
    _need(dk == d, "pools must match q in head dim")
    _need(page_table.dim() == 2 and page_table.shape[0] == B and seq_lens.shape == (B,),
          "bad index shapes")
    max_pages = page_table.shape[1]
    if scale is None:
        scale = default_scale(d)
    need = int(lib.fa_decode_cascade_workspace_size(B, Hq, d, int(prefix_len), max_pages,
                                                    page_size))
    workspace = _workspace(workspace, need, q.device)
    o, l = _outputs(q, out, lse, (B, Hq))
    pp = prefix_pages.data_ptr() if (prefix_pages is not None and prefix_len > 0) else None
    _lib.check(lib.fa_decode_cascade(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                     o.data_ptr(), l.data_ptr(), pp, int(prefix_len),
                                     page_table.data_ptr(), seq_lens.data_ptr(), B, max_pages,
                                     num_pages, page_size, Hq, Hkv, d, _dtype(q), float(scale),
                                     workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(q)))
    return o, l


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
              v_pool: torch.Tensor, cu_new: torch.Tensor, page_table: torch.Tensor,
              seq_lens_before: torch.Tensor) -> None:
    """Write new tokens' K/V rows ([T_new, Hkv, d], packed by cu_new int32
    [B+1]) into the pools after the seq_lens_before tokens each sequence
    holds. The pools are updated in place; seq_lens is the caller's."""
    lib = _lib.load()
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool),
                 ("cu_new", cu_new), ("page_table", page_table),
                 ("seq_lens_before", seq_lens_before)):
        _dev_tensor(t, n)
    _need(k_new.dim() == 3 and k_new.shape == v_new.shape and k_pool.dim() == 4
          and k_pool.shape == v_pool.shape, "bad shapes")
    _need(k_new.dtype == v_new.dtype == k_pool.dtype == v_pool.dtype, "tensors must share a dtype")
    _need(cu_new.dtype == page_table.dtype == seq_lens_before.dtype == torch.int32,
          "indices must be int32")
    T_new, Hkv, d = k_new.shape
    num_pages, page_size, Hkv_p, d_p = k_pool.shape
    _need(Hkv_p == Hkv and d_p == d, "pool row shape differs from the new rows")
    _need(cu_new.dim() == 1 and cu_new.shape[0] >= 2, "bad cu_new")
    B = cu_new.shape[0] - 1
    _need(page_table.dim() == 2 and page_table.shape[0] == B and seq_lens_before.shape == (B,),
          "bad index shapes")
    _lib.check(lib.fa_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                                v_pool.data_ptr(), cu_new.data_ptr(), page_table.data_ptr(),
                                seq_lens_before.data_ptr(), B, T_new, page_table.shape[1],
                                num_pages, page_size, Hkv, d, _dtype(k_new), _stream(k_new)))


def decode_workspace_size(B: int, Hq: int, d: int, max_pages: int, page_size: int = 16,
                          num_splits: int = 0) -> int:
    return int(_lib.load().fa_decode_paged_workspace_size(B, Hq, d, max_pages, page_size,
                                                          num_splits))


def bwd_workspace_size(B: int, Nq: int, Hq: int) -> int:
    return int(_lib.load().fa_bwd_workspace_size(B, Nq, Hq))


def _decode_args(q, k_pool, v_pool, page_table, seq_lens):
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("page_table", page_table),
                 ("seq_lens", seq_lens)):
        _dev_tensor(t, n)
    _need(q.dim() == 3 and k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "bad shapes")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "q and pools must share a dtype")
    _need(page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "indices must be int32")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_pool.shape
    _need(dk == d, "pools must match q in head dim")
    _need(page_table.dim() == 2 and page_table.shape[0] == B and seq_lens.shape == (B,),
          "bad index shapes")
    return B, Hq, d, num_pages, page_size, Hkv, page_table.shape[1]


def decode_paged_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                         page_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int = 0,
                         scale: float | None = None, out: torch.Tensor | None = None,
                         lse: torch.Tensor | None = None):
    """Paged decode through ``fa_decode_paged_noalloc``: the library call
    allocates nothing (its split partials go to a fixed device buffer of
    DECODE_NOALLOC_MAX_WORKSPACE bytes; FaError FA_ERR_NO_SPACE beyond it).
    Pass ``out`` and ``lse`` to keep this function from allocating them.
    Same arguments and results as ``decode_paged``."""
    lib = _lib.load()
    B, Hq, d, num_pages, page_size, Hkv, max_pages = _decode_args(q, k_pool, v_pool, page_table,
                                                                  seq_lens)
    if scale is None:
        scale = default_scale(d)
    o, l = _outputs(q, out, lse, (B, Hq))
    _lib.check(lib.fa_decode_paged_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                           o.data_ptr(), l.data_ptr(), page_table.data_ptr(),
                                           seq_lens.data_ptr(), B, max_pages, num_pages, page_size,
                                           Hq, Hkv, d, _dtype(q), float(scale), int(num_splits),
                                           _stream(q)))
    return o, l


def decode_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 page_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int = 0,
                 scale: float | None = None, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Paged decode. q [B, Hq, d]; pools [num_pages, 16, Hkv, d]; page_table
    int32 [B, max_pages]; seq_lens int32 [B] -> (O like q, LSE float32 [B, Hq])."""
    lib = _lib.load()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("page_table", page_table),
                 ("seq_lens", seq_lens)):
        _dev_tensor(t, n)
    _need(q.dim() == 3 and k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "bad shapes")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "q and pools must share a dtype")
    _need(page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "indices must be int32")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_pool.shape
    _need(dk == d, "pools must match q in head dim")
    _need(page_table.dim() == 2 and page_table.shape[0] == B and seq_lens.shape == (B,),
          "bad index shapes")
    max_pages = page_table.shape[1]
    if scale is None:
        scale = default_scale(d)
    need = int(lib.fa_decode_paged_workspace_size(B, Hq, d, max_pages, page_size, num_splits))
    workspace = _workspace(workspace, need, q.device)
    o, l = _outputs(q, out, lse, (B, Hq))
    _lib.check(lib.fa_decode_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                   o.data_ptr(), l.data_ptr(), page_table.data_ptr(),
                                   seq_lens.data_ptr(), B, max_pages, num_pages, page_size, Hq,
                                   Hkv, d, _dtype(q), float(scale), int(num_splits),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(q)))
    return o, l


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, scale: float | None = None,
        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Gradients of dense attention. q, o, dout [B, Nq, Hq, d]; k, v [B, Nk,
    Hkv, d]; lse float32 [B, Nq, Hq] as returned by ``fwd`` -> (dQ like q,
    dK like k, dV like v)."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        _dev_tensor(t, n)
    _need(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "bad shapes")
    _need(o.shape == q.shape and dout.shape == q.shape, "o and dout must be shaped like q")
    _need(q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype, "tensors must share a dtype")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, dk_ = k.shape
    _need(k.shape[0] == B and dk_ == d, "k/v must match q in batch and head dim")
    _need(tuple(lse.shape) == (B, Nq, Hq) and lse.dtype == torch.float32, "bad lse")
    for t in (k, v, o, lse, dout):
        _need(t.device == q.device, "tensors must be on one device")
    if scale is None:
        scale = default_scale(d)
    grads = []
    for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        g = torch.empty_like(like) if g is None else g
        _dev_tensor(g, name)
        _need(g.shape == like.shape and g.dtype == like.dtype and g.device == q.device,
              f"bad {name}")
        grads.append(g)
    need = int(lib.fa_bwd_workspace_size(B, Nq, Hq))
    workspace = _workspace(workspace, need, q.device)
    _lib.check(lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                          grads[2].data_ptr(), B, Nq, Nk, Hq, Hkv, d, _dtype(q), float(scale),
                          int(bool(causal)), workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream(q)))
    return tuple(grads)
