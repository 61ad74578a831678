"""ctypes binding of ``libfa_amd.so`` (the C ABI declared in include/fa.h).

Argument marshalling only: every arithmetic step runs in the library's HIP
kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_amd.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_NO_SPACE = 0, 1, 2, 3, 4
# bytes of the fixed device buffer behind fa_decode_paged_noalloc
DECODE_NOALLOC_MAX_WORKSPACE = 64 << 20
FA_F32, FA_F16, FA_BF16 = 0, 1, 2

EXPORTS = ("fa_status_string", "fa_version", "fa_fwd", "fa_fwd_varlen", "fa_fwd_paged",
           "fa_decode_paged_workspace_size", "fa_decode_paged", "fa_decode_cascade_workspace_size",
           "fa_decode_cascade", "fa_kv_append", "fa_decode_paged_noalloc", "fa_bwd_workspace_size",
           "fa_bwd")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_version": (_i, []),
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "fa_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                           _i, _f, _i, _vp]),
    # q k_pool v_pool o lse cu_q page_table seq_lens B max_q Tq max_pages num_pages page_size
    # Hq Hkv d dtype scale causal stream
    "fa_fwd_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                          _i, _i, _f, _i, _vp]),
    "fa_decode_paged_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "fa_decode_cascade_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    # q k_pool v_pool o lse prefix_pages prefix_len page_table seq_lens B max_pages num_pages
    # page_size Hq Hkv d dtype scale workspace workspace_bytes stream
    "fa_decode_cascade": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                               _i, _i, _f, _vp, _sz, _vp]),
    # k_new v_new k_pool v_pool cu_new page_table seq_lens_before B T_new max_pages num_pages
    # page_size Hkv d dtype stream
    "fa_kv_append": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "fa_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                             _f, _i, _vp, _sz, _vp]),
    "fa_bwd_workspace_size": (_sz, [_i, _i, _i]),
    # q k v o lse dout dq dk dv B Nq Nk Hq Hkv d dtype scale causal workspace workspace_bytes stream
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                    _vp, _sz, _vp]),
    # the same without workspace and workspace_bytes
    "fa_decode_paged_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                     _i, _f, _i, _vp]),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it is missing: there is no
    fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m io_aware_exact_flashattention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FA_OK:
        raise FaError(status, load().fa_status_string(status).decode())
