"""ctypes loader of libdg_fp8.so. Fails loudly when the library is missing."""
from __future__ import annotations

import ctypes
import os

from . import build as _build

_i64 = ctypes.c_int64
_p = ctypes.c_void_p

# Entry points declared in include/dg_fp8.h, with their argument types.
SIGNATURES = {
    "dg_abi_version": (ctypes.c_int, []),
    "dg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dg_last_hip_error": (ctypes.c_int, []),
    "dg_fp8_gemm_nt": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64,
                                      _p, _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_gemm_nt_ws": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64,
                                         _p, _i64, _i64, _i64, _i64, _p, _i64, _p]),
    "dg_fp8_gemm_nt_workspace_bytes": (ctypes.c_int64, [_i64, _i64, _i64]),
    "dg_fp8_gemm_nt_noalloc": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64,
                                              _p, _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous_ws": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                         _p, _i64, _i64, _i64, _p, _p, _p, _p, _i64, _i64,
                                                         _i64, _i64, _i64, _i64, _p, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous_workspace_bytes": (ctypes.c_int64, [_i64, _i64, _i64, _i64]),
    "dg_fp8_gemm_nt_fmt": (ctypes.c_int, [_p, ctypes.c_int, _i64, _p, _i64, _i64, _p, ctypes.c_int, _i64,
                                          _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                      _p, _i64, _i64, _i64, _p, _p, _i64,
                                                      _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous_to_tokens": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                                _p, _i64, _i64, _i64, _p, _p, _p, _p, _i64, _i64,
                                                                _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous_layout": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                             _p, _i64, _i64, _i64, _p, _p, _p, _i64,
                                                             _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_contiguous_fmt": (ctypes.c_int, [_p, ctypes.c_int, _i64, _p, _i64, _i64, _p, ctypes.c_int,
                                                          _i64, _i64, _p, _i64, _i64, _i64, _p, _p, _i64,
                                                          _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_masked_fmt": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _p, _i64, _i64, _i64,
                                                      _p, ctypes.c_int, _i64, _i64, _p, _i64, _i64, _i64, _p,
                                                      _p, _i64, _i64, _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_grouped_gemm_masked": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _i64, _i64,
                                                  _p, _i64, _i64, _p, _i64, _i64, _i64, _p,
                                                  _p, _i64, _i64, _i64, _i64, _i64, _i64, _p]),
    "dg_fp8_quantize_1x128": (ctypes.c_int, [_p, ctypes.c_int, _i64, _p, _i64, _p, _i64, _i64,
                                             _i64, _i64, _p]),
    "dg_fp8_quantize_1x128_gather": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _p, _p, _i64, _p, _i64,
                                                    _i64, _i64, _i64, _p]),
    "dg_moe_route_contiguous": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _p, _i64, _p]),
    "dg_moe_contiguous_max_rows": (ctypes.c_int64, [_i64, _i64]),
    "dg_moe_unpermute": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _i64, _p, _i64, _p]),
}

_lib = None


def path() -> str:
    return _build.LIBRARY


def load() -> ctypes.CDLL:
    """Load the HIP library (built beforehand by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIBRARY):
            raise ImportError(
                "libdg_fp8.so is not built (expected at %s); run "
                "`python -c 'import __graft_entry__ as g; g.build()'` first" % _build.LIBRARY)
        lib = ctypes.CDLL(_build.LIBRARY)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
