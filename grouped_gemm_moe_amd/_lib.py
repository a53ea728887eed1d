"""ctypes loader for libmoegmm.so (the C ABI declared in include/moegmm.h).

There is no fallback: if the library is missing or does not load, importing
the binding raises.  Build it with ``python -m grouped_gemm_moe_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.environ.get("MOEGMM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libmoegmm.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int

# name -> (restype, argtypes); mirrors include/moegmm.h
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_int]),
    "moegmm_abi_version": (_int, []),
    "moe_permute_workspace_size": (_sz, [_i64, _i64, _i64]),
    "moe_permute": (_int, [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_permute_noalloc": (_int, [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "moe_permute_index": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p, _p]),
    "gmm_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "gmm_fwd": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _sz, _p, _p]),
    "gmm_fwd_swiglu": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _sz, _p, _p]),
    "gmm_fwd_gather": (_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _sz, _p, _p]),
    "gmm_fwd_swiglu_gather": (_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p,
                                     _sz, _p, _p]),
    "swiglu_gmm_fwd": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p]),
    "gmm_bwd_input": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _sz, _p, _p]),
    "gmm_bwd_weight": (_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _sz, _p, _p]),
    "gmm_bwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _sz, _p, _p]),
    "gmm_bwd_swiglu": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _sz, _p, _p]),
    "swiglu": (_int, [_p, _p, _i64, _i64, _i64, _p, _p]),
    "swiglu_bwd": (_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p]),
    "moe_unpermute": (_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p]),
    "moe_decode_fwd_mx": (_int, [_p, _p, _i64, _p, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _p, _p, _p, _p, _p, _p, _i64, _p, _p, _p]),
    "moe_decode_fwd": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p,
                              _p, _p]),
    "moe_unpermute_bwd": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "moe_permute_bwd": (_int, [_p, _p, _i64, _i64, _i64, _p, _p, _p]),
    "mx_quantize": (_int, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "moe_permute_mx": (_int, [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _p, _p, _sz,
                              _p, _p]),
    "gmm_mx_fwd": (_int, [_p, _p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "gmm_mx_fwd_swiglu": (_int, [_p, _p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _p,
                                 _i64, _p, _p]),
    "gmm_mx_fwd_swiglu_gather": (_int, [_p, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _p, _i64, _i64, _i64,
                                        _i64, _p, _p, _i64, _p, _p]),
}

ABI_VERSION = 11

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m grouped_gemm_moe_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moegmm_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {lib.moegmm_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib
