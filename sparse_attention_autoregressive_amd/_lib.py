"""ctypes view of libfastar.so (the C ABI declared in include/fastar.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfastar.so")

FASTAR_OK = 0
FASTAR_EINVAL = -1
FASTAR_EDTYPE = -2
FASTAR_ESHAPE = -3
FASTAR_EWORKSPACE = -4
FASTAR_ECAPACITY = -5
FASTAR_EHIP = -6
FASTAR_ESCRATCH = -7

FASTAR_F32 = 0
FASTAR_BF16 = 1
FASTAR_MAX_PLANES = 10
FASTAR_MAX_HASH_PLANES = 16
FASTAR_MAX_TABLES = 8
FASTAR_MAX_CODEWORDS = 65536
FASTAR_HASH_BATCH = 4
FASTAR_TIMER_MAX = 8192
FASTAR_ABI_VERSION = 3
FASTAR_STATIC_SCRATCH_BYTES = 16 << 20


class FastarCache(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("cap", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("ids", ctypes.c_void_p), ("ts", ctypes.c_void_p), ("n_valid", ctypes.c_void_p),
                ("knorm", ctypes.c_void_p), ("count", ctypes.c_void_p)]


class FastarKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_float)]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "fastar_status_string": (ctypes.c_char_p, [_i32]),
    "fastar_abi_version": (_i32, []),
    "fastar_ann_hash": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "fastar_ann_hash_batch": (_i32, [_i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp]),
    "fastar_ann_quantize": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "fastar_ann_quantize_batch": (_i32, [_i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp]),
    "fastar_bucket_sort_workspace": (_sz, [_i32, _i32, _i32]),
    "fastar_bucket_sort": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "fastar_annsa_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "fastar_annsa_forward": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, ctypes.POINTER(FastarCache),
                                    _vp, _vp, _vp, _i32, _i32, _f32, _vp, _i32, _vp, _vp, _vp,
                                    _vp, _sz, _vp]),
    "fastar_annsa_forward_static": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, ctypes.POINTER(FastarCache),
                                           _vp, _vp, _vp, _i32, _i32, _f32, _vp, _i32, _vp, _vp, _vp, _vp]),
    "fastar_annsa_multi_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "fastar_annsa_multi_forward": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32,
                                          ctypes.POINTER(FastarCache), _vp, _vp, _vp, _i32, _i32,
                                          _i32, _f32, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fastar_annca_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "fastar_annca_forward": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                                    _i32, _f32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "fastar_tempcache_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "fastar_tempcache_update": (_i32, [ctypes.POINTER(FastarCache), _vp, _vp, _vp, _vp, _vp, _i32,
                                       _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _sz, _vp]),
    "fastar_tempcache_order": (_i32, [ctypes.POINTER(FastarCache), _i32, _vp, _vp]),
    "fastar_timer_start": (_i32, []),
    "fastar_timer_stop": (_i32, [ctypes.POINTER(FastarKernelTime), _i32]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_attention_autoregressive_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.fastar_abi_version() != FASTAR_ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.fastar_abi_version()}, the binding "
                               f"expects {FASTAR_ABI_VERSION}: rebuild the library")
        _lib = lib
    return _lib


class FastarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = load().fastar_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")


def check(fn: str, status: int) -> None:
    if status != FASTAR_OK:
        raise FastarError(fn, status)
