"""ctypes binding of ``libsapaged.so`` (the C ABI declared in include/paged_attn.h).

Argument marshalling only: tensors supply device pointers, shapes and strides;
the current torch stream is passed through; every step of the computation
runs in the library's HIP kernels.  Importing this module fails loudly when
the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsapaged.so")

PA_BF16, PA_FP16, PA_FP8_E4M3, PA_F32 = 1, 2, 3, 4
PA_OK, PA_EINVAL, PA_ENOTSUP, PA_EWORKSPACE, PA_EHIP = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "PA_OK", -1: "PA_EINVAL", -2: "PA_ENOTSUP", -3: "PA_EWORKSPACE", -4: "PA_EHIP"}


class PaKvDesc(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_kvp = ctypes.POINTER(PaKvDesc)

# name -> (restype, argtypes); mirrors include/paged_attn.h
SIGNATURES = {
    "paged_attn_run": (ctypes.c_int, [_vp, _i32, _kvp, _vp, _i64, _i32, _vp, _i32, _i32, _i32, _i32,
                                      _f32, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "paged_attn_run_noalloc": (ctypes.c_int, [_vp, _i32, _kvp, _vp, _i64, _i32, _vp, _i32, _i32,
                                              _i32, _i32, _f32, _i32, _i32, _vp, _i32, _vp, _vp]),
    "paged_attn_run_causal": (ctypes.c_int, [_vp, _i32, _kvp, _vp, _i64, _i32, _vp, _i32, _i32, _i32,
                                             _i32, _f32, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "paged_attn_resolve_splits": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attn_plan": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attn_partial": (ctypes.c_int, [_vp, _i32, _kvp, _vp, _i64, _i32, _vp, _i32, _i32, _i32,
                                          _i32, _f32, _i32, _i32, _vp, _vp, _vp]),
    "split_kv_combine": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp]),
    "segment_attn_combine": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp,
                                            _i32, _vp, _vp]),
    "segment_attn_run": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "segment_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "paged_attn_window_width": (_i32, [_i32, _i32, _i32, _i32]),
    "paged_attn_describe": (ctypes.c_int, [_vp, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _vp, _vp, _i32, _vp, _vp]),
    "paged_attn_describe_host": (ctypes.c_int, [_vp, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "paged_kv_write": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp, _kvp, _vp]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
}

_LIB = None


def load() -> ctypes.CDLL:
    """Load the built library (RuntimeError if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m segmented_attention_paged_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(code: int) -> None:
    if code != PA_OK:
        raise PagedAttnError(code, load().pa_last_error().decode())


def last_error() -> str:
    return load().pa_last_error().decode()
