"""ctypes loader for libmxsg.so (the C ABI declared in include/mxsg.h).

Argument marshalling only. The library must have been built first
(``python -m mx_scaled_grouped_amd.build``); a missing library raises, so
nothing silently falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxsg.so")

OK, INVALID_ARGUMENT, BAD_SHAPE, UNSUPPORTED, HIP_ERROR = 0, 1, 2, 3, 4

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32

# name -> (restype, argtypes), mirroring include/mxsg.h
SIGNATURES = {
    "mxsg_status_str": (ctypes.c_char_p, [_i32]),
    "mxsg_last_error": (ctypes.c_char_p, []),
    "mxsg_version": (_i32, []),
    "mxsg_padded_capacity": (_i64, [_i64, _i32]),
    "mxsg_quantize_act_sizes": (_i32, [_i64, _i64, _i32, _i32, _i32, _c_p]),
    "mxsg_quantize_weight_sizes": (_i32, [_i32, _i64, _i64, _i32, _i32, _c_p]),
    "mxsg_grouped_mm_check": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _i64,
                                     _i32]),
    "mxsg_quantize_act": (_i32, [_c_p, _i64, _i64, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                 _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "mxsg_quantize_act_swiglu": (_i32, [_c_p, _i64, _i64, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p,
                                        _c_p, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "mxsg_quantize_act_gather": (_i32, [_c_p, _i64, _c_p, _i64, _i64, _i32, _i32, _i32, _c_p, _c_p,
                                        _c_p, _c_p, _c_p, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "mxsg_quantize_weight": (_i32, [_c_p, _i32, _i64, _i64, _i32, _i32, _c_p, _c_p, _c_p, _c_p,
                                    _c_p, _c_p, _c_p, _c_p, _c_p]),
    "mxsg_delayed_update": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _i32, _i32, _i32, _c_p]),
    "mxsg_grouped_mm": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64, _i64, _i64, _c_p, _c_p, _c_p,
                               _c_p, _i64, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p]),
    "mxsg_cast_sweep": (_i32, [_u32, _i64, _i32, _c_p, _c_p]),
    "mxsg_route": (_i32, [_c_p, _i64, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "mxsg_swiglu": (_i32, [_c_p, _i64, _i64, _c_p, _c_p]),
    "mxsg_sigmoid_sweep": (_i32, [_c_p, _c_p]),
    "mxsg_stream_copy": (_i32, [_c_p, _c_p, _i64, _c_p]),
    "mxsg_clock_probe": (_i32, [_i32, _i32, _c_p, _c_p]),
    "mxsg_wall_clock_rate_khz": (_i32, [_c_p]),
}

_lib = None


class MxsgError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed ({status}): {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mx_scaled_grouped_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call an entry point returning mxsg_status; raise MxsgError unless OK."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != OK:
        raise MxsgError(st, name, lib.mxsg_last_error().decode())


def status_of(name: str, *args) -> int:
    """Call an entry point and return its status (for tests of argument checking)."""
    return getattr(load(), name)(*args)
