"""ctypes loader of libmoe_mi355x.so (the C ABI of include/moe.h).

The library is built in-tree by ``mixture_experts_layer_expert_amd.csrc.build``.
Loading fails loudly when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_ACT_GELU = 0
MOE_ACT_RELU = 1
MOE_ACT_SWIGLU = 2
MOE_RENORM = 1
MOE_RESIDUAL = 2
MOE_HAS_BIAS = 4
MOE_ROUTER_BIAS = 8
MOE_FUSED_DECODE = 16
MOE_SLOT_MAJOR = 32
MOE_PADDED = 64
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("moe_capacity", "moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn",
            "moe_expert_up", "moe_expert_down", "moe_combine", "moe_forward", "moe_stats_workspace_bytes",
            "moe_route_stats", "moe_router_stats", "moe_route_fallback", "moe_dispatch_reroute",
            "moe_status_string", "moe_clock_probe", "moe_forward_noalloc")


class MoeShapeC(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("D", ctypes.c_int32),
        ("F", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("n_shared", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_shape_p = ctypes.POINTER(MoeShapeC)
_SIGS = {
    "moe_capacity": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]),
    "moe_workspace_bytes": (ctypes.c_int, [_shape_p, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_stats_workspace_bytes": (ctypes.c_int, [_shape_p, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route_stats": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_router_stats": (ctypes.c_int, [_shape_p, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_dispatch": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_route_fallback": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                          _vp]),
    "moe_dispatch_reroute": (ctypes.c_int, [_shape_p, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp]),
    "moe_expert_ffn": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]),
    "moe_expert_up": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                     _vp]),
    "moe_expert_down": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_combine": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_forward": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_forward_noalloc": (ctypes.c_int, [_shape_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_clock_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_double, ctypes.c_int32, _vp, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build the HIP library first "
            "(python -m mixture_experts_layer_expert_amd.csrc.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
