"""ctypes view of ``libmoe_mxfp4.so`` (declared in include/moe_mxfp4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Loading fails loudly when the library has not been built; there
is no fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe_mxfp4.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_MODE = -3
MOE_ERR_ALIGN = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_HIP = -6

MOE_SCORING_SOFTMAX = 0
MOE_SCORING_SIGMOID = 1
MOE_ACT_SILU_MUL = 0
MOE_ACT_SWIGLU_OAI = 1
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_ENCODE_OCP = 0
MOE_ENCODE_QUARK = 1
MOE_LAYOUT_ROWS = 0
MOE_LAYOUT_TILE16 = 1
MOE_PAIRING_AUTO = 0
MOE_PAIRING_ON = 1
MOE_PAIRING_OFF = 2
MOE_W13_GATE_UP = 0
MOE_W13_INTERLEAVED = 1
MOE_MMA_BF16 = 0
MOE_MMA_SCALED_FP4 = 1
MOE_SCRATCH_BYTES = 64 << 20

EXPORTED = (
    "moe_mxfp4_workspace_bytes",
    "moe_mxfp4_decode",
    "moe_mxfp4_decode_noalloc",
    "moe_mxfp4_plan",
    "moe_mxfp4_route",
    "moe_mxfp4_bucket",
    "moe_mxfp4_plan_read",
    "moe_mxfp4_gate_up",
    "moe_mxfp4_down",
    "moe_mxfp4_decode_routes",
    "moe_mxfp4_down_routes",
    "moe_mxfp4_prefill_workspace_bytes",
    "moe_mxfp4_prefill",
    "moe_mxfp4_unpack",
    "moe_mxfp4_dequant",
    "moe_mxfp4_tile_weights",
    "moe_mxfp4_encode",
    "moe_mxfp4_status_string",
    "moe_mxfp4_version",
)


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("E_global", ctypes.c_int32),
        ("E_local", ctypes.c_int32),
        ("expert_offset", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("scoring", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("swiglu_alpha", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float),
        ("weight_layout", ctypes.c_int32),
        ("down_pairing", ctypes.c_int32),
        ("w13_order", ctypes.c_int32),
        ("mma", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_DESC = ctypes.POINTER(MoeDesc)

_SIGNATURES = {
    "moe_mxfp4_workspace_bytes": (_I32, [_DESC, ctypes.POINTER(_SZ)]),
    "moe_mxfp4_decode": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_decode_noalloc": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_mxfp4_plan": (_I32, [_DESC, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_gate_up": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_down": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_decode_routes": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_down_routes": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_prefill_workspace_bytes": (_I32, [_DESC, ctypes.POINTER(_SZ)]),
    "moe_mxfp4_prefill": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_unpack": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_route": (_I32, [_DESC, _P, _P, _P, _P]),
    "moe_mxfp4_bucket": (_I32, [_DESC, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_plan_read": (_I32, [_DESC, _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "moe_mxfp4_dequant": (_I32, [_P, _P, _I64, _I64, _I32, _P, _P]),
    "moe_mxfp4_tile_weights": (_I32, [_P, _I64, _I64, _I32, _P]),
    "moe_mxfp4_encode": (_I32, [_P, _I32, _I64, _I64, _I32, _P, _P, _P]),
    "moe_mxfp4_status_string": (ctypes.c_char_p, [_I32]),
    "moe_mxfp4_version": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m mxfp4_mixture_experts_router_amd.build "
                "or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib
