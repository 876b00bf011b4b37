"""MI355X (gfx950) routed-expert MXFP4 MoE decode layer.

Python binding of ``libmoe_mxfp4.so`` with the same entry points as the C ABI
in ``include/moe_mxfp4.h``.  It only marshals arguments: it checks dtypes,
shapes, devices and contiguity of torch tensors (refusing anything unexpected
rather than re-typing it) and passes their device pointers and the stream
handle to the library, where every step of the layer runs.  PyTorch supplies
device memory and streams.
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import (  # noqa: F401
    MOE_ACT_SILU_MUL,
    MOE_ACT_SWIGLU_OAI,
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_ENCODE_OCP,
    MOE_ENCODE_QUARK,
    MOE_ERR_ALIGN,
    MOE_ERR_HIP,
    MOE_ERR_MODE,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_WORKSPACE,
    MOE_LAYOUT_ROWS,
    MOE_LAYOUT_TILE16,
    MOE_PAIRING_AUTO,
    MOE_PAIRING_OFF,
    MOE_PAIRING_ON,
    MOE_SCRATCH_BYTES,
    MOE_W13_GATE_UP,
    MOE_W13_INTERLEAVED,
    MOE_MMA_BF16,
    MOE_MMA_SCALED_FP4,
    MOE_OK,
    MOE_SCORING_SIGMOID,
    MOE_SCORING_SOFTMAX,
    MoeDesc,
)

__all__ = [
    "MoeDesc", "MoeError", "make_desc", "moe_mxfp4_workspace_bytes", "moe_mxfp4_decode", "moe_mxfp4_decode_noalloc",
    "moe_mxfp4_plan", "moe_mxfp4_gate_up", "moe_mxfp4_down", "moe_mxfp4_route", "moe_mxfp4_bucket",
    "moe_mxfp4_plan_read", "moe_mxfp4_decode_routes", "moe_mxfp4_down_routes", "moe_mxfp4_prefill",
    "moe_mxfp4_prefill_workspace_bytes", "moe_mxfp4_unpack",
    "moe_mxfp4_dequant", "moe_mxfp4_tile_weights", "moe_mxfp4_encode", "moe_mxfp4_status_string", "moe_mxfp4_version",
]

_SCORING = {"softmax": MOE_SCORING_SOFTMAX, "sigmoid": MOE_SCORING_SIGMOID}
_ACT = {"silu_mul": MOE_ACT_SILU_MUL, "swiglu_oai": MOE_ACT_SWIGLU_OAI}
_LAYOUT = {"rows": MOE_LAYOUT_ROWS, "tile16": MOE_LAYOUT_TILE16}
_PAIRING = {"auto": MOE_PAIRING_AUTO, "on": MOE_PAIRING_ON, "off": MOE_PAIRING_OFF}
_W13_ORDER = {"gate_up": MOE_W13_GATE_UP, "interleaved": MOE_W13_INTERLEAVED}
_MMA = {"bf16": MOE_MMA_BF16, "scaled_fp4": MOE_MMA_SCALED_FP4}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_mxfp4_status_string(status)} ({status})")


def make_desc(T: int, K: int, I: int, E_global: int, E_local: int, top_k: int, expert_offset: int = 0,
              scoring="softmax", activation="silu_mul", swiglu_alpha: float = 1.702,
              swiglu_limit: float = 7.0, weight_layout="rows", down_pairing="auto",
              w13_order="gate_up", mma="bf16") -> MoeDesc:
    sc = _SCORING[scoring] if isinstance(scoring, str) else int(scoring)
    ac = _ACT[activation] if isinstance(activation, str) else int(activation)
    wl = _LAYOUT[weight_layout] if isinstance(weight_layout, str) else int(weight_layout)
    dp = _PAIRING[down_pairing] if isinstance(down_pairing, str) else int(down_pairing)
    wo = _W13_ORDER[w13_order] if isinstance(w13_order, str) else int(w13_order)
    mm = _MMA[mma] if isinstance(mma, str) else int(mma)
    return MoeDesc(T, K, I, E_global, E_local, expert_offset, top_k, sc, ac, swiglu_alpha, swiglu_limit, wl, dp, wo, mm)


def moe_mxfp4_status_string(status: int) -> str:
    return _lib.lib().moe_mxfp4_status_string(int(status)).decode()


def moe_mxfp4_version() -> str:
    return _lib.lib().moe_mxfp4_version().decode()


def _torch():
    import torch
    return torch


def _ptr(t, dtype, shape, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_mxfp4_workspace_bytes(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.lib().moe_mxfp4_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "moe_mxfp4_workspace_bytes")
    return n.value


def _workspace(desc, workspace, device, stream=None):
    torch = _torch()
    need = moe_mxfp4_workspace_bytes(desc)
    if workspace is None:
        # Allocated on the stream the call runs on: the caching allocator then
        # hands the block out again only to later work on that same stream, so
        # a workspace the caller drops is never given to another stream (or
        # thread) while the call's kernels still read it.
        if stream is None:
            ts = torch.cuda.current_stream(device)
        elif isinstance(stream, torch.cuda.Stream):
            ts = stream
        else:
            ts = torch.cuda.ExternalStream(int(stream), device=device)
        with torch.cuda.stream(ts):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 device tensor")
    return workspace, workspace.data_ptr(), workspace.numel()


def _planned_workspace(desc, workspace, name):
    """The workspace of a step that reads a plan: it must be the caller's,
    holding the plan of an earlier call (a fresh buffer holds none)."""
    torch = _torch()
    if workspace is None:
        raise ValueError(f"{name} reads the plan held in a workspace: pass the workspace of the "
                         "moe_mxfp4_plan (or layer) call that made it")
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 device tensor")
    if workspace.numel() < moe_mxfp4_workspace_bytes(desc):
        raise ValueError(f"{name}: workspace smaller than moe_mxfp4_workspace_bytes()")
    return workspace, workspace.data_ptr(), workspace.numel()


def _weights_shapes(d: MoeDesc, E: Optional[int] = None):
    E = d.E_local if E is None else E
    return ((E, 2 * d.I, d.K // 2), (E, 2 * d.I, d.K // 32), (E, 2 * d.I),
            (E, d.K, d.I // 2), (E, d.K, d.I // 32), (E, d.K))


def moe_mxfp4_decode(desc: MoeDesc, x, w13_packed, w13_scales, w2_packed, w2_scales, out,
                     router_logits=None, topk_ids=None, topk_weights=None, w13_bias=None, w2_bias=None,
                     workspace=None, stream=None):
    """One layer call; ``out`` (bf16 [T, K]) is overwritten.  Returns the workspace used."""
    torch = _torch()
    d = desc
    s13p, s13s, s13b, s2p, s2s, s2b = _weights_shapes(d)
    ws, wsp, wsn = _workspace(d, workspace, x.device, stream)
    _check(_lib.lib().moe_mxfp4_decode(
        ctypes.byref(d),
        _ptr(x, torch.bfloat16, (d.T, d.K), "x"),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits", True),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w13_bias, torch.bfloat16, s13b, "w13_bias", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out, torch.bfloat16, (d.T, d.K), "out"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_decode")
    return ws


def moe_mxfp4_decode_noalloc(desc: MoeDesc, x, w13_packed, w13_scales, w2_packed, w2_scales, out,
                             router_logits=None, topk_ids=None, topk_weights=None, w13_bias=None, w2_bias=None,
                             stream=None):
    """One layer call on the library's own per-GPU workspace (no allocation
    anywhere in the call); ``out`` (bf16 [T, K]) is overwritten.  Calls that
    overlap on one GPU race."""
    torch = _torch()
    d = desc
    s13p, s13s, s13b, s2p, s2s, s2b = _weights_shapes(d)
    _check(_lib.lib().moe_mxfp4_decode_noalloc(
        ctypes.byref(d),
        _ptr(x, torch.bfloat16, (d.T, d.K), "x"),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits", True),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w13_bias, torch.bfloat16, s13b, "w13_bias", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out, torch.bfloat16, (d.T, d.K), "out"),
        _stream(stream)), "moe_mxfp4_decode_noalloc")


def moe_mxfp4_plan(desc: MoeDesc, router_logits=None, topk_ids=None, topk_weights=None, workspace=None,
                   stream=None, device=None):
    """Routing + bucketing into the workspace (returned)."""
    torch = _torch()
    d = desc
    dev = next((t.device for t in (router_logits, topk_ids, topk_weights) if t is not None), device)
    ws, wsp, wsn = _workspace(d, workspace, dev, stream)
    _check(_lib.lib().moe_mxfp4_plan(
        ctypes.byref(d),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits", True),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        wsp, wsn, _stream(stream)), "moe_mxfp4_plan")
    return ws


def moe_mxfp4_gate_up(desc: MoeDesc, x, w13_packed, w13_scales, workspace, a=None, w13_bias=None, stream=None):
    """Gate/up step on the plan held in ``workspace``; writes ``a`` [T*top_k, I] bf16 (or the workspace copy)."""
    torch = _torch()
    d = desc
    s13p, s13s, s13b, _, _, _ = _weights_shapes(d)
    ws, wsp, wsn = _planned_workspace(d, workspace, "moe_mxfp4_gate_up")
    _check(_lib.lib().moe_mxfp4_gate_up(
        ctypes.byref(d),
        _ptr(x, torch.bfloat16, (d.T, d.K), "x"),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w13_bias, torch.bfloat16, s13b, "w13_bias", True),
        _ptr(a, torch.bfloat16, (d.T * d.top_k, d.I), "a", True),
        wsp, wsn, _stream(stream)), "moe_mxfp4_gate_up")


def moe_mxfp4_down(desc: MoeDesc, w2_packed, w2_scales, out, workspace, a=None, w2_bias=None, stream=None):
    """Down + combine step on the plan held in ``workspace``; ``a`` None reads the workspace copy."""
    torch = _torch()
    d = desc
    _, _, _, s2p, s2s, s2b = _weights_shapes(d)
    ws, wsp, wsn = _planned_workspace(d, workspace, "moe_mxfp4_down")
    _check(_lib.lib().moe_mxfp4_down(
        ctypes.byref(d),
        _ptr(a, torch.bfloat16, (d.T * d.top_k, d.I), "a", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out, torch.bfloat16, (d.T, d.K), "out"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_down")


def moe_mxfp4_decode_routes(desc: MoeDesc, x, w13_packed, w13_scales, w2_packed, w2_scales, out_routes,
                            router_logits=None, topk_ids=None, topk_weights=None, w13_bias=None, w2_bias=None,
                            workspace=None, stream=None):
    """One layer call with per-route output: ``out_routes`` fp32 [T*top_k, K] gets
    W2 a_r + b2 of every local route r (no routing weight), zeros elsewhere."""
    torch = _torch()
    d = desc
    s13p, s13s, s13b, s2p, s2s, s2b = _weights_shapes(d)
    ws, wsp, wsn = _workspace(d, workspace, x.device, stream)
    _check(_lib.lib().moe_mxfp4_decode_routes(
        ctypes.byref(d),
        _ptr(x, torch.bfloat16, (d.T, d.K), "x"),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits", True),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w13_bias, torch.bfloat16, s13b, "w13_bias", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out_routes, torch.float32, (d.T * d.top_k, d.K), "out_routes"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_decode_routes")
    return ws


def moe_mxfp4_down_routes(desc: MoeDesc, w2_packed, w2_scales, out_routes, workspace, a=None, w2_bias=None,
                          stream=None):
    """Per-route down step on the plan held in ``workspace``; ``a`` None reads the workspace copy."""
    torch = _torch()
    d = desc
    _, _, _, s2p, s2s, s2b = _weights_shapes(d)
    ws, wsp, wsn = _planned_workspace(d, workspace, "moe_mxfp4_down_routes")
    _check(_lib.lib().moe_mxfp4_down_routes(
        ctypes.byref(d),
        _ptr(a, torch.bfloat16, (d.T * d.top_k, d.I), "a", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out_routes, torch.float32, (d.T * d.top_k, d.K), "out_routes"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_down_routes")


def moe_mxfp4_prefill_workspace_bytes(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.lib().moe_mxfp4_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "moe_mxfp4_prefill_workspace_bytes")
    return n.value


def moe_mxfp4_prefill(desc: MoeDesc, x, w13_packed, w13_scales, w2_packed, w2_scales, out,
                      router_logits=None, topk_ids=None, topk_weights=None, w13_bias=None, w2_bias=None,
                      workspace=None, stream=None):
    """The prefill path (unpack the touched experts to bf16, then bf16 MFMA GEMMs);
    same results as ``moe_mxfp4_decode``.  Returns the workspace used."""
    torch = _torch()
    d = desc
    s13p, s13s, s13b, s2p, s2s, s2b = _weights_shapes(d)
    need = moe_mxfp4_prefill_workspace_bytes(d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 device tensor")
    _check(_lib.lib().moe_mxfp4_prefill(
        ctypes.byref(d),
        _ptr(x, torch.bfloat16, (d.T, d.K), "x"),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits", True),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w13_bias, torch.bfloat16, s13b, "w13_bias", True),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w2_bias, torch.bfloat16, s2b, "w2_bias", True),
        _ptr(out, torch.bfloat16, (d.T, d.K), "out"),
        workspace.data_ptr(), workspace.numel(), _stream(stream)), "moe_mxfp4_prefill")
    return workspace


def moe_mxfp4_unpack(desc: MoeDesc, w13_packed, w13_scales, w2_packed, w2_scales, w13_out, w2_out, workspace,
                     stream=None):
    """bf16 values of the packed weights of every expert the plan in ``workspace`` touches."""
    torch = _torch()
    d = desc
    s13p, s13s, _, s2p, s2s, _ = _weights_shapes(d)
    ws, wsp, wsn = _planned_workspace(d, workspace, "moe_mxfp4_unpack")
    _check(_lib.lib().moe_mxfp4_unpack(
        ctypes.byref(d),
        _ptr(w13_packed, torch.uint8, s13p, "w13_packed"),
        _ptr(w13_scales, torch.uint8, s13s, "w13_scales"),
        _ptr(w2_packed, torch.uint8, s2p, "w2_packed"),
        _ptr(w2_scales, torch.uint8, s2s, "w2_scales"),
        _ptr(w13_out, torch.bfloat16, (d.E_local, 2 * d.I, d.K), "w13_out"),
        _ptr(w2_out, torch.bfloat16, (d.E_local, d.K, d.I), "w2_out"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_unpack")


def moe_mxfp4_route(desc: MoeDesc, router_logits, topk_ids, topk_weights, stream=None):
    torch = _torch()
    d = desc
    _check(_lib.lib().moe_mxfp4_route(
        ctypes.byref(d),
        _ptr(router_logits, torch.float32, (d.T, d.E_global), "router_logits"),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids"),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights"),
        _stream(stream)), "moe_mxfp4_route")


def moe_mxfp4_bucket(desc: MoeDesc, topk_ids, counts, offsets, routes, workspace=None, stream=None):
    torch = _torch()
    d = desc
    ws, wsp, wsn = _workspace(d, workspace, topk_ids.device, stream)
    _check(_lib.lib().moe_mxfp4_bucket(
        ctypes.byref(d),
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids"),
        _ptr(counts, torch.int32, (d.E_local,), "counts"),
        _ptr(offsets, torch.int32, (d.E_local + 1,), "offsets"),
        _ptr(routes, torch.int32, (d.T * d.top_k,), "routes"),
        wsp, wsn, _stream(stream)), "moe_mxfp4_bucket")
    return ws


def moe_mxfp4_plan_read(desc: MoeDesc, workspace, topk_ids=None, topk_weights=None, counts=None, offsets=None,
                        routes=None, stream=None):
    """Copies of the routing (ids, weights [T, top_k]) and bucketing (counts
    [E_local], offsets [E_local + 1], routes [T*top_k]) held by the plan in
    ``workspace``; outputs left None are not written."""
    torch = _torch()
    d = desc
    ws, wsp, wsn = _planned_workspace(d, workspace, "moe_mxfp4_plan_read")
    _check(_lib.lib().moe_mxfp4_plan_read(
        ctypes.byref(d), wsp, wsn,
        _ptr(topk_ids, torch.int32, (d.T, d.top_k), "topk_ids", True),
        _ptr(topk_weights, torch.float32, (d.T, d.top_k), "topk_weights", True),
        _ptr(counts, torch.int32, (d.E_local,), "counts", True),
        _ptr(offsets, torch.int32, (d.E_local + 1,), "offsets", True),
        _ptr(routes, torch.int32, (d.T * d.top_k,), "routes", True),
        _stream(stream)), "moe_mxfp4_plan_read")


def moe_mxfp4_encode(values, packed, scales, rule="quark", stream=None):
    """values fp32 or bf16 [..., cols] -> packed u8 [..., cols/2] and scales u8 [..., cols/32] (MXFP4)."""
    torch = _torch()
    if values.dtype == torch.float32:
        code = MOE_DTYPE_F32
    elif values.dtype == torch.bfloat16:
        code = MOE_DTYPE_BF16
    else:
        raise TypeError(f"values must be float32 or bfloat16, got {values.dtype}")
    if values.dim() < 1:
        raise ValueError("values must have at least 1 dimension")
    cols = values.shape[-1]
    rows = values.numel() // cols if cols else 0
    lead = tuple(values.shape[:-1])
    r = {"ocp": MOE_ENCODE_OCP, "quark": MOE_ENCODE_QUARK}[rule] if isinstance(rule, str) else int(rule)
    _check(_lib.lib().moe_mxfp4_encode(
        _ptr(values, values.dtype, tuple(values.shape), "values"), code, rows, cols, r,
        _ptr(packed, torch.uint8, lead + (cols // 2,), "packed"),
        _ptr(scales, torch.uint8, lead + (cols // 32,), "scales"), _stream(stream)), "moe_mxfp4_encode")


def moe_mxfp4_tile_weights(packed, inverse=False, stream=None):
    """In place: packed u8 [..., rows, cols/2] between the row and the tiled layout.

    Leading axes (experts) are folded into the rows; rows per expert must be a
    multiple of 16.
    """
    torch = _torch()
    if packed.dim() < 2:
        raise ValueError("packed must have at least 2 dimensions")
    half = packed.shape[-1]
    rows = packed.numel() // half if half else 0
    _check(_lib.lib().moe_mxfp4_tile_weights(
        _ptr(packed, torch.uint8, tuple(packed.shape), "packed"), rows, 2 * half, 1 if inverse else 0,
        _stream(stream)), "moe_mxfp4_tile_weights")


def moe_mxfp4_dequant(packed, scales, out, stream=None):
    """packed u8 [rows, cols/2] + scales u8 [rows, cols/32] -> out fp32 or bf16 [rows, cols]."""
    torch = _torch()
    rows, half = packed.shape
    cols = 2 * half
    if out.dtype == torch.float32:
        code = MOE_DTYPE_F32
    elif out.dtype == torch.bfloat16:
        code = MOE_DTYPE_BF16
    else:
        raise TypeError(f"out must be float32 or bfloat16, got {out.dtype}")
    _check(_lib.lib().moe_mxfp4_dequant(
        _ptr(packed, torch.uint8, (rows, half), "packed"),
        _ptr(scales, torch.uint8, (rows, cols // 32), "scales"),
        rows, cols, code, _ptr(out, out.dtype, (rows, cols), "out"), _stream(stream)), "moe_mxfp4_dequant")
