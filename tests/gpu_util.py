"""Helpers for the GPU tests: move seeded numpy inputs to the device and run
the library's entry points through the Python binding (which calls the C ABI).
"""

import numpy as np

import mxfp4_mixture_experts_router_amd as moe


def torch():
    import torch as _t
    return _t


def dev_u8(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_bf16(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(t.bfloat16)


def dev_f32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bf16_to_np(t):
    """Device bf16 tensor -> float32 numpy (exact)."""
    bits = t.detach().view(torch().int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32)


def bf16_bits_np(t):
    return t.detach().view(torch().int16).cpu().numpy().view(np.uint16)


class DeviceLayer:
    """Weights of one layer slice resident on the device.

    layout "tile16" tiles the packed weights in place on the device with the
    library's own entry point after the upload (the row-layout bytes are what
    the generators and the oracle use).
    """

    def __init__(self, w, layout="rows"):
        self.w13p = dev_u8(w.w13_packed)
        self.w13s = dev_u8(w.w13_scales)
        self.w2p = dev_u8(w.w2_packed)
        self.w2s = dev_u8(w.w2_scales)
        self.b13 = dev_bf16(w.b13) if w.b13 is not None else None
        self.b2 = dev_bf16(w.b2) if w.b2 is not None else None
        self.E_local = w.w13_packed.shape[0]
        self.layout = layout
        if layout == "tile16":
            moe.moe_mxfp4_tile_weights(self.w13p)
            moe.moe_mxfp4_tile_weights(self.w2p)


def desc_for(cfg, T, E_local=None, expert_offset=None, weight_layout="rows", down_pairing="auto",
             w13_order="gate_up", mma="bf16"):
    return moe.make_desc(T=T, K=cfg.K, I=cfg.I, E_global=cfg.E_global,
                         E_local=cfg.E_local if E_local is None else E_local, top_k=cfg.top_k,
                         expert_offset=cfg.expert_offset if expert_offset is None else expert_offset,
                         scoring=cfg.scoring, activation=cfg.activation,
                         swiglu_alpha=cfg.swiglu_alpha, swiglu_limit=cfg.swiglu_limit,
                         weight_layout=weight_layout, down_pairing=down_pairing, w13_order=w13_order, mma=mma)


def run_decode(cfg, layer, inp, expert_offset=None, workspace=None, stream=None, down_pairing="auto",
               w13_order="gate_up", mma="bf16"):
    t = torch()
    T = inp.x.shape[0]
    d = desc_for(cfg, T, E_local=layer.E_local, expert_offset=expert_offset, weight_layout=layer.layout,
                 down_pairing=down_pairing, w13_order=w13_order, mma=mma)
    x = dev_bf16(inp.x)
    out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    kw = {}
    if inp.logits is not None:
        kw["router_logits"] = dev_f32(inp.logits)
    else:
        kw["topk_ids"] = dev_i32(inp.topk_ids)
        kw["topk_weights"] = dev_f32(inp.topk_weights)
    moe.moe_mxfp4_decode(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, out,
                         w13_bias=layer.b13, w2_bias=layer.b2, workspace=workspace, stream=stream, **kw)
    t.cuda.synchronize()
    return out
