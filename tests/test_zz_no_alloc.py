"""moe_mxfp4_decode_noalloc (the layer call on the library's own per-GPU
workspace) against moe_mxfp4_decode with a caller workspace, through the C
ABI: two calls in a row, the second smaller, bit-identical outputs that also
meet the oracle bar; a call whose workspace would not fit is refused."""

import numpy as np
import pytest

import mxfp4_mixture_experts_router_amd as moe
import oracle
from workloads import get_config, make_inputs, make_weights

from gpu_util import DeviceLayer, bf16_bits_np, bf16_to_np, desc_for, dev_bf16, dev_f32, torch

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _both(cfg, layer, inp):
    t = torch()
    T = inp.x.shape[0]
    d = desc_for(cfg, T, weight_layout=layer.layout)
    x, lg = dev_bf16(inp.x), dev_f32(inp.logits)
    ref_out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_decode(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, ref_out, router_logits=lg,
                         w13_bias=layer.b13, w2_bias=layer.b2, workspace=ws)
    out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_decode_noalloc(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, out, router_logits=lg,
                                 w13_bias=layer.b13, w2_bias=layer.b2)
    t.cuda.synchronize()
    return out, ref_out


@pytest.mark.parametrize("name,layout,tokens", [("gptoss20b", "tile16", (32, 4)), ("tiny", "rows", (16, 3))])
def test_noalloc_matches_decode_on_consecutive_calls(name, layout, tokens):
    cfg = get_config(name)
    w = make_weights(cfg)
    layer = DeviceLayer(w, layout=layout)
    for call, T in enumerate(tokens):
        inp = make_inputs(cfg, T, call=call)
        out, ref_out = _both(cfg, layer, inp)
        assert np.array_equal(bf16_bits_np(out), bf16_bits_np(ref_out)), (name, T)
        y = bf16_to_np(out)
        ref = oracle.moe_forward_cfg(cfg, w, inp)["y"]
        assert np.isfinite(y).all()
        r, c = oracle.rel_l2(y, ref), oracle.cosine(y, ref)
        print(f"noalloc {name} T={T}: rel_l2 {r:.3e} cosine {c:.7f}", flush=True)
        assert r <= 3e-3 and c >= 0.9999, (name, T, r, c)


def test_noalloc_refuses_a_call_larger_than_its_workspace():
    t = torch()
    cfg = get_config("widek")
    T = 2048  # 16384 routes: the per-route rows alone are far above the fixed workspace
    d = desc_for(cfg, T)
    assert moe.moe_mxfp4_workspace_bytes(d) > moe.MOE_SCRATCH_BYTES
    x = t.zeros((T, cfg.K), dtype=t.bfloat16, device="cuda")
    lg = t.zeros((T, cfg.E_global), dtype=t.float32, device="cuda")
    out = t.zeros((T, cfg.K), dtype=t.bfloat16, device="cuda")
    w13p = t.zeros((cfg.E_local, 2 * cfg.I, cfg.K // 2), dtype=t.uint8, device="cuda")
    w13s = t.zeros((cfg.E_local, 2 * cfg.I, cfg.K // 32), dtype=t.uint8, device="cuda")
    w2p = t.zeros((cfg.E_local, cfg.K, cfg.I // 2), dtype=t.uint8, device="cuda")
    w2s = t.zeros((cfg.E_local, cfg.K, cfg.I // 32), dtype=t.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_mxfp4_decode_noalloc(d, x, w13p, w13s, w2p, w2s, out, router_logits=lg)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
