"""Parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: dequantised values, top-k ids (the routing hook and the router
inside the plan kernel, read back from the plan), the bucketing permutation,
and a closed-form dyadic chain.  Floating-point outputs: rel_l2 <= 3e-3 and
cosine >= 0.9999 against the fp32 oracle (the acceptance bar of the layer;
the bf16 rounding of the output alone costs about 1.7e-3) over the whole
output and over every token on its own, every element within 2^-8 of its
reference plus 4e-3 of its token's RMS (a single wrong element cannot hide
in the norms), exact zeros for tokens without a local route, no non-finite
values.  Every token of every workload shape and token count is compared,
with the weights in the tiled layout the benchmark times, under the pages'
routings (random, and every route local) at activation RMS 1 and 4.
"""

import numpy as np
import pytest

import mxfp4_mixture_experts_router_amd as moe
import oracle
from workloads import (LayerConfig, LayerInputs, LayerWeights, get_config, make_inputs, make_topk_inputs,
                       make_weights)

from gpu_util import (DeviceLayer, bf16_bits_np, bf16_to_np, desc_for, dev_bf16, dev_f32, dev_i32, dev_u8,
                      run_decode, torch)

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

REL_L2 = 3e-3
COSINE = 0.9999


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    print("device:", t.cuda.get_device_name(0), "|", moe.moe_mxfp4_version(), flush=True)


def _cfg(**kw):
    base = dict(name="case", description="case", K=256, I=256, E_global=8, E_local=8, expert_offset=0,
                top_k=2, scoring="softmax", activation="silu_mul", bias=False, tokens=(4,),
                scale_lo=118, scale_hi=130, index=90)
    base.update(kw)
    return LayerConfig(**base)


ELEM_REL = 2.0 ** -8     # twice the bf16 output rounding
ELEM_RMS = 4e-3          # of the row's RMS: fp32 order and bf16 intermediate flips (~1e-4 expected)
# The element bound holds for the bf16 MFMA path, whose products are exact
# and whose sums are fp32.  v_mfma_scale_f32_16x16x128_f8f6f4 sums each
# 128-value chunk with an error of up to ~2^-10 of its largest product
# (measured on the device), so an output formed by cancellation can move by
# more than that bound; the scaled-FP4 path is held to the layer's bar
# (rel_l2 and cosine) over the whole output and for every token.


def _assert_close(y_gpu, y_ref, what, elementwise=True):
    assert np.isfinite(y_gpu).all(), f"{what}: {np.count_nonzero(~np.isfinite(y_gpu))} non-finite outputs"
    if not np.any(y_ref):
        assert not np.any(y_gpu), f"{what}: expected all zeros"
        return
    r = oracle.rel_l2(y_gpu, y_ref)
    c = oracle.cosine(y_gpu, y_ref)
    print(f"{what}: rel_l2 {r:.3e} cosine {c:.7f}", flush=True)
    assert r <= REL_L2 and c >= COSINE, (what, r, c)
    # every row (token, or route for per-route outputs) on its own
    g2 = np.atleast_2d(np.asarray(y_gpu, np.float64))
    r2 = np.atleast_2d(np.asarray(y_ref, np.float64))
    g2 = g2.reshape(-1, g2.shape[-1])
    r2 = r2.reshape(-1, r2.shape[-1])
    worst = 0.0
    for i in range(r2.shape[0]):
        if not np.any(r2[i]):
            assert not np.any(g2[i]), f"{what}: row {i} has no local route and must be zero"
            continue
        ri = oracle.rel_l2(g2[i], r2[i])
        worst = max(worst, ri)
        assert ri <= REL_L2, (what, "row", i, ri)
        if not elementwise:
            continue
        rms = np.sqrt(np.mean(r2[i] ** 2))
        bad = np.abs(g2[i] - r2[i]) > ELEM_REL * np.abs(r2[i]) + ELEM_RMS * rms
        assert not bad.any(), (what, "row", i, "elements", np.flatnonzero(bad)[:8].tolist(),
                               g2[i][bad][:4].tolist(), r2[i][bad][:4].tolist())
    print(f"{what}: worst row rel_l2 {worst:.3e}", flush=True)


# --------------------------------------------------------------------------
# dequantisation: bit-exact over every (code, scale, nibble position)
# --------------------------------------------------------------------------

def test_dequant_exhaustive_bit_exact():
    t = torch()
    byte_row = np.array([(i & 0xF) | ((15 - i) << 4) for i in range(16)], dtype=np.uint8)
    packed = np.tile(byte_row, (256, 4))            # 256 rows x 128 values (4 blocks)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 4, axis=1)
    scales[:, 1] = scales[:, 0][::-1]               # vary the scale per block too
    want = oracle.dequantize(packed, scales)
    out32 = t.empty((256, 128), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_dequant(dev_u8(packed), dev_u8(scales), out32)
    got = out32.cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))  # sign of -0 included
    out16 = t.empty((256, 128), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_dequant(dev_u8(packed), dev_u8(scales), out16)
    got16 = bf16_to_np(out16)
    # every finite E2M1 * 2^k value is a bf16 value, so the bf16 output is exact too
    assert np.array_equal(np.isnan(got16), nan)
    assert np.array_equal(got16[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_dequant_random_large():
    t = torch()
    rng = np.random.default_rng(1)
    rows, cols = 1000, 2880
    packed = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(100, 140, size=(rows, cols // 32), dtype=np.uint8)
    out = t.empty((rows, cols), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_dequant(dev_u8(packed), dev_u8(scales), out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.dequantize(packed, scales).view(np.uint32))


# --------------------------------------------------------------------------
# tiled weight layout: bit-exact permutation, in place
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(3, 64, 48), (32, 1440), (16, 4096), (48, 16), (2, 5760, 1440)])
def test_tile_weights_matches_oracle_and_inverts(shape):
    rng = np.random.default_rng(sum(shape))
    a = rng.integers(0, 256, size=shape, dtype=np.uint8)
    d = dev_u8(a)
    moe.moe_mxfp4_tile_weights(d)
    torch().cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), oracle.tile16(a))
    moe.moe_mxfp4_tile_weights(d, inverse=True)
    torch().cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), a)


# --------------------------------------------------------------------------
# MXFP4 encoder: bit-exact against the oracle under both rules
# --------------------------------------------------------------------------

def _encode_on_device(v, rule, bf16):
    t = torch()
    rows, cols = v.shape
    if bf16:
        bits = (np.ascontiguousarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        x = dev_bf16(bits)
        v = (bits.astype(np.uint32) << 16).view(np.float32)   # the values the device sees
    else:
        x = dev_f32(v)
    packed = t.empty((rows, cols // 2), dtype=t.uint8, device="cuda")
    scales = t.empty((rows, cols // 32), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_encode(x, packed, scales, rule=rule)
    t.cuda.synchronize()
    return v, packed, scales


@pytest.mark.parametrize("rule", ["ocp", "quark"])
@pytest.mark.parametrize("bf16", [False, True])
def test_encode_bit_exact(rule, bf16):
    rng = np.random.default_rng(31 + bf16)
    rows, cols = 300, 2880
    mag = np.exp2(rng.integers(-115, 115, size=(rows, 1))).astype(np.float32)       # 1e-35 .. 1e35 per row
    v = (rng.standard_normal((rows, cols)) * mag).astype(np.float32)
    v[0, :64] = 0.0                                                                # an all-zero block (and -0)
    v[0, 40] = -0.0
    v[1, :32] = np.float32(1e-40) * np.arange(32)                                  # subnormal block
    v[2, :8] = [7.0, -3.2, 0.26, 0.25, 0.75, -1.25, 2.5, 5.0]                       # the golden block
    v, packed, scales = _encode_on_device(v, rule, bf16)
    p_ref, s_ref = oracle.encode_mxfp4(v, rule)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    # and the device dequantises them back to the oracle's values
    out = torch().empty((rows, cols), dtype=torch().float32, device="cuda")
    moe.moe_mxfp4_dequant(packed, scales, out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.dequantize(p_ref, s_ref).view(np.uint32))


def test_encode_then_layer_matches_oracle():
    # weights quantised on the device from Gaussian values, then one layer call
    t = torch()
    cfg = _cfg(K=1024, I=512, E_global=4, E_local=4, top_k=2)
    rng = np.random.default_rng(33)
    w13 = (rng.standard_normal((4, 2 * 512, 1024)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((4, 1024, 512)) * 0.05).astype(np.float32)
    d13p = t.empty((4, 1024, 512), dtype=t.uint8, device="cuda")
    d13s = t.empty((4, 1024, 32), dtype=t.uint8, device="cuda")
    d2p = t.empty((4, 1024, 256), dtype=t.uint8, device="cuda")
    d2s = t.empty((4, 1024, 16), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_encode(dev_f32(w13), d13p, d13s)
    moe.moe_mxfp4_encode(dev_f32(w2), d2p, d2s)
    t.cuda.synchronize()
    p13, s13 = oracle.encode_mxfp4(w13)
    p2, s2 = oracle.encode_mxfp4(w2)
    assert np.array_equal(d13p.cpu().numpy(), p13) and np.array_equal(d13s.cpu().numpy(), s13)
    assert np.array_equal(d2p.cpu().numpy(), p2) and np.array_equal(d2s.cpu().numpy(), s2)
    w = make_weights(cfg)
    w.w13_packed, w.w13_scales, w.w2_packed, w.w2_scales = p13, s13, p2, s2
    inp = make_inputs(cfg, 6, t_index=1)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    _assert_close(bf16_to_np(run_decode(cfg, DeviceLayer(w), inp)), ref["y"], "encoded weights")


# --------------------------------------------------------------------------
# routing and bucketing: bit-exact ids and permutation
# --------------------------------------------------------------------------

ROUTE_CASES = [("tiny", 4), ("gptoss20b", 32), ("gptoss120b", 32), ("glm5_ep", 32), ("widek", 2048)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_topk(name, T):
    t = torch()
    cfg = get_config(name)
    inp = make_inputs(cfg, T)
    d = desc_for(cfg, T)
    ids = t.empty((T, cfg.top_k), dtype=t.int32, device="cuda")
    w = t.empty((T, cfg.top_k), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_route(d, dev_f32(inp.logits), ids, w)
    t.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk(inp.logits, cfg.top_k, cfg.scoring, dtype=np.float64)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.allclose(w.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)


# the router inside the plan kernel (T <= 64) and the one-wave-per-token router
# above it, read back from the plan with moe_mxfp4_plan_read: ids and the
# bucketing are bit-exact, weights within a few fp32 ulps
PLAN_ROUTE_CASES = [("tiny", 4), ("gptoss20b", 1), ("gptoss20b", 32), ("gptoss120b", 1), ("gptoss120b", 8),
                    ("gptoss120b", 32), ("glm5_ep", 1), ("glm5_ep", 32), ("widek", 32), ("gptoss120b", 64),
                    ("gptoss120b", 65), ("widek", 256)]


def _plan_read(cfg, T, d, ws):
    t = torch()
    k, E_l = cfg.top_k, cfg.E_local
    out = dict(ids=t.full((T, k), -7, dtype=t.int32, device="cuda"),
               w=t.full((T, k), float("nan"), dtype=t.float32, device="cuda"),
               counts=t.full((E_l,), -7, dtype=t.int32, device="cuda"),
               offsets=t.full((E_l + 1,), -7, dtype=t.int32, device="cuda"),
               routes=t.full((T * k,), -7, dtype=t.int32, device="cuda"))
    moe.moe_mxfp4_plan_read(d, ws, out["ids"], out["w"], out["counts"], out["offsets"], out["routes"])
    t.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in out.items()}


def _check_plan(cfg, logits, got, what):
    ids_ref, w_ref = oracle.route_topk(logits, cfg.top_k, cfg.scoring, dtype=np.float64)
    assert np.array_equal(got["ids"], ids_ref), what
    fin = np.isfinite(w_ref)
    assert np.array_equal(np.isnan(got["w"]), np.isnan(w_ref)), what
    assert np.allclose(got["w"][fin], w_ref[fin], rtol=2e-6, atol=1e-7), what
    c_ref, o_ref, r_ref = oracle.bucket_routes(ids_ref, cfg.E_local, cfg.expert_offset)
    assert np.array_equal(got["counts"], c_ref), what
    assert np.array_equal(got["offsets"], o_ref), what
    assert np.array_equal(got["routes"][:len(r_ref)], r_ref), what
    assert (got["routes"][len(r_ref):] == -1).all(), what


@pytest.mark.parametrize("name,T", PLAN_ROUTE_CASES)
def test_plan_router_bit_exact(name, T):
    t = torch()
    cfg = get_config(name)
    for variant, inp in (("random", make_inputs(cfg, T)), ("all-local", make_inputs(cfg, T, all_local_boost=8.0))):
        d = desc_for(cfg, T, weight_layout="tile16")
        ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
        moe.moe_mxfp4_plan(d, router_logits=dev_f32(inp.logits), workspace=ws)
        _check_plan(cfg, inp.logits, _plan_read(cfg, T, d, ws), f"{name} T={T} {variant}")
    # many ties: logits on a quarter grid, one row all equal
    rng = np.random.default_rng(T)
    logits = (np.round(rng.standard_normal((T, cfg.E_global)) * 4) / 4).astype(np.float32)
    logits[0] = 0.25
    d = desc_for(cfg, T)
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_plan(d, router_logits=dev_f32(logits), workspace=ws)
    _check_plan(cfg, logits, _plan_read(cfg, T, d, ws), f"{name} T={T} ties")


@pytest.mark.parametrize("T", [3, 40, 100])
def test_plan_router_nan_logits_rank_last(T):
    # finite logits are the layer's precondition; a NaN still gets the
    # oracle's place (below every number, ties to the lower id) in both routers
    t = torch()
    cfg = _cfg(E_global=96, E_local=96, top_k=6, scoring="softmax")
    rng = np.random.default_rng(40 + T)
    logits = (np.round(rng.standard_normal((T, 96)) * 4) / 4).astype(np.float32)
    logits[rng.random((T, 96)) < 0.3] = np.nan
    logits[1] = np.nan
    logits[2, :93] = np.nan
    d = desc_for(cfg, T)
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_plan(d, router_logits=dev_f32(logits), workspace=ws)
    _check_plan(cfg, logits, _plan_read(cfg, T, d, ws), f"NaN T={T} plan")
    ids = t.empty((T, 6), dtype=t.int32, device="cuda")
    w = t.empty((T, 6), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_route(d, dev_f32(logits), ids, w)
    t.cuda.synchronize()
    ids_ref, _ = oracle.route_topk(logits, 6, "softmax")
    assert np.array_equal(ids.cpu().numpy(), ids_ref)


def test_plan_read_in_ids_mode_returns_the_callers_routing():
    t = torch()
    cfg = _cfg(E_global=64, E_local=16, expert_offset=16, top_k=4)
    inp = make_topk_inputs(cfg, 20, seed=5, pad_fraction=0.2)
    d = desc_for(cfg, 20)
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_plan(d, topk_ids=dev_i32(inp.topk_ids), topk_weights=dev_f32(inp.topk_weights), workspace=ws)
    got = _plan_read(cfg, 20, d, ws)
    assert np.array_equal(got["ids"], inp.topk_ids)
    assert np.array_equal(got["w"], inp.topk_weights.astype(np.float32))
    c_ref, o_ref, r_ref = oracle.bucket_routes(inp.topk_ids, 16, 16)
    assert np.array_equal(got["counts"], c_ref) and np.array_equal(got["offsets"], o_ref)
    assert np.array_equal(got["routes"][:len(r_ref)], r_ref)


def test_steps_on_a_workspace_without_a_plan_write_nothing():
    # a workspace holding no plan of this descriptor (zeros, or a plan of
    # another shape): the expert kernels leave the outputs untouched instead
    # of following its entries
    t = torch()
    cfg = _cfg()
    w = make_weights(cfg)
    layer = DeviceLayer(w)
    inp = make_inputs(cfg, 4)
    d = desc_for(cfg, 4)
    ws = t.zeros(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    a = t.full((4 * cfg.top_k, cfg.I), 3.0, dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws, a=a)
    t.cuda.synchronize()
    assert bool((a == 3.0).all())
    d5 = desc_for(cfg, 5)
    ws5 = t.empty(moe.moe_mxfp4_workspace_bytes(d5), dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_plan(d5, router_logits=dev_f32(make_inputs(cfg, 5).logits), workspace=ws5)
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws5, a=a)
    t.cuda.synchronize()
    assert bool((a == 3.0).all())


def test_route_ties_break_to_lower_id():
    t = torch()
    cfg = _cfg(E_global=200, E_local=8, top_k=8, scoring="sigmoid")
    rng = np.random.default_rng(2)
    logits = (np.round(rng.standard_normal((64, 200)) * 2) / 2).astype(np.float32)  # many ties
    logits[0] = 1.0
    d = desc_for(cfg, 64)
    ids = t.empty((64, 8), dtype=t.int32, device="cuda")
    w = t.empty((64, 8), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_route(d, dev_f32(logits), ids, w)
    ids_ref, w_ref = oracle.route_topk(logits, 8, "sigmoid", dtype=np.float64)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert ids.cpu().numpy()[0].tolist() == list(range(8))
    assert np.allclose(w.cpu().numpy(), w_ref, rtol=2e-6)


BUCKET_CASES = [
    (8, 8, 0, 2, 4, 0.0), (32, 32, 0, 4, 1, 0.0), (128, 128, 0, 4, 32, 0.0), (256, 32, 64, 8, 32, 0.1),
    (384, 48, 336, 8, 2048, 0.05), (384, 48, 0, 8, 2047, 0.0), (512, 512, 0, 8, 300, 0.0), (16, 4, 12, 16, 3, 0.3),
    # up to 64 routes: the plan kernel's one-wave bucketing (512 experts: 9 id bits; one expert: 1 bit)
    (512, 512, 0, 8, 8, 0.0), (64, 16, 48, 4, 16, 0.2), (1, 1, 0, 1, 64, 0.0), (600, 512, 88, 2, 32, 0.1),
    # 65 - 128 routes: the general path just above the one-wave limit
    (32, 32, 0, 4, 32, 0.0), (8, 8, 0, 2, 33, 0.0), (512, 512, 0, 8, 16, 0.1), (64, 16, 48, 4, 20, 0.2),
    (1, 1, 0, 1, 100, 0.0), (256, 32, 0, 8, 12, 0.0), (4, 4, 0, 1, 65, 0.0),
    # 65 - 512 routes: one wave in 64-route chunks; 520: the general path again
    (64, 64, 0, 8, 64, 0.0), (384, 48, 336, 8, 64, 0.1), (600, 512, 88, 4, 128, 0.05), (64, 64, 0, 8, 65, 0.0),
    (256, 32, 0, 8, 40, 0.0), (2, 2, 0, 2, 200, 0.0),
]


@pytest.mark.parametrize("case", range(len(BUCKET_CASES)))
def test_bucket_permutation_bit_exact(case):
    t = torch()
    E_g, E_l, off, k, T, pad = BUCKET_CASES[case]
    cfg = _cfg(E_global=E_g, E_local=E_l, expert_offset=off, top_k=k)
    inp = make_topk_inputs(cfg, T, seed=100 + case, pad_fraction=pad)
    d = desc_for(cfg, T)
    counts = t.empty(E_l, dtype=t.int32, device="cuda")
    offsets = t.empty(E_l + 1, dtype=t.int32, device="cuda")
    routes = t.empty(T * k, dtype=t.int32, device="cuda")
    moe.moe_mxfp4_bucket(d, dev_i32(inp.topk_ids), counts, offsets, routes)
    t.cuda.synchronize()
    c_ref, o_ref, r_ref = oracle.bucket_routes(inp.topk_ids, E_l, off)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    r = routes.cpu().numpy()
    assert np.array_equal(r[:len(r_ref)], r_ref)
    assert (r[len(r_ref):] == -1).all()


def test_bucket_duplicate_ids_are_separate_routes():
    t = torch()
    cfg = _cfg(E_global=8, E_local=8, top_k=4)
    ids = np.array([[3, 3, 1, 3], [0, 7, 7, -1]], np.int32)
    d = desc_for(cfg, 2)
    counts = t.empty(8, dtype=t.int32, device="cuda")
    offsets = t.empty(9, dtype=t.int32, device="cuda")
    routes = t.empty(8, dtype=t.int32, device="cuda")
    moe.moe_mxfp4_bucket(d, dev_i32(ids), counts, offsets, routes)
    c_ref, o_ref, r_ref = oracle.bucket_routes(ids, 8, 0)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(routes.cpu().numpy()[:len(r_ref)], r_ref)


# --------------------------------------------------------------------------
# gate/up and down steps alone
# --------------------------------------------------------------------------

STEP_CASES = [
    dict(),                                                                    # tiny
    dict(K=2880, I=2880, E_global=32, E_local=4, expert_offset=8, top_k=4, activation="swiglu_oai",
         bias=True, scale_lo=115, scale_hi=127),                               # ragged 90-block rows
    dict(K=6144, I=2048, E_global=16, E_local=2, top_k=8, scoring="sigmoid", scale_lo=115, scale_hi=127),
    dict(K=96, I=160, E_global=3, E_local=3, top_k=2, bias=True, activation="swiglu_oai"),
    dict(K=1056, I=1120, E_global=6, E_local=6, top_k=3, bias=True, activation="swiglu_oai"),  # stream path
]


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
@pytest.mark.parametrize("T", [1, 5, 19])
def test_gate_up_step(case, T):
    t = torch()
    cfg = _cfg(**STEP_CASES[case])
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=T, x_scale=4.0 if case == 1 else 1.0)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    layer = DeviceLayer(w)
    d = desc_for(cfg, T)
    ws = moe.moe_mxfp4_plan(d, topk_ids=dev_i32(ref["ids"]), topk_weights=dev_f32(ref["weights"]))
    a = t.zeros((T * cfg.top_k, cfg.I), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws, a=a, w13_bias=layer.b13)
    t.cuda.synchronize()
    Rl = len(ref["routes"])
    got = bf16_to_np(a)[:Rl]
    _assert_close(got, ref["a"], f"a case{case} T{T}")
    if Rl:
        assert np.mean(got == ref["a"]) > 0.98   # bf16 values agree except rare rounding-boundary cases


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
@pytest.mark.parametrize("T", [1, 5, 19])
def test_down_step(case, T):
    t = torch()
    cfg = _cfg(**STEP_CASES[case])
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=T)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    layer = DeviceLayer(w)
    d = desc_for(cfg, T)
    R = T * cfg.top_k
    a_bits = np.zeros((R, cfg.I), np.uint16)
    a_bits[:len(ref["routes"])] = (ref["a"].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ws = moe.moe_mxfp4_plan(d, router_logits=dev_f32(inp.logits))
    out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_down(d, layer.w2p, layer.w2s, out, ws, a=dev_bf16(a_bits), w2_bias=layer.b2)
    t.cuda.synchronize()
    _assert_close(bf16_to_np(out), ref["y"], f"down case{case} T{T}")


def test_steps_compose_to_decode():
    t = torch()
    cfg = _cfg(**STEP_CASES[1])
    w = make_weights(cfg)
    inp = make_inputs(cfg, 6, t_index=3)
    layer = DeviceLayer(w)
    d = desc_for(cfg, 6)
    logits = dev_f32(inp.logits)
    ws = moe.moe_mxfp4_plan(d, router_logits=logits)
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws, w13_bias=layer.b13)
    out1 = t.empty((6, cfg.K), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_down(d, layer.w2p, layer.w2s, out1, ws, w2_bias=layer.b2)
    out2 = run_decode(cfg, layer, inp)
    assert np.array_equal(bf16_bits_np(out1), bf16_bits_np(out2))


# Calls of at most 128 routes and 32 tokens (more than 16 only with top_k <=
# 16 and at most 64 experts) whose two projections both run in the stream
# regime skip the plan kernel: the gate/up launch of
# moe_mxfp4_decode routes and buckets the call in every workgroup and its
# workgroup 0 writes the plan.  The layer output is bit-identical to the
# three steps (plan kernel, gate/up, down) and the plan left in the
# workspace is the plan kernel's, bit for bit.  _self_planned mirrors the
# library's rule so that every case below is known to take that path.
def _stream_fits(red, split):
    return split > 0 and (((red // 32) + 3) // 4 + split - 1) // split >= 4


def _self_planned(cfg, T):
    R = T * cfg.top_k
    if not (T <= 64 or (R < 65536 and R <= 16 * cfg.E_global)):
        return False
    split = 4 if T <= 4 else (2 if T <= 8 else 1)
    while split > 1 and not (_stream_fits(cfg.K, split) and _stream_fits(cfg.I, split)):
        split //= 2
    dsplit = split
    if 0 < split < 4 and T <= 32 and R <= 2 * cfg.E_global and _stream_fits(cfg.I, 4):
        dsplit = 4
    return (_stream_fits(cfg.K, split) and _stream_fits(cfg.I, dsplit) and T <= 32 and R <= 128
            and (T <= 16 or (cfg.top_k <= 16 and cfg.E_global <= 64)))


SELF_PLAN_CFGS = {
    "top4": dict(K=2048, I=2048, E_global=128, E_local=16, expert_offset=40, top_k=4, activation="swiglu_oai",
                 bias=True, scale_lo=115, scale_hi=127),
    "top8-sigmoid": dict(K=2048, I=1024, E_global=256, E_local=32, expert_offset=96, top_k=8, scoring="sigmoid",
                         scale_lo=115, scale_hi=127),
    "all-experts": dict(K=1024, I=2048, E_global=24, E_local=24, top_k=4, bias=True),
    # 384 experts: above 256 a token's top-k takes a whole wave, also at T > 4
    "wide-e": dict(K=1024, I=1024, E_global=384, E_local=48, expert_offset=96, top_k=8, scoring="sigmoid"),
    # 512 local experts: the largest chunked-bucketing arrays in the launch's LDS
    "e512": dict(K=512, I=512, E_global=512, E_local=512, top_k=8, scoring="sigmoid"),
    "top4-e64": dict(K=2048, I=2048, E_global=64, E_local=16, expert_offset=40, top_k=4, activation="swiglu_oai",
                     bias=True, scale_lo=115, scale_hi=127),
}
SELF_PLAN_CASES = [("top4", 1, "random"), ("top4", 1, "all-local"), ("top4", 4, "random"), ("top4", 4, "all-local"),
                   ("top4", 8, "all-local"), ("top4", 16, "random"), ("top4", 16, "all-local"),
                   ("top4", 5, "ties"), ("top8-sigmoid", 2, "all-local"), ("top8-sigmoid", 8, "random"),
                   ("top8-sigmoid", 8, "all-local"), ("all-experts", 16, "random"), ("all-experts", 3, "ids"),
                   ("top4", 12, "ids"), ("wide-e", 8, "random"), ("wide-e", 8, "all-local"),
                   # 65 - 128 routes: the chunked bucketing inside the gate/up launch
                   ("top4-e64", 20, "random"), ("top4-e64", 32, "random"), ("top4-e64", 32, "all-local"),
                   ("top4-e64", 32, "ties"), ("top4-e64", 28, "ids"), ("top8-sigmoid", 16, "random"),
                   ("top8-sigmoid", 16, "all-local"),
                   ("all-experts", 32, "random"), ("e512", 16, "random")]


@pytest.mark.parametrize("name,T,variant", SELF_PLAN_CASES)
def test_self_planned_decode_matches_the_steps(name, T, variant):
    t = torch()
    cfg = _cfg(**SELF_PLAN_CFGS[name])
    assert _self_planned(cfg, T), (name, T)
    w = make_weights(cfg)
    layer = DeviceLayer(w, layout="tile16")
    if variant == "ids":
        inp = make_topk_inputs(cfg, T, seed=T, pad_fraction=0.2)
    elif variant == "ties":
        inp = make_inputs(cfg, T, t_index=T)
        rng = np.random.default_rng(T)
        logits = (np.round(rng.standard_normal((T, cfg.E_global)) * 2) / 2).astype(np.float32)
        logits[0] = 0.5
        logits[1, cfg.expert_offset:cfg.expert_offset + 8] = 9.0
        inp = LayerInputs(x=inp.x, logits=logits)
    else:
        inp = make_inputs(cfg, T, t_index=T, all_local_boost=30.0 if variant == "all-local" else 0.0)
    d = desc_for(cfg, T, weight_layout="tile16")
    nbytes = moe.moe_mxfp4_workspace_bytes(d)
    ws1 = t.full((nbytes,), 0x5A, dtype=t.uint8, device="cuda")
    out1 = run_decode(cfg, layer, inp, workspace=ws1)
    if inp.logits is not None:
        route = dict(router_logits=dev_f32(inp.logits))
    else:
        route = dict(topk_ids=dev_i32(inp.topk_ids), topk_weights=dev_f32(inp.topk_weights))
    ws2 = t.full((nbytes,), 0xA5, dtype=t.uint8, device="cuda")
    moe.moe_mxfp4_plan(d, workspace=ws2, **route)
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws2, w13_bias=layer.b13)
    out2 = t.empty((T, cfg.K), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_down(d, layer.w2p, layer.w2s, out2, ws2, w2_bias=layer.b2)
    t.cuda.synchronize()
    what = f"{name} T={T} {variant}"
    assert np.array_equal(bf16_bits_np(out1), bf16_bits_np(out2)), what
    p1, p2 = _plan_read(cfg, T, d, ws1), _plan_read(cfg, T, d, ws2)
    for k in ("ids", "counts", "offsets", "routes"):
        assert np.array_equal(p1[k], p2[k]), (what, k)
    assert np.array_equal(p1["w"].view(np.uint32), p2["w"].view(np.uint32)), what
    if inp.logits is not None:
        _check_plan(cfg, inp.logits, p1, what)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    _assert_close(bf16_to_np(out1), ref["y"], what)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

LAYER_CASES = [
    ("tiny", dict(), 4, 1.0),
    ("tiny", dict(), 1, 4.0),
    ("swiglu-slice", dict(K=2880, I=2880, E_global=32, E_local=6, expert_offset=20, top_k=4,
                          activation="swiglu_oai", bias=True, scale_lo=115, scale_hi=127), 7, 4.0),
    ("sigmoid-slice", dict(K=6144, I=2048, E_global=64, E_local=4, expert_offset=4, top_k=8,
                           scoring="sigmoid", scale_lo=115, scale_hi=127), 9, 1.0),
    ("many-tokens-per-expert", dict(K=512, I=768, E_global=2, E_local=2, top_k=2), 37, 1.0),
    ("odd-blocks", dict(K=96, I=224, E_global=5, E_local=5, top_k=3, activation="swiglu_oai", bias=True), 11, 1.0),
    ("two-mfma-passes", dict(K=256, I=128, E_global=1, E_local=1, top_k=1), 100, 1.0),
    ("wide-k-mixed-regimes", dict(K=7168, I=2048, E_global=16, E_local=3, expert_offset=2, top_k=4,
                                  scoring="sigmoid", scale_lo=115, scale_hi=127), 12, 1.0),
    # decode-regime stream kernel: reduction split 4 ways (T <= 4), 2 ways (T <= 8), none (T <= 64)
    ("stream-split4-ring-exact", dict(K=2048, I=2048, E_global=8, E_local=8, top_k=2, activation="swiglu_oai",
                                      bias=True, scale_lo=115, scale_hi=127), 3, 1.0),
    ("stream-split4-ragged", dict(K=2080, I=2080, E_global=6, E_local=6, top_k=3, bias=True), 4, 1.0),
    ("stream-split2", dict(K=1056, I=1120, E_global=4, E_local=4, top_k=2, bias=True,
                           activation="swiglu_oai"), 7, 1.0),
    ("stream-partial-tile", dict(K=544, I=608, E_global=4, E_local=4, top_k=2), 20, 1.0),
    ("stream-multi-pass", dict(K=640, I=512, E_global=2, E_local=2, top_k=2, bias=True), 64, 1.0),
    ("stream-split-lowered", dict(K=512, I=1024, E_global=4, E_local=4, top_k=2), 2, 1.0),
    ("stream-gate-up-only", dict(K=2048, I=256, E_global=4, E_local=4, top_k=2, bias=True), 3, 1.0),
    ("stream-slice-sigmoid", dict(K=6144, I=2048, E_global=64, E_local=8, expert_offset=16, top_k=8,
                                  scoring="sigmoid", scale_lo=115, scale_hi=127), 32, 1.0),
    # T > 64 with few routes per expert (T * top_k <= 16 * E_global): still the stream kernel,
    # routing in its own kernel, passes of 16 routes, an expert with several passes
    ("stream-regime-large-T", dict(K=512, I=768, E_global=64, E_local=16, expert_offset=8, top_k=2, bias=True,
                                   activation="swiglu_oai"), 200, 1.0),
    ("stream-regime-large-T-sigmoid", dict(K=1024, I=512, E_global=32, E_local=32, top_k=4, scoring="sigmoid"),
     128, 1.0),
    # 8 < T <= 32 with the down projection split 2 ways (its own pass list,
    # 8 routes per pass) under a gate/up split of 1, which needs T * top_k <=
    # 2 * E_global; logits boosted on the slice make every route local, so
    # each expert's routes span several down passes.  768 routes take the
    # plan's general bucketing path (24 routes per expert, 3 down passes)
    ("stream-down-split2-general-plan", dict(K=512, I=2048, E_global=384, E_local=32, top_k=24, bias=True), 32,
     1.0, 30.0),
    # the same split pair with the one-wave (64 routes) and chunked (256 routes) plans
    ("stream-down-split2-one-wave-plan", dict(K=1024, I=2048, E_global=32, E_local=8, expert_offset=8, top_k=4),
     16, 1.0, 30.0),
    ("stream-down-split2-chunked-plan", dict(K=1024, I=2048, E_global=128, E_local=12, expert_offset=4, top_k=8,
                                             scoring="sigmoid"), 32, 1.0, 30.0),
    # 4 < T <= 8: the down projection split 4 ways (4 routes per pass) under a
    # gate/up split of 2 (8 routes per pass); 8 local routes per expert, so
    # every expert has two down passes and one gate/up pass
    ("stream-down-split4-under-split2", dict(K=1024, I=2048, E_global=64, E_local=8, expert_offset=8, top_k=8,
                                             scoring="sigmoid"), 8, 1.0, 30.0),
]


@pytest.mark.parametrize("case", range(len(LAYER_CASES)))
def test_layer_elementwise(case):
    name, kw, T, xs, *boost = LAYER_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=case, x_scale=xs, all_local_boost=boost[0] if boost else 0.0)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    out = run_decode(cfg, DeviceLayer(w), inp)
    _assert_close(bf16_to_np(out), ref["y"], f"layer {name} T{T}")


TILED_CASES = [
    ("split4", dict(K=2880, I=2880, E_global=32, E_local=6, expert_offset=20, top_k=4, activation="swiglu_oai",
                    bias=True, scale_lo=115, scale_hi=127), 1),
    ("split2", dict(K=1056, I=1120, E_global=4, E_local=4, top_k=2, bias=True), 7),
    ("split1", dict(K=544, I=608, E_global=4, E_local=4, top_k=2), 20),
    ("fallback-lists", dict(), 4),                                         # K = I = 256: GEMV / MFMA list kernels
    ("large-T-lists", dict(K=512, I=768, E_global=2, E_local=2, top_k=2), 80),
    ("gate-up-only", dict(K=2048, I=256, E_global=4, E_local=4, top_k=2, bias=True), 3),
]


@pytest.mark.parametrize("case", range(len(TILED_CASES)))
def test_layer_tiled_weights_bit_identical_to_rows(case):
    name, kw, T = TILED_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=case)
    rows = bf16_bits_np(run_decode(cfg, DeviceLayer(w), inp))
    tiled = bf16_bits_np(run_decode(cfg, DeviceLayer(w, layout="tile16"), inp))
    assert np.array_equal(rows, tiled), name
    if case == 0:
        ref = oracle.moe_forward_cfg(cfg, w, inp)
        _assert_close(bf16_to_np(run_decode(cfg, DeviceLayer(w, layout="tile16"), inp)), ref["y"], "tiled")


# paired down rows (two 16-row sets per wave) against unpaired: same MFMA
# sequence and reduction order per output row, so bit-identical
PAIRING_CASES = [
    ("split4", dict(K=2080, I=2048, E_global=8, E_local=6, expert_offset=1, top_k=2, activation="swiglu_oai",
                    bias=True, scale_lo=115, scale_hi=127), 2, "rows"),
    ("split4-tiled", dict(K=2080, I=2048, E_global=8, E_local=6, expert_offset=1, top_k=2, activation="swiglu_oai",
                          bias=True, scale_lo=115, scale_hi=127), 3, "tile16"),
    ("split2", dict(K=1120, I=1056, E_global=4, E_local=4, top_k=2, bias=True), 7, "tile16"),
    ("split1", dict(K=544, I=608, E_global=4, E_local=4, top_k=2), 20, "rows"),
    ("split1-multipass", dict(K=640, I=512, E_global=2, E_local=2, top_k=2, bias=True), 40, "tile16"),
    # many routes per expert: the MFMA list kernel, 128-row paired down tiles
    ("mfma-lists", dict(K=512, I=768, E_global=2, E_local=2, top_k=2, bias=True), 80, "tile16"),
    ("mfma-lists-ragged-tile", dict(K=416, I=544, E_global=3, E_local=3, top_k=2, activation="swiglu_oai",
                                    bias=True), 150, "rows"),
]


@pytest.mark.parametrize("case", range(len(PAIRING_CASES)))
def test_down_pairing_bit_identical_and_matches_oracle(case):
    name, kw, T, layout = PAIRING_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=case)
    layer = DeviceLayer(w, layout=layout)
    off = bf16_bits_np(run_decode(cfg, layer, inp, down_pairing="off"))
    on = bf16_bits_np(run_decode(cfg, layer, inp, down_pairing="on"))
    assert np.array_equal(off, on), name
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    _assert_close(bf16_to_np(run_decode(cfg, layer, inp, down_pairing="on")), ref["y"], name)


# interleaved gate/up rows: the same per-row arithmetic as [gate; up], so the
# output is bit-identical to the [gate; up] storage of the same weights
def _interleaved_weights(w, I):
    def il(a):
        out = np.empty_like(a)
        out[:, 0::2] = a[:, :I]
        out[:, 1::2] = a[:, I:]
        return out
    return LayerWeights(w13_packed=il(w.w13_packed), w13_scales=il(w.w13_scales), w2_packed=w.w2_packed,
                        w2_scales=w.w2_scales, b13=None if w.b13 is None else il(w.b13), b2=w.b2)


INTERLEAVED_CASES = [
    ("stream-split4", dict(K=2080, I=2048, E_global=8, E_local=6, expert_offset=1, top_k=2,
                           activation="swiglu_oai", bias=True, scale_lo=115, scale_hi=127), 2, "rows"),
    ("stream-split4-tiled", dict(K=2080, I=2048, E_global=8, E_local=6, expert_offset=1, top_k=2,
                                 activation="swiglu_oai", bias=True, scale_lo=115, scale_hi=127), 3, "tile16"),
    ("stream-split2-tiled", dict(K=1120, I=1056, E_global=4, E_local=4, top_k=2, bias=True), 7, "tile16"),
    ("stream-split1", dict(K=544, I=608, E_global=4, E_local=4, top_k=2), 20, "rows"),
    ("gemv-lists", dict(bias=True, activation="swiglu_oai", scale_lo=115, scale_hi=127), 4, "rows"),
    ("mfma-lists-tiled", dict(K=512, I=768, E_global=2, E_local=2, top_k=2, bias=True), 80, "tile16"),
]


@pytest.mark.parametrize("case", range(len(INTERLEAVED_CASES)))
def test_interleaved_rows_bit_identical_and_match_oracle(case):
    name, kw, T, layout = INTERLEAVED_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    wi = _interleaved_weights(w, cfg.I)
    inp = make_inputs(cfg, T, t_index=case)
    blocked = bf16_bits_np(run_decode(cfg, DeviceLayer(w, layout=layout), inp))
    y = run_decode(cfg, DeviceLayer(wi, layout=layout), inp, w13_order="interleaved")
    assert np.array_equal(bf16_bits_np(y), blocked), name
    ref = oracle.moe_forward_cfg(cfg, wi, inp, w13_order="interleaved")
    _assert_close(bf16_to_np(y), ref["y"], name)


# per-route output: W2 a_r + b2 of each local route, zeros elsewhere
ROUTE_OUT_CASES = [
    ("stream-slice", dict(K=1120, I=1056, E_global=8, E_local=4, expert_offset=2, top_k=2, bias=True), 6, "tile16"),
    ("stream-split1", dict(K=544, I=608, E_global=6, E_local=4, expert_offset=1, top_k=2, activation="swiglu_oai", bias=True,
                           scale_lo=115, scale_hi=127), 20, "rows"),
    ("gemv-lists-slice", dict(E_global=8, E_local=5, expert_offset=3), 4, "rows"),
    ("mfma-lists-slice", dict(K=512, I=768, E_global=4, E_local=2, expert_offset=1, top_k=2, bias=True), 80,
     "tile16"),
]


@pytest.mark.parametrize("case", range(len(ROUTE_OUT_CASES)))
def test_route_outputs_match_oracle(case):
    t = torch()
    name, kw, T, layout = ROUTE_OUT_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=case)
    layer = DeviceLayer(w, layout=layout)
    d = desc_for(cfg, T, weight_layout=layout)
    R = T * cfg.top_k
    x, lg = dev_bf16(inp.x), dev_f32(inp.logits)
    rows = t.full((R, cfg.K), float("nan"), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_decode_routes(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, rows, router_logits=lg,
                                w13_bias=layer.b13, w2_bias=layer.b2)
    t.cuda.synchronize()
    got = rows.cpu().numpy()
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    want = oracle.route_outputs(ref, T, cfg.top_k)
    local = np.zeros(R, bool)
    local[ref["routes"]] = True
    assert (~local).any() and local.any(), name
    assert np.array_equal(got[~local], np.zeros_like(got[~local])), name
    _assert_close(got[local], want[local], name)
    # the steps one by one give the same bits
    ws = moe.moe_mxfp4_plan(d, router_logits=lg)
    moe.moe_mxfp4_gate_up(d, x, layer.w13p, layer.w13s, ws, w13_bias=layer.b13)
    rows2 = t.full((R, cfg.K), float("nan"), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_down_routes(d, layer.w2p, layer.w2s, rows2, ws, w2_bias=layer.b2)
    t.cuda.synchronize()
    assert np.array_equal(rows2.cpu().numpy(), got), name
    # the routing-weighted sum of the rows is the layer output
    y = bf16_to_np(run_decode(cfg, layer, inp)).astype(np.float64)
    ysum = np.einsum("tj,tjk->tk", ref["weights"].astype(np.float64), got.reshape(T, cfg.top_k, cfg.K))
    assert oracle.rel_l2(y, ysum) <= 3e-3, name


# One-token calls with top_k <= 4 take one launch for the down projection
# and the token sum (token_down_kernel); calls of 2 - 4 tokens run the stream
# kernel and the combine.  Either way, against the per-route rows of the same
# call (the stream kernel's 4-way split, routes of one expert side by side in
# its MFMA columns) summed here with the combine's fp32 arithmetic (route
# order, product then sum, one rounding each, bf16 at the end): the same
# bits; and against the oracle within the bar.
TOKEN_CASES = [
    ("gpt-oss-slice", dict(K=2880, I=2880, E_global=16, E_local=6, expert_offset=4, top_k=4,
                           activation="swiglu_oai", bias=True, scale_lo=115, scale_hi=127), 1, "tile16", "logits", 0.0),
    ("gpt-oss-all-local", dict(K=2880, I=2880, E_global=8, E_local=8, top_k=4, activation="swiglu_oai", bias=True,
                               scale_lo=115, scale_hi=127), 1, "rows", "logits", 0.0),
    ("gpt-oss-4-tokens-shared-experts", dict(K=2880, I=2880, E_global=8, E_local=8, top_k=4,
                                             activation="swiglu_oai", bias=True, scale_lo=115, scale_hi=127), 4,
     "tile16", "logits", 0.0),
    ("top2-short-K", dict(K=1056, I=2048, E_global=8, E_local=8, top_k=2), 3, "tile16", "logits", 0.0),
    ("top3-ragged-I", dict(K=1024, I=2080, E_global=12, E_local=3, expert_offset=5, top_k=3, bias=True), 2, "rows",
     "logits", 30.0),
    ("ids-padding-foreign", dict(K=2048, I=2048, E_global=16, E_local=4, expert_offset=6, top_k=4, bias=True), 4,
     "tile16", "ids", 0.0),
    ("ids-no-local-route", dict(K=2048, I=2048, E_global=16, E_local=2, expert_offset=14, top_k=4), 1, "rows", "ids",
     0.0),
]


@pytest.mark.parametrize("case", range(len(TOKEN_CASES)))
def test_few_token_call_bit_identical_to_route_rows(case):
    t = torch()
    name, kw, T, layout, mode, boost = TOKEN_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    layer = DeviceLayer(w, layout=layout)
    d = desc_for(cfg, T, weight_layout=layout)
    k = cfg.top_k
    if mode == "logits":
        inp = make_inputs(cfg, T, t_index=case, all_local_boost=boost)
        route = dict(router_logits=dev_f32(inp.logits))
    else:
        inp = make_topk_inputs(cfg, T, seed=40 + case, pad_fraction=0.25)
        if name == "ids-no-local-route":
            inp.topk_ids[:] = np.array([0, 3, -1, 7], np.int32)   # all outside experts 14..15
        route = dict(topk_ids=dev_i32(inp.topk_ids), topk_weights=dev_f32(inp.topk_weights))
    x = dev_bf16(inp.x)
    y = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    moe.moe_mxfp4_decode(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, y, w13_bias=layer.b13,
                         w2_bias=layer.b2, **route)
    rows = t.full((T * k, cfg.K), float("nan"), dtype=t.float32, device="cuda")
    moe.moe_mxfp4_decode_routes(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, rows, w13_bias=layer.b13,
                                w2_bias=layer.b2, **route)
    ws = moe.moe_mxfp4_plan(d, **route)
    plan = _plan_read(cfg, T, d, ws)
    t.cuda.synchronize()
    local = set(int(r) for r in plan["routes"] if r >= 0)
    o = rows.cpu().numpy()
    acc = np.zeros((T, cfg.K), np.float32)
    for tt in range(T):
        for j in range(k):
            if tt * k + j in local:
                prod = (np.float32(plan["w"][tt, j]) * o[tt * k + j]).astype(np.float32)
                acc[tt] = (acc[tt] + prod).astype(np.float32)
    want = bf16_bits_np(t.from_numpy(acc).to(t.bfloat16))
    got = bf16_bits_np(y)
    assert np.array_equal(got, want), f"{name}: {np.count_nonzero(got != want)} of {got.size} outputs differ"
    if name == "ids-no-local-route":
        assert not local and not np.any(got)
    if name.startswith("gpt-oss-4-tokens"):
        experts = plan["ids"][plan["ids"] >= 0].ravel()
        assert len(set(experts.tolist())) < experts.size, "some expert should serve several routes"
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    _assert_close(bf16_to_np(y), ref["y"], name)


# Calls from two host threads at once, each on its own stream and workspace,
# give the bits of the same calls made one after the other.
def test_concurrent_calls_from_two_threads():
    import threading
    t = torch()
    cfg = _cfg(K=2880, I=2880, E_global=32, E_local=32, top_k=4, activation="swiglu_oai", bias=True,
               scale_lo=115, scale_hi=127)
    w = make_weights(cfg)
    layer = DeviceLayer(w, layout="tile16")
    cases = [(T, make_inputs(cfg, T, t_index=T)) for T in (1, 4, 16, 32)]
    want = {T: bf16_bits_np(run_decode(cfg, layer, inp)) for T, inp in cases}
    got, errors = {}, []

    def worker(sub):
        try:
            s = t.cuda.Stream()
            for T, inp in sub:
                d = desc_for(cfg, T, weight_layout="tile16")
                x, lg = dev_bf16(inp.x), dev_f32(inp.logits)
                out = t.empty((T, cfg.K), dtype=t.bfloat16, device="cuda")
                for _ in range(3):
                    moe.moe_mxfp4_decode(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, out, router_logits=lg,
                                         w13_bias=layer.b13, w2_bias=layer.b2, stream=s)
                s.synchronize()
                got[T] = bf16_bits_np(out)
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(cases[i::2],)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for T, _ in cases:
        assert np.array_equal(got[T], want[T]), T


# A decode call captured in a HIP graph: every replay, with eager calls on
# other inputs in between, gives the eager result's bits (stream kernels at
# reduction splits 4 / 2 / 1, and the GEMV/MFMA list path).
@pytest.mark.parametrize("T", [1, 8, 32, 100])
def test_graph_capture_replays_match_eager(T):
    t = torch()
    cfg = _cfg(K=1024, I=1024, E_global=16, E_local=16, top_k=4, activation="swiglu_oai", bias=True,
               scale_lo=115, scale_hi=127)
    w = make_weights(cfg)
    layer = DeviceLayer(w, layout="tile16")
    inp = make_inputs(cfg, T, t_index=T)
    other = make_inputs(cfg, T, t_index=T + 1)
    want = bf16_bits_np(run_decode(cfg, layer, inp))
    d = desc_for(cfg, T, weight_layout="tile16")
    x, lg = dev_bf16(inp.x), dev_f32(inp.logits)
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(d), dtype=t.uint8, device="cuda")
    out = t.empty((T, cfg.K), dtype=t.bfloat16, device="cuda")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        moe.moe_mxfp4_decode(d, x, layer.w13p, layer.w13s, layer.w2p, layer.w2s, out, router_logits=lg,
                             w13_bias=layer.b13, w2_bias=layer.b2, workspace=ws, stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(bf16_bits_np(out), want), (T, rep)
        run_decode(cfg, layer, other)  # eager work on other inputs between replays


# prefill path: unpack the touched experts to bf16, then bf16 MFMA GEMMs
@pytest.mark.parametrize("layout", ["rows", "tile16"])
def test_unpack_touched_experts_bit_exact(layout):
    t = torch()
    cfg = _cfg(K=544, I=320, E_global=8, E_local=6, expert_offset=1, top_k=2)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 3, seed=5)
    d = desc_for(cfg, 3, weight_layout=layout)
    layer = DeviceLayer(w, layout=layout)
    ws = moe.moe_mxfp4_plan(d, topk_ids=dev_i32(inp.topk_ids), topk_weights=dev_f32(inp.topk_weights))
    sentinel = 0x7FBF                                   # a NaN pattern the unpack never writes
    w13o = t.full((cfg.E_local, 2 * cfg.I, cfg.K), 0, dtype=t.int16, device="cuda")
    w2o = t.full((cfg.E_local, cfg.K, cfg.I), 0, dtype=t.int16, device="cuda")
    w13o.fill_(sentinel)
    w2o.fill_(sentinel)
    moe.moe_mxfp4_unpack(d, layer.w13p, layer.w13s, layer.w2p, layer.w2s, w13o.view(t.bfloat16),
                         w2o.view(t.bfloat16), ws)
    t.cuda.synchronize()
    g13 = w13o.cpu().numpy().view(np.uint16)
    g2 = w2o.cpu().numpy().view(np.uint16)
    ids = inp.topk_ids.ravel()
    touched = {int(i) - cfg.expert_offset for i in ids if cfg.expert_offset <= i < cfg.expert_offset + cfg.E_local}
    assert 0 < len(touched) < cfg.E_local
    for e in range(cfg.E_local):
        if e in touched:
            assert np.array_equal(g13[e], oracle.unpack_bf16(w.w13_packed[e], w.w13_scales[e])), e
            assert np.array_equal(g2[e], oracle.unpack_bf16(w.w2_packed[e], w.w2_scales[e])), e
        else:
            assert (g13[e] == sentinel).all() and (g2[e] == sentinel).all(), e


def _run_prefill(cfg, layer, inp, w13_order="gate_up"):
    t = torch()
    T = inp.x.shape[0]
    d = desc_for(cfg, T, E_local=layer.E_local, weight_layout=layer.layout, w13_order=w13_order)
    out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
    kw = {"router_logits": dev_f32(inp.logits)} if inp.logits is not None else {
        "topk_ids": dev_i32(inp.topk_ids), "topk_weights": dev_f32(inp.topk_weights)}
    moe.moe_mxfp4_prefill(d, dev_bf16(inp.x), layer.w13p, layer.w13s, layer.w2p, layer.w2s, out,
                          w13_bias=layer.b13, w2_bias=layer.b2, **kw)
    t.cuda.synchronize()
    return out


PREFILL_CASES = [
    # (name, config, T, layout, w13 order, decode takes the MFMA path for every touched expert)
    ("mfma-both", dict(K=1024, I=512, E_global=16, E_local=8, expert_offset=4, top_k=4, scoring="sigmoid"),
     96, "rows", "gate_up", True),
    ("mfma-both-tiled-il", dict(K=768, I=1056, E_global=4, E_local=4, top_k=2, activation="swiglu_oai", bias=True,
                                scale_lo=115, scale_hi=127), 80, "tile16", "interleaved", True),
    ("groups4-ragged", dict(K=544, I=608, E_global=2, E_local=2, top_k=2, bias=True), 300, "rows", "gate_up", True),
    ("small-T", dict(K=1120, I=1056, E_global=8, E_local=4, expert_offset=2, top_k=2, bias=True), 6, "tile16",
     "gate_up", False),
    ("tiny", dict(), 4, "rows", "gate_up", False),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_matches_oracle_and_decode(case):
    name, kw, T, layout, order, same_path = PREFILL_CASES[case]
    cfg = _cfg(**kw)
    w = make_weights(cfg)
    if order == "interleaved":
        w = _interleaved_weights(w, cfg.I)
    inp = make_inputs(cfg, T, t_index=case)
    layer = DeviceLayer(w, layout=layout)
    y = _run_prefill(cfg, layer, inp, order)
    ref = oracle.moe_forward_cfg(cfg, w, inp, w13_order=order)
    _assert_close(bf16_to_np(y), ref["y"], name)
    if same_path:
        assert int(ref["counts"][ref["counts"] > 0].min()) > 2, name   # decode's MFMA regime for every expert
        yd = run_decode(cfg, layer, inp, w13_order=order)
        assert np.array_equal(bf16_bits_np(y), bf16_bits_np(yd)), name


def test_layer_ids_mode_with_padding_and_foreign_ids():
    cfg = _cfg(K=2880, I=2880, E_global=32, E_local=5, expert_offset=3, top_k=4, activation="swiglu_oai",
               bias=True, scale_lo=115, scale_hi=127)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 12, seed=7, pad_fraction=0.2)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    _assert_close(y, ref["y"], "ids mode")
    no_route = ~np.any((inp.topk_ids >= 3) & (inp.topk_ids < 8), axis=1)
    assert not y[no_route].any()


def test_layer_duplicate_ids_more_routes_than_tokens():
    # ids mode lets one token route to an expert several times: expert 1 gets
    # 3 * 7 routes from 3 tokens (several passes), each weighted on its own
    cfg = _cfg(K=1024, I=1024, E_global=8, E_local=4, top_k=8, bias=True)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 3, seed=11)
    inp.topk_ids[:] = np.array([1, 1, 1, 1, 1, 1, 1, 3], np.int32)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    _assert_close(y, ref["y"], "duplicate ids")


# Routes per expert for the list path (T > 64, or a reduction too short for
# the stream kernel): passes of every column-group count in one launch.
GROUP_COUNT_CASES = [
    # T = 100, 4 groups of 16 tokens per pass: 2 routes (in the MFMA list too:
    # 25 routes per expert expected leave the GEMV list out), 18, 40, 55, 75
    # (a full 64-route pass, then 11) and 10 give passes of 2, 3, 4 and 1
    # groups; I = 384 and K = 512 leave ragged row tiles in both projections
    (100, 512, 384, [2, 18, 40, 55, 75, 10, 0, 0]),
    # T = 40 with K = I = 256 (too short for the stream kernel), 2 groups per
    # pass: 1 route (GEMV), then 5 (1 group), 20, 30 and 24 (2 groups)
    (40, 256, 256, [1, 5, 20, 30, 24, 0, 0, 0]),
]


@pytest.mark.parametrize("case", range(len(GROUP_COUNT_CASES)))
def test_mfma_lists_every_column_group_count(case):
    T, K, I, counts = GROUP_COUNT_CASES[case]
    cfg = _cfg(K=K, I=I, bias=True)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, T, seed=17 + case)
    slots = np.repeat(np.arange(8, dtype=np.int32), counts)
    ids = np.stack([slots[:T], slots[T:]], axis=1)
    assert (ids[:, 0] != ids[:, 1]).all()
    inp.topk_ids[:] = ids
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    _assert_close(y, ref["y"], f"column group counts T={T}")


# The scaled-FP4 MFMA path (MOE_MMA_SCALED_FP4) on list-path calls (T > 64
# with many routes per expert, or a reduction too short for the stream
# kernel, so that the MFMA lists run): passes of
# every column-group count, a reduction with a partial last 128-value chunk
# (K = 96, I = 224: the split rows are zero-filled past the row), RMS-4
# activations, tiled weights with the down pairing on and off, and the
# SwiGLU-OAI clamp with biases.  Same bar as the bf16 path.
SCALED_CASES = [
    ("group-counts-100", None, 0, "rows", "auto", 1.0),
    ("group-counts-40", None, 1, "rows", "auto", 1.0),
    ("partial-chunks", dict(K=96, I=224, E_global=5, E_local=5, top_k=3, activation="swiglu_oai", bias=True), 40,
     "rows", "auto", 1.0),
    ("many-tokens-per-expert-rms4", dict(K=512, I=768, E_global=2, E_local=2, top_k=2), 100, "rows", "auto", 4.0),
    ("two-passes-tiled-paired", dict(K=256, I=128, E_global=1, E_local=1, top_k=1), 100, "tile16", "on", 1.0),
    ("large-T-tiled-unpaired", dict(K=512, I=768, E_global=4, E_local=4, top_k=2, bias=True,
                                    activation="swiglu_oai"), 80, "tile16", "off", 1.0),
    ("wide-k-slice", dict(K=7168, I=2048, E_global=16, E_local=3, expert_offset=2, top_k=4, scoring="sigmoid",
                          scale_lo=115, scale_hi=127), 96, "tile16", "auto", 1.0),
]


@pytest.mark.parametrize("case", range(len(SCALED_CASES)))
def test_scaled_fp4_list_path_matches_oracle(case):
    name, kw, T, layout, pairing, xs = SCALED_CASES[case]
    if kw is None:  # forced routing of the column-group cases
        T, K, I, counts = GROUP_COUNT_CASES[T]
        cfg = _cfg(K=K, I=I, bias=True)
        w = make_weights(cfg)
        inp = make_topk_inputs(cfg, T, seed=31 + case)
        slots = np.repeat(np.arange(8, dtype=np.int32), counts)
        inp.topk_ids[:] = np.stack([slots[:T], slots[T:]], axis=1)
    else:
        cfg = _cfg(**kw)
        w = make_weights(cfg)
        inp = make_inputs(cfg, T, t_index=case, x_scale=xs)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w, layout=layout), inp, down_pairing=pairing, mma="scaled_fp4"))
    _assert_close(y, ref["y"], f"scaled-FP4 list path {name} T={T}", elementwise=False)


def test_list_path_top1_just_above_one_wave_plan():
    # T = 100, top-1 over 4 experts: 100 routes (just above the plan kernel's
    # one-wave bucketing, in its 64-route chunked path) and more than 16 per
    # expert, so the MFMA lists take them
    cfg = _cfg(K=512, I=512, E_global=4, E_local=4, top_k=1, bias=True)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 100, seed=23)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    _assert_close(y, ref["y"], "top-1 list call just above the one-wave plan")


@pytest.mark.parametrize("T", [3, 100])
def test_layer_at_maximum_dimensions(T):
    # K = I = 8192 (the largest the descriptor accepts), 2 experts, top-1:
    # T = 3 runs the stream kernel, T = 100 (50 routes per expert) the MFMA
    # lists with 4 column groups, whose LDS per workgroup is largest here
    cfg = _cfg(K=8192, I=8192, E_global=2, E_local=2, top_k=1, bias=True)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, T, seed=29 + T)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    _assert_close(y, ref["y"], f"K = I = 8192, T = {T}")


def test_layer_no_local_route_writes_zeros():
    cfg = _cfg(E_global=16, E_local=4, expert_offset=12, top_k=2)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 6, seed=8)
    inp.topk_ids[:] = np.array([0, 1], np.int32)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    assert np.array_equal(y, np.zeros_like(y)) and not np.signbit(y).any()


def test_layer_no_local_route_writes_zeros_stream_path():
    cfg = _cfg(K=1024, I=1024, E_global=16, E_local=4, expert_offset=12, top_k=2)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 6, seed=9)
    inp.topk_ids[:] = np.array([0, 1], np.int32)
    y = bf16_to_np(run_decode(cfg, DeviceLayer(w), inp))
    assert np.array_equal(y, np.zeros_like(y)) and not np.signbit(y).any()


@pytest.mark.parametrize("T", [3, 7, 24])
def test_down_step_twice_on_one_plan(T):
    # the down step reads only the plan and the intermediate the workspace
    # holds: a second down call on the same plan gives the same bits
    t = torch()
    cfg = _cfg(K=1056, I=1120, E_global=8, E_local=6, expert_offset=1, top_k=3, bias=True)
    w = make_weights(cfg)
    inp = make_inputs(cfg, T, t_index=T)
    ref = oracle.moe_forward_cfg(cfg, w, inp)
    layer = DeviceLayer(w)
    d = desc_for(cfg, T)
    ws = moe.moe_mxfp4_plan(d, router_logits=dev_f32(inp.logits))
    moe.moe_mxfp4_gate_up(d, dev_bf16(inp.x), layer.w13p, layer.w13s, ws, w13_bias=layer.b13)
    outs = []
    for _ in range(2):
        out = t.full((T, cfg.K), float("nan"), dtype=t.bfloat16, device="cuda")
        moe.moe_mxfp4_down(d, layer.w2p, layer.w2s, out, ws, w2_bias=layer.b2)
        t.cuda.synchronize()
        outs.append(bf16_bits_np(out))
    assert np.array_equal(outs[0], outs[1])
    _assert_close(bf16_to_np(out), ref["y"], f"down twice T{T}")


def test_layer_exact_chain_bit_exact():
    from test_oracle_layer import build_exact_chain
    t = torch()
    for c0 in (37, 70):
        arrays, want = build_exact_chain(c0, False)
        d = moe.make_desc(T=2, K=arrays["K"], I=arrays["I"], E_global=2, E_local=2, top_k=2)
        out = t.empty((2, arrays["K"]), dtype=t.bfloat16, device="cuda")
        moe.moe_mxfp4_decode(d, dev_bf16(arrays["x_bits"]), dev_u8(arrays["w13_packed"]),
                             dev_u8(arrays["w13_scales"]), dev_u8(arrays["w2_packed"]),
                             dev_u8(arrays["w2_scales"]), out, topk_ids=dev_i32(arrays["topk_ids"]),
                             topk_weights=dev_f32(arrays["topk_weights"]))
        t.cuda.synchronize()
        assert np.array_equal(bf16_to_np(out).astype(np.float64), want)


def test_layer_repeat_calls_bit_identical():
    t = torch()
    cfg = get_config("gptoss20b")
    w = make_weights(cfg, E_local=8)
    cfg2 = LayerConfig(**{**cfg.__dict__, "E_global": 8, "E_local": 8})
    inp = make_inputs(cfg2, 16)
    layer = DeviceLayer(w)
    ws = t.empty(moe.moe_mxfp4_workspace_bytes(desc_for(cfg2, 16)), dtype=t.uint8, device="cuda")
    first = bf16_bits_np(run_decode(cfg2, layer, inp, workspace=ws))
    for _ in range(3):
        assert np.array_equal(bf16_bits_np(run_decode(cfg2, layer, inp, workspace=ws)), first)


# --------------------------------------------------------------------------
# full workload shapes: every token count of every workload, weights tiled as
# the benchmark stores them, every token compared
# --------------------------------------------------------------------------
# The pages' parity runs ("MXFP4 MoE decode kernels", Parity) use random
# top-k routing and routing with every route local, at activation RMS 1 and 4.
# For the slices that hold every expert (the gpt-oss shapes) every route is
# local already; for the expert-parallel slices the all-local variant adds 8
# to the local experts' logits.  One layer per workload is kept (device
# weights and the oracle's dequantised experts) while its cases run.

_FULL = {}


def _full(name):
    if _FULL.get("name") != name:
        _FULL.clear()
        t = torch()
        t.cuda.empty_cache()
        cfg = get_config(name)
        print(f"full shape {name}: generating weights", flush=True)
        w = make_weights(cfg)
        _FULL.update(name=name, cfg=cfg, w=w, layer=DeviceLayer(w, layout="tile16"), cache={})
    return _FULL


FULL_CASES = ([("gptoss20b", T, "random") for T in (1, 4, 16, 32)] + [("gptoss20b", 4, "rms4")] +
              [("gptoss120b", T, "random") for T in (1, 4, 8, 16, 32)] +
              [("gptoss120b", 1, "rms4"), ("gptoss120b", 32, "rms4")] +
              [("glm5_ep", T, "random") for T in (1, 8, 32)] +
              [("glm5_ep", 1, "all_local"), ("glm5_ep", 8, "all_local"), ("glm5_ep", 32, "all_local_rms4")] +
              [("widek", T, "random") for T in (32, 256, 2048)] +
              [("widek", 32, "all_local"), ("widek", 32, "rms4"), ("widek", 256, "all_local_rms4")] +
              # the scaled-FP4 MFMA path at the calls whose experts take many routes
              [("widek", 256, "scaled_fp4"), ("widek", 2048, "scaled_fp4"), ("widek", 256, "all_local_rms4_scaled_fp4")])


@pytest.mark.parametrize("name,T,variant", FULL_CASES)
def test_full_shape_every_token(name, T, variant):
    F = _full(name)
    cfg = F["cfg"]
    inp = make_inputs(cfg, T, x_scale=4.0 if "rms4" in variant else 1.0,
                      all_local_boost=8.0 if "all_local" in variant else 0.0)
    print(f"full shape {name} T={T} {variant}: device call", flush=True)
    out = bf16_to_np(run_decode(cfg, F["layer"], inp, mma="scaled_fp4" if "scaled_fp4" in variant else "bf16"))
    print(f"full shape {name} T={T} {variant}: oracle", flush=True)
    ref = oracle.moe_forward_cfg(cfg, F["w"], inp, experts_cache=F["cache"])
    if "all_local" in variant:
        assert len(ref["routes"]) == T * cfg.top_k  # every route landed in the slice
    _assert_close(out, ref["y"], f"{name} T={T} {variant}", elementwise="scaled_fp4" not in variant)
