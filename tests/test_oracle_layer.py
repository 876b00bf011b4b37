"""Pins of the oracle's whole layer: brute force, an exact closed-form chain,
negative controls on the [gate; up] order, invariants, and planted mistakes.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import bruteforce as bf
from oracle import moe_oracle as mo
from workloads import LayerConfig, make_inputs, make_topk_inputs, make_weights, get_config

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cfg(**kw):
    base = dict(name="mini", description="mini", K=64, I=64, E_global=4, E_local=4, expert_offset=0,
                top_k=2, scoring="softmax", activation="silu_mul", bias=False, tokens=(3,),
                scale_lo=120, scale_hi=130, index=77)
    base.update(kw)
    return LayerConfig(**base)


def _bf_cfg(cfg, w, inp):
    return bf.moe_bruteforce(
        x_bits=inp.x, logits=inp.logits, topk_ids=inp.topk_ids, topk_weights=inp.topk_weights,
        w13_packed=w.w13_packed, w13_scales=w.w13_scales, w2_packed=w.w2_packed,
        w2_scales=w.w2_scales, b13=w.b13, b2=w.b2, K=cfg.K, I=cfg.I, E_global=cfg.E_global,
        E_local=w.w13_packed.shape[0], top_k=cfg.top_k, expert_offset=cfg.expert_offset,
        scoring=cfg.scoring, activation_kind=cfg.activation)


BRUTE_CASES = [
    dict(),
    dict(scoring="sigmoid", top_k=3),
    dict(activation="swiglu_oai", bias=True, scale_lo=118, scale_hi=124),
    dict(K=96, I=32, E_global=8, E_local=3, expert_offset=2, top_k=4, scoring="sigmoid"),
    dict(K=32, I=96, activation="swiglu_oai", bias=True, top_k=1),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
def test_oracle_matches_bruteforce(case):
    cfg = _cfg(**BRUTE_CASES[case])
    w = make_weights(cfg)
    inp = make_inputs(cfg, 3, x_scale=1.0)
    want = np.array(_bf_cfg(cfg, w, inp), dtype=np.float64)
    for dt, tol in ((np.float64, 1e-12), (np.float32, 1e-5)):
        got = oracle.moe_forward_cfg(cfg, w, inp, dtype=dt, round_intermediate=False)["y"]
        assert oracle.rel_l2(got, want) <= tol, (case, dt, oracle.rel_l2(got, want))
    # with the bf16 intermediate the result stays at the bf16 rounding floor
    got = oracle.moe_forward_cfg(cfg, w, inp)["y"]
    assert oracle.rel_l2(got, want) <= 3e-3


def test_oracle_matches_bruteforce_ids_mode_with_padding():
    cfg = _cfg(E_global=6, E_local=4, expert_offset=1, top_k=3)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 4, seed=5, pad_fraction=0.25)
    want = np.array(_bf_cfg(cfg, w, inp))
    got = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64, round_intermediate=False)["y"]
    assert oracle.rel_l2(got, want) <= 1e-12


# --------------------------------------------------------------------------
# exact dyadic chain with a hand closed form
# --------------------------------------------------------------------------

def _e2m1_code(value):
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        mag = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        v = -mag if s else mag
        if v == value and math.copysign(1, v) == math.copysign(1, value):
            return c
    raise ValueError(value)


def build_exact_chain(c0, with_bias=False):
    """One-hot activations, dyadic weights: every product and sum is exact.

    K=96, I=64, 2 experts, top-2 in ids mode, T=2.  Only column c0 of w13 is
    non-zero; gate values are >= 64 so sigmoid(gate) is exactly 1 and
    SiLU(gate) == gate; row kk of w2 has one non-zero, at column pi(kk), and
    only in expert kk % 2.  Returns (arrays, closed-form y) with y computed
    from the chosen values, not from the bytes.
    """
    K, I, E, k = 96, 64, 2, 2
    w13p = np.zeros((E, 2 * I, K // 2), np.uint8)
    w13s = np.full((E, 2 * I, K // 32), 127, np.uint8)
    w2p = np.zeros((E, K, I // 2), np.uint8)
    w2s = np.full((E, K, I // 32), 127, np.uint8)
    G = np.zeros((E, I))
    U = np.zeros((E, I))
    gate_mags = [2.0, 3.0, 4.0, 6.0]
    up_vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    blk = c0 // 32

    def put(arr, e, row, col, code):
        b = arr[e, row, col // 2]
        arr[e, row, col // 2] = (b & 0xF0) | code if col % 2 == 0 else (b & 0x0F) | (code << 4)

    for e in range(E):
        for n in range(I):
            g = gate_mags[(n + e) % 4]
            u = up_vals[(3 * n + 5 * e) % len(up_vals)]
            put(w13p, e, n, c0, _e2m1_code(g))
            w13s[e, n, blk] = 132                   # x 2^5
            put(w13p, e, I + n, c0, _e2m1_code(u))
            w13s[e, I + n, blk] = 126               # x 2^-1
            G[e, n] = g * 32.0
            U[e, n] = u * 0.5
    V = np.zeros((E, K))
    PI = [(5 * kk + 3) % I for kk in range(K)]
    for kk in range(K):
        e = kk % 2
        v = [1.0, -2.0, 1.5, -0.5, 3.0, 6.0, -4.0][kk % 7]
        put(w2p, e, kk, PI[kk], _e2m1_code(v))
        s2 = 126 + (kk % 3)
        w2s[e, kk, PI[kk] // 32] = s2
        V[e, kk] = v * 2.0 ** (s2 - 127)

    ids = np.array([[0, 1], [1, 0]], np.int32)
    wts = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    xs = [1.0, 2.0]                                  # token t has x[t, c0] = xs[t]
    x = np.zeros((2, K), np.uint16)
    x[0, c0] = 0x3F80
    x[1, c0] = 0x4000
    b13 = b2 = None
    gb, ub, ob = 32.0, 0.5, -0.125     # keep g*u within bf16's 8 significant bits
    if with_bias:
        b13 = np.zeros((E, 2 * I), np.uint16)
        b13[:, :I] = 0x4200      # 32.0
        b13[:, I:] = 0x3F00      # 0.5
        b2 = np.full((E, K), 0xBE00, np.uint16)  # -0.125

    y = np.zeros((2, K))
    for t in range(2):
        for j in range(k):
            e = ids[t, j]
            for kk in range(K):
                g = xs[t] * G[e, PI[kk]] + (gb if with_bias else 0.0)
                u = xs[t] * U[e, PI[kk]] + (ub if with_bias else 0.0)
                o = V[e, kk] * (g * u) + (ob if with_bias else 0.0)
                y[t, kk] += float(wts[t, j]) * o
    arrays = dict(x_bits=x, topk_ids=ids, topk_weights=wts, w13_packed=w13p, w13_scales=w13s,
                  w2_packed=w2p, w2_scales=w2s, b13=b13, b2=b2, K=K, I=I, E_global=E, E_local=E,
                  top_k=k)
    return arrays, y


def exact_chain_holds(dtype=np.float32):
    for c0 in (37, 70):              # odd column = high nibble (block 1), even = low nibble (block 2)
        for with_bias in (False, True):
            arrays, want = build_exact_chain(c0, with_bias)
            got = oracle.moe_forward(**arrays, dtype=dtype)["y"]
            if not np.array_equal(got.astype(np.float64), want):
                return False
    return True


def test_exact_chain_closed_form():
    assert exact_chain_holds(np.float32)
    assert exact_chain_holds(np.float64)
    # the bias-free chain output is exactly representable in bf16 (usable as a bit-exact device check)
    for c0 in (37, 70):
        _, want = build_exact_chain(c0, False)
        assert np.array_equal(oracle.round_to_bf16(want), want)


# --------------------------------------------------------------------------
# planted mistakes: each must break at least one pin
# --------------------------------------------------------------------------

def _high_nibble_first(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = packed >> 4
    codes[..., 1::2] = packed & 0x0F
    return codes


def test_planted_mistakes_are_caught(monkeypatch):
    real_dequant = mo.dequantize
    real_act = mo.activation

    with monkeypatch.context() as m:
        m.setattr(mo, "unpack_codes", _high_nibble_first)
        assert not exact_chain_holds()

    def up_gate(gate, up, kind, alpha=1.702, limit=7.0):
        return real_act(up, gate, kind, alpha, limit)
    with monkeypatch.context() as m:
        m.setattr(mo, "activation", up_gate)
        assert not exact_chain_holds()

    def wrong_scale_block(packed, scales):  # scales applied to the neighbouring block
        return real_dequant(packed, np.roll(scales, 1, axis=-1))
    with monkeypatch.context() as m:
        m.setattr(mo, "dequantize", wrong_scale_block)
        assert not exact_chain_holds()

    def no_bias_f(bits):
        return np.zeros(np.shape(bits), np.float32)
    with monkeypatch.context() as m:   # biases dropped
        orig = mo.bf16_bits_to_float
        m.setattr(mo, "bf16_bits_to_float",
                  lambda b: no_bias_f(b) if np.ndim(b) == 1 else orig(b))
        assert not exact_chain_holds()

    def silu_without_sigmoid(gate, up, kind, alpha=1.702, limit=7.0):
        return gate * up * np.asarray(0.5, gate.dtype)
    with monkeypatch.context() as m:
        m.setattr(mo, "activation", silu_without_sigmoid)
        assert not exact_chain_holds()


def test_planted_routing_mistakes_are_caught(monkeypatch):
    logits = np.array([[0.1, 2.0, -1.0, 2.0, 0.5]], np.float32)
    real_lexsort = np.lexsort
    with monkeypatch.context() as m:   # ties to the higher id
        m.setattr(mo.np, "lexsort", lambda keys: real_lexsort((-keys[0], keys[1])))
        ids, _ = mo.route_topk(logits, 2, "softmax")
    assert ids[0].tolist() != [1, 3]


# --------------------------------------------------------------------------
# negative controls on the [gate; up] order
# --------------------------------------------------------------------------

def _swap_halves(w13p, w13s, I):
    return (np.concatenate([w13p[:, I:], w13p[:, :I]], axis=1),
            np.concatenate([w13s[:, I:], w13s[:, :I]], axis=1))


def _as_interleaved(w13p, w13s):
    # read the same rows as if they were interleaved gate/up: gate = even rows, up = odd rows
    return (np.concatenate([w13p[:, 0::2], w13p[:, 1::2]], axis=1),
            np.concatenate([w13s[:, 0::2], w13s[:, 1::2]], axis=1))


@pytest.mark.parametrize("cfg_name", ["tiny"])
def test_gate_up_negative_controls(cfg_name):
    cfg = get_config(cfg_name)   # scales 118..130 put the gate far into SiLU's non-linear range
    w = make_weights(cfg)
    inp = make_inputs(cfg, 4)
    ref = oracle.moe_forward_cfg(cfg, w, inp)["y"]
    for name, (p, s) in (("[up; gate]", _swap_halves(w.w13_packed, w.w13_scales, cfg.I)),
                         ("interleaved", _as_interleaved(w.w13_packed, w.w13_scales))):
        y = oracle.moe_forward(
            x_bits=inp.x, logits=inp.logits, w13_packed=p, w13_scales=s,
            w2_packed=w.w2_packed, w2_scales=w.w2_scales, K=cfg.K, I=cfg.I,
            E_global=cfg.E_global, E_local=cfg.E_local, top_k=cfg.top_k,
            scoring=cfg.scoring, activation_kind=cfg.activation)["y"]
        err = oracle.rel_l2(y, ref)
        if err < 0.05:
            pytest.fail(f"inconclusive: the {name} control survived (rel_l2 {err:.3g})")


# --------------------------------------------------------------------------
# interleaved gate/up rows and the per-route output
# --------------------------------------------------------------------------

def interleave_rows(a, I):
    """[E, 2I, ...] rows [gate; up] -> rows gate 0, up 0, gate 1, up 1, ..."""
    out = np.empty_like(a)
    out[:, 0::2] = a[:, :I]
    out[:, 1::2] = a[:, I:]
    return out


INTERLEAVED_CASES = [
    dict(),
    dict(activation="swiglu_oai", bias=True, scale_lo=118, scale_hi=124),
    dict(K=96, I=32, E_global=8, E_local=3, expert_offset=2, top_k=4, scoring="sigmoid", bias=True),
]


@pytest.mark.parametrize("case", range(len(INTERLEAVED_CASES)))
def test_interleaved_order_matches_bruteforce_and_gate_up(case):
    cfg = _cfg(**INTERLEAVED_CASES[case])
    w = make_weights(cfg)
    inp = make_inputs(cfg, 3, x_scale=1.0)
    I = cfg.I
    p, sc = interleave_rows(w.w13_packed, I), interleave_rows(w.w13_scales, I)
    b13 = None if w.b13 is None else interleave_rows(w.b13, I)
    want = np.array(bf.moe_bruteforce(
        x_bits=inp.x, logits=inp.logits, w13_packed=p, w13_scales=sc, w2_packed=w.w2_packed,
        w2_scales=w.w2_scales, b13=b13, b2=w.b2, K=cfg.K, I=I, E_global=cfg.E_global,
        E_local=w.w13_packed.shape[0], top_k=cfg.top_k, expert_offset=cfg.expert_offset,
        scoring=cfg.scoring, activation_kind=cfg.activation, w13_order="interleaved"), dtype=np.float64)
    kw = dict(x_bits=inp.x, logits=inp.logits, w2_packed=w.w2_packed, w2_scales=w.w2_scales, b2=w.b2,
              K=cfg.K, I=I, E_global=cfg.E_global, E_local=w.w13_packed.shape[0], top_k=cfg.top_k,
              expert_offset=cfg.expert_offset, scoring=cfg.scoring, activation_kind=cfg.activation,
              dtype=np.float64, round_intermediate=False)
    got = oracle.moe_forward(w13_packed=p, w13_scales=sc, b13=b13, w13_order="interleaved", **kw)["y"]
    assert oracle.rel_l2(got, want) <= 1e-12
    same = oracle.moe_forward(w13_packed=w.w13_packed, w13_scales=w.w13_scales, b13=w.b13, **kw)["y"]
    assert oracle.rel_l2(got, same) <= 1e-12
    # each order read as the other is far off
    wrong = oracle.moe_forward(w13_packed=p, w13_scales=sc, b13=b13, **kw)["y"]
    wrong2 = oracle.moe_forward(w13_packed=w.w13_packed, w13_scales=w.w13_scales, b13=w.b13,
                                w13_order="interleaved", **kw)["y"]
    assert oracle.rel_l2(wrong, want) > 0.05 and oracle.rel_l2(wrong2, want) > 0.05


def test_exact_chain_interleaved_storage():
    # the closed form does not depend on how the rows are stored
    for c0 in (37, 70):
        for with_bias in (False, True):
            arrays, want = build_exact_chain(c0, with_bias)
            I = arrays["I"]
            arrays["w13_packed"] = interleave_rows(arrays["w13_packed"], I)
            arrays["w13_scales"] = interleave_rows(arrays["w13_scales"], I)
            if arrays["b13"] is not None:
                arrays["b13"] = interleave_rows(arrays["b13"], I)
            for dt in (np.float32, np.float64):
                got = oracle.moe_forward(**arrays, dtype=dt, w13_order="interleaved")["y"]
                assert np.array_equal(got.astype(np.float64), want), (c0, with_bias, dt)


@pytest.mark.parametrize("case", [dict(), dict(K=96, I=32, E_global=8, E_local=3, expert_offset=2, top_k=4,
                                               scoring="sigmoid", bias=True)])
def test_route_outputs_match_bruteforce_and_sum_to_y(case):
    cfg = _cfg(**case)
    w = make_weights(cfg)
    T = 3
    inp = make_inputs(cfg, T, x_scale=1.0)
    res = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64, round_intermediate=False)
    rows = oracle.route_outputs(res, T, cfg.top_k)
    assert rows.shape == (T * cfg.top_k, cfg.K)
    _, want = bf.moe_bruteforce(
        x_bits=inp.x, logits=inp.logits, w13_packed=w.w13_packed, w13_scales=w.w13_scales,
        w2_packed=w.w2_packed, w2_scales=w.w2_scales, b13=w.b13, b2=w.b2, K=cfg.K, I=cfg.I,
        E_global=cfg.E_global, E_local=w.w13_packed.shape[0], top_k=cfg.top_k,
        expert_offset=cfg.expert_offset, scoring=cfg.scoring, activation_kind=cfg.activation,
        per_route=True)
    local = np.zeros(T * cfg.top_k, bool)
    for r, row in want.items():
        local[r] = True
        assert oracle.rel_l2(rows[r], np.array(row)) <= 1e-12, r
    assert not rows[~local].any()                       # routes outside the slice: zero rows
    if case:
        assert (~local).any()                           # the slice case has some
    # sum over j of w[t, j] * row(t, j) is the layer output
    y = np.einsum("tj,tjk->tk", res["weights"].astype(np.float64),
                  rows.reshape(T, cfg.top_k, cfg.K))
    assert oracle.rel_l2(y, res["y"]) <= 1e-12


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_identical_experts_make_routing_irrelevant():
    cfg = _cfg(K=128, I=64, E_global=6, E_local=6, top_k=3, scoring="sigmoid")
    w = make_weights(cfg)
    for arr in (w.w13_packed, w.w13_scales, w.w2_packed, w.w2_scales):
        arr[:] = arr[0:1]
    inp = make_inputs(cfg, 5)
    y = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64)["y"]
    single = oracle.moe_forward(
        x_bits=inp.x, topk_ids=np.zeros((5, 1), np.int32), topk_weights=np.ones((5, 1), np.float32),
        w13_packed=w.w13_packed[:1], w13_scales=w.w13_scales[:1], w2_packed=w.w2_packed[:1],
        w2_scales=w.w2_scales[:1], K=cfg.K, I=cfg.I, E_global=1, E_local=1, top_k=1,
        dtype=np.float64)["y"]
    assert oracle.rel_l2(y, single) < 1e-12


def test_linearity_in_routing_weights():
    cfg = _cfg(K=128, I=64, E_global=8, E_local=8, top_k=2)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 6, seed=9)
    y1 = oracle.moe_forward_cfg(cfg, w, inp)["y"]
    inp.topk_weights = inp.topk_weights * np.float32(2)
    y2 = oracle.moe_forward_cfg(cfg, w, inp)["y"]
    assert np.array_equal(y2, y1 * np.float32(2))


def test_expert_parallel_slices_sum_to_full_layer():
    cfg = _cfg(K=128, I=64, E_global=8, E_local=8, top_k=3, scoring="sigmoid")
    w = make_weights(cfg)
    inp = make_inputs(cfg, 7)
    full = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64)["y"]
    parts = np.zeros_like(full)
    for off in (0, 3, 5):
        n = {0: 3, 3: 2, 5: 3}[off]
        sub = make_weights(cfg)
        for name in ("w13_packed", "w13_scales", "w2_packed", "w2_scales"):
            setattr(sub, name, getattr(w, name)[off:off + n])
        parts += oracle.moe_forward_cfg(cfg, sub, inp, dtype=np.float64, expert_offset=off)["y"]
    assert oracle.rel_l2(parts, full) < 1e-12


def test_batch_invariance():
    cfg = _cfg(K=128, I=64, E_global=8, E_local=8, top_k=2)
    w = make_weights(cfg)
    inp = make_inputs(cfg, 6)
    yb = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64)["y"]
    for t in range(6):
        one = make_inputs(cfg, 6)
        one.x = inp.x[t:t + 1]
        one.logits = inp.logits[t:t + 1]
        yt = oracle.moe_forward_cfg(cfg, w, one, dtype=np.float64)["y"]
        assert oracle.rel_l2(yt[0], yb[t]) < 1e-14


def test_fp32_oracle_within_fp64_bound():
    cfg = get_config("tiny")
    w = make_weights(cfg)
    inp = make_inputs(cfg, 4)
    y64 = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float64, round_intermediate=False)["y"]
    y32 = oracle.moe_forward_cfg(cfg, w, inp, dtype=np.float32, round_intermediate=False)["y"]
    assert oracle.rel_l2(y32, y64) < 1e-5


def test_no_local_routes_gives_zero():
    cfg = _cfg(E_global=8, E_local=2, expert_offset=6, top_k=1)
    w = make_weights(cfg)
    inp = make_topk_inputs(cfg, 3, seed=1)
    inp.topk_ids[:] = 0
    r = oracle.moe_forward_cfg(cfg, w, inp)
    assert not r["y"].any() and r["routes"].size == 0


def test_empty_batch():
    cfg = _cfg()
    w = make_weights(cfg)
    inp = make_inputs(cfg, 3)
    inp.x = inp.x[:0]
    inp.logits = inp.logits[:0]
    r = oracle.moe_forward_cfg(cfg, w, inp)
    assert r["y"].shape == (0, cfg.K)
