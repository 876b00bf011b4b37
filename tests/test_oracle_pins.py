"""Pins of the CPU oracle's building blocks against facts fixed outside it.

Each test checks one oracle function against something other than itself:
the format's bit-field definition, IEEE bit patterns, hand-worked examples
stored under tests/golden/ (with the passage they come from), library routines
(torch's bf16 cast, scipy's softmax/expit) or brute force.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import bruteforce as bf

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _e2m1_bitfields(code):
    # OCP E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal.
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_table_matches_bit_fields():
    for code in range(16):
        v = float(oracle.e2m1_to_float(np.array([code]))[0])
        assert v == _e2m1_bitfields(code)
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0), code
    mags = np.abs(oracle.e2m1_to_float(np.arange(16)))
    assert mags.max() == 6.0  # the encoder section: everything above 6.0 clamps


def test_e8m0_matches_ieee_exponent_field():
    s = np.arange(256)
    got = oracle.e8m0_to_float(s)
    # IEEE binary32 with exponent field s and zero fraction is 2**(s-127) for 1 <= s <= 254;
    # s = 0 is below the normal range: 2**-127 is the subnormal with fraction bit 22 set.
    want = (s[1:255].astype(np.uint32) << 23).view(np.float32)
    assert np.array_equal(got[1:255], want)
    assert got[0] == np.array([0x00400000], dtype=np.uint32).view(np.float32)[0]
    assert got[0] == 2.0 ** -127
    assert np.isnan(got[255])


def test_dequant_exhaustive_codes_scales_nibble_positions():
    # row s carries scale s; byte i holds code i in the low nibble and code 15-i in the high nibble
    byte_row = np.array([(i & 0xF) | ((15 - i) << 4) for i in range(16)], dtype=np.uint8)
    packed = np.tile(byte_row, (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = oracle.dequantize(packed, scales)
    assert got.shape == (256, 32) and got.dtype == np.float32
    for s in range(256):
        for col in range(32):
            code = (col // 2) if col % 2 == 0 else 15 - col // 2
            v = got[s, col]
            if s == 255:
                assert np.isnan(v)
                continue
            want = np.float32(math.ldexp(_e2m1_bitfields(code), s - 127)) if abs(
                math.ldexp(_e2m1_bitfields(code), s - 127)) < 3.5e38 else np.float32(
                math.copysign(math.inf, _e2m1_bitfields(code)))
            assert v == want and np.signbit(v) == np.signbit(want), (s, col, v, want)


def test_unpack_bf16_exhaustive_is_exact():
    # every code x every scale x both nibble positions: the bf16 pattern widens
    # back to the fp32 dequantisation exactly and equals round-to-nearest-even
    # of it (computed from float64, a separate path); NaN stays NaN
    byte_row = np.array([(i & 0xF) | ((15 - i) << 4) for i in range(16)], dtype=np.uint8)
    packed = np.tile(byte_row, (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    bits = oracle.unpack_bf16(packed, scales)
    f = oracle.dequantize(packed, scales)
    wide = oracle.bf16_bits_to_float(bits)
    nan = np.isnan(f)
    assert np.array_equal(np.isnan(wide), nan) and nan[255].all() and not nan[:255].any()
    assert np.array_equal(wide[~nan].view(np.uint32), f[~nan].view(np.uint32))
    rn = oracle.round_to_bf16(f[~nan].astype(np.float64))
    assert np.array_equal(rn, f[~nan].astype(np.float64))


def test_nibble_order_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "mxfp4_format.json")))
    for ex in g["nibble_examples"]:
        row = np.zeros((1, 16), dtype=np.uint8)
        row[0, 0] = ex["byte"]
        got = oracle.dequantize(row, np.array([[ex["scale"]]], dtype=np.uint8))[0, :2]
        for v, w in zip(got, ex["values"]):
            assert v == w and np.signbit(v) == np.signbit(np.float32(w)), ex


def test_nibble_order_agrees_with_lane_map(golden_dir):
    # The pages' lane map: nibble plane p of 16-bit lane i carries element 4i+p of the chunk.
    g = json.load(open(os.path.join(golden_dir, "mxfp4_format.json")))["lane_map"]
    rng = np.random.default_rng(3)
    chunk = rng.integers(0, 256, size=g["chunk"] // 2, dtype=np.uint8)
    codes = oracle.unpack_codes(chunk)
    lanes = chunk.view("<u2")
    for i, lane in enumerate(lanes):
        for p in range(g["planes"]):
            assert (int(lane) >> (4 * p)) & 0xF == codes[4 * i + p]


def test_scale_indexing_one_block_per_row():
    rng = np.random.default_rng(5)
    rows, cols = 6, 128
    packed = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    base = np.full((rows, cols // 32), 127, dtype=np.uint8)
    ref = oracle.dequantize(packed, base)
    for n in range(rows):
        blk = (n * 3 + 1) % (cols // 32)
        sc = base.copy()
        sc[n, blk] = 129
        got = oracle.dequantize(packed, sc)
        changed = got != ref
        expect = np.zeros_like(changed)
        expect[n, blk * 32:(blk + 1) * 32] = ref[n, blk * 32:(blk + 1) * 32] != 0
        assert np.array_equal(changed, expect)
        assert np.array_equal(got[n, blk * 32:(blk + 1) * 32], ref[n, blk * 32:(blk + 1) * 32] * 4)


def test_bf16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = rng.standard_normal(20000).astype(np.float32) * np.float32(1000)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    v2 = bits.view(np.float32)
    v2 = v2[np.isfinite(v2)]
    # exact ties: low 16 bits = 0x8000, with even and odd kept parts
    ties = ((rng.integers(0x3F00, 0x4100, size=2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3961776e38, -3.3961776e38, 1e-40, -1e-40,
                        1.17549435e-38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135], dtype=np.float32)
    allv = np.concatenate([v, v2, ties, special]).astype(np.float32)
    got = oracle.round_to_bf16(allv)
    want = torch.from_numpy(allv).to(torch.bfloat16).to(torch.float32).numpy()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), allv[~same][:10]
    assert np.array_equal(np.signbit(got[np.isfinite(got)]), np.signbit(want[np.isfinite(want)]))


def test_bf16_rounding_float64_is_direct():
    # fp64 input rounds once: 1 + 2^-8 + 2^-30 lies just above the tie and must round up,
    # whereas rounding through fp32 first would land on the tie and round to even (down).
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30], dtype=np.float64)
    assert oracle.round_to_bf16(v)[0] == 1.0 + 2.0 ** -7
    assert oracle.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def test_routing_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "routing_examples.json")))
    for case in g["cases"]:
        l = np.array([case["logits"]], dtype=np.float32)
        ids, w = oracle.route_topk(l, case["top_k"], case["scoring"], dtype=np.float64)
        assert ids.dtype == np.int32
        assert ids[0].tolist() == case["ids"], case
        if "weights" in case:
            assert np.allclose(w[0], case["weights"], rtol=1e-12, atol=0)
    ids, w = oracle.route_topk(np.array([[1.0, 3.0, 2.0]], np.float32), 2, "softmax", dtype=np.float64)
    e = math.exp(-1.0)
    assert np.allclose(w[0], [1 / (1 + e), e / (1 + e)], rtol=1e-14)


def test_routing_against_library_and_bruteforce():
    sp = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(11)
    for scoring in ("softmax", "sigmoid"):
        for E, k in ((8, 2), (32, 4), (128, 4), (256, 8), (384, 8)):
            # quantise to force ties
            logits = (np.round(rng.standard_normal((16, E)) * 4) / 4).astype(np.float32)
            ids, w = oracle.route_topk(logits, k, scoring, dtype=np.float64)
            for t in range(16):
                assert ids[t].tolist() == bf.topk_by_argmax([float(v) for v in logits[t]], k)
                assert len(set(ids[t].tolist())) == k
                sel = logits[t, ids[t]].astype(np.float64)
                rest = np.delete(logits[t], ids[t])
                assert sel.min() >= rest.max()
                if scoring == "softmax":
                    want = sp.softmax(sel)
                else:
                    want = sp.expit(sel) / sp.expit(sel).sum()
                assert np.allclose(w[t], want, rtol=1e-12)
                assert abs(w[t].sum() - 1) < 1e-12
            # float32 weights are within a few ulps of the fp64 ones and sum to 1
            _, w32 = oracle.route_topk(logits, k, scoring, dtype=np.float32)
            assert np.allclose(w32, w, rtol=2e-6)
            assert np.all(np.abs(w32.sum(axis=1, dtype=np.float64) - 1) < 1e-6)


def test_bucketing_against_bruteforce():
    rng = np.random.default_rng(13)
    for E_g, E_l, off, k, T in ((8, 8, 0, 2, 4), (256, 32, 64, 8, 32), (384, 48, 336, 8, 257),
                                (128, 128, 0, 4, 1), (32, 32, 0, 4, 0)):
        ids = np.stack([rng.choice(E_g, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        if T:
            ids[rng.random(ids.shape) < 0.1] = -1
        counts, offsets, routes = oracle.bucket_routes(ids, E_l, off)
        flat = ids.reshape(-1)
        bf_routes = []
        for e in range(E_l):  # O(E * R) scan
            mine = [r for r in range(flat.size) if flat[r] == e + off]
            assert counts[e] == len(mine)
            bf_routes += mine
        assert routes.tolist() == bf_routes
        assert offsets[0] == 0 and offsets[-1] == len(routes)
        assert np.array_equal(np.diff(offsets), counts)
        assert routes.dtype == np.int32 and counts.dtype == np.int32


def test_activation_closed_forms():
    f32 = np.float32
    # SwiGLU-OAI: gate capped at 7 (upper only), up clamped to +-7, then g*sigmoid(1.702 g)*(u+1)
    a = oracle.activation(np.array([10.0]), np.array([-9.0]), "swiglu_oai")[0]
    assert a == pytest.approx(7 * (1 / (1 + math.exp(-1.702 * 7))) * (-6), rel=1e-14)
    a = oracle.activation(np.array([-3.0]), np.array([2.5]), "swiglu_oai")[0]
    assert a == pytest.approx(-3 / (1 + math.exp(1.702 * 3)) * 3.5, rel=1e-14)
    a = oracle.activation(np.array([1.0]), np.array([9.0]), "swiglu_oai", alpha=1.702, limit=7.0)[0]
    assert a == pytest.approx(1 / (1 + math.exp(-1.702)) * 8, rel=1e-14)
    # SiLU * up
    assert oracle.activation(np.array([0.0]), np.array([5.0]), "silu_mul")[0] == 0.0
    a = oracle.activation(np.array([2.0]), np.array([-0.5]), "silu_mul")[0]
    assert a == pytest.approx(2 / (1 + math.exp(-2)) * -0.5, rel=1e-14)
    # sigmoid saturates to exactly 1 in fp32 above ~17: SiLU(g) == g exactly
    g = np.array([64.0, 96.0, 17.5], dtype=f32)
    assert np.array_equal(oracle.activation(g, np.ones(3, f32), "silu_mul"), g)
    # a very negative gate gives -0 / 0, never NaN
    assert np.isfinite(oracle.activation(np.array([-200.0], f32), np.array([3.0], f32), "silu_mul")).all()


# --------------------------------------------------------------------------
# tiled weight layout: a byte permutation, pinned by labelling every piece
# --------------------------------------------------------------------------

def _labelled_rows(groups, blocks):
    """Rows whose 16-byte pieces carry (row, block) in their first bytes."""
    rows = 16 * groups
    a = np.zeros((rows, 16 * blocks), np.uint8)
    for r in range(rows):
        for b in range(blocks):
            a[r, 16 * b] = r % 256
            a[r, 16 * b + 1] = r // 256
            a[r, 16 * b + 2] = b
            a[r, 16 * b + 3:16 * b + 16] = np.arange(13, dtype=np.uint8) + (r * 7 + b) % 200
    return a


@pytest.mark.parametrize("groups,blocks", [(1, 1), (1, 4), (3, 90), (2, 17)])
def test_tile16_places_block_b_of_row_r_at_256b_plus_16r(groups, blocks):
    a = _labelled_rows(groups, blocks)
    t = oracle.tile16(a).reshape(-1)
    for g in range(groups):
        base = g * 16 * 16 * blocks
        for r in range(16):
            for b in range(blocks):
                off = base + 256 * b + 16 * r
                assert list(t[off:off + 16]) == list(a[16 * g + r, 16 * b:16 * b + 16])


def test_tile16_round_trip_and_leading_axes():
    rng = np.random.default_rng(5)
    a = rng.integers(0, 256, size=(3, 64, 48), dtype=np.uint8)   # 3 experts, 64 rows, 96 values per row
    t = oracle.tile16(a)
    assert t.shape == a.shape and not np.array_equal(t, a)
    assert np.array_equal(oracle.untile16(t), a)
    for e in range(3):                                             # experts are tiled on their own
        assert np.array_equal(t[e], oracle.tile16(a[e]))
    assert np.array_equal(np.sort(t.reshape(-1)), np.sort(a.reshape(-1)))


def test_tile16_single_block_rows_are_unchanged():
    # with one block per row, block-major and row-major orders coincide
    a = np.arange(32 * 16, dtype=np.uint32).astype(np.uint8).reshape(32, 16)
    assert np.array_equal(oracle.tile16(a), a)


# --------------------------------------------------------------------------
# MXFP4 encoder (OCP and Quark exponent rules)
# --------------------------------------------------------------------------

def test_e2m1_rounding_ties_to_even_and_saturates():
    vals = np.array([0.0, 0.25, 0.2500001, 0.75, 1.25, 1.2500001, 1.75, 2.5, 3.5, 5.0, 5.0000001, 6.0, 6.9, 1e9])
    want = [0, 0, 1, 2, 2, 3, 4, 4, 6, 6, 7, 7, 7, 7]
    assert oracle.round_to_e2m1(vals).tolist() == want


def test_encoder_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "mxfp4_encoder.json")))
    for blk in g["blocks"]:
        v = np.zeros(32, np.float32)
        v[:len(blk["values"])] = blk["values"]
        for rule in ("ocp", "quark"):
            packed, scales = oracle.encode_mxfp4(v[None, :], rule)
            codes = oracle.unpack_codes(packed)[0][:len(blk["values"])]
            assert int(scales[0, 0]) == blk[rule]["scale"], (blk["note"], rule)
            assert codes.tolist() == blk[rule]["codes"], (blk["note"], rule, codes.tolist())


def test_encoder_round_trip_of_decoded_blocks():
    # dequantised blocks whose largest code is 4 or 6 re-encode to the same bytes
    # under both rules (amax / 2^X is 4 or 6, below the bump threshold 7)
    rng = np.random.default_rng(21)
    rows, cols = 64, 256
    packed = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    codes = oracle.unpack_codes(packed).reshape(rows, cols // 32, 32)
    codes[..., 0] = rng.choice([6, 7, 14, 15], size=(rows, cols // 32))   # |value| 4 or 6 in every block
    lo = codes.reshape(rows, cols)
    packed = (lo[:, 0::2] | (lo[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(2, 250, size=(rows, cols // 32), dtype=np.uint8)
    v = oracle.dequantize(packed, scales)
    for rule in ("ocp", "quark"):
        p2, s2 = oracle.encode_mxfp4(v, rule)
        assert np.array_equal(s2, scales) and np.array_equal(p2, packed), rule


def test_encoder_rules_disagree_on_about_a_fifth_of_gaussian_blocks():
    # the page: the spec rule matches only about 80% of Quark's scale bytes;
    # for amax spread over octaves the bump fires when frac(log2 amax) >= log2(7/4)
    rng = np.random.default_rng(22)
    w = rng.standard_normal((512, 2048)).astype(np.float32)
    _, s_ocp = oracle.encode_mxfp4(w, "ocp")
    _, s_q = oracle.encode_mxfp4(w, "quark")
    diff = np.mean(s_ocp != s_q)
    assert 0.10 < diff < 0.30, diff
    assert np.all((s_q.astype(int) - s_ocp.astype(int)) >= 0) and np.all((s_q.astype(int) - s_ocp.astype(int)) <= 1)


def test_encoder_error_bounds_and_quark_is_more_accurate():
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((256, 1024)) * np.exp(rng.standard_normal((256, 1)))).astype(np.float32)
    errs = {}
    for rule, bound in (("ocp", 2.0), ("quark", 1.0)):
        packed, scales = oracle.encode_mxfp4(w, rule)
        d = oracle.dequantize(packed, scales).astype(np.float64)
        step = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
        # nearest-grid rounding: half the widest gap (1 * 2^X) unless the value
        # is above 6 * 2^X, which only the OCP rule allows (clamped from below 8 * 2^X)
        assert np.all(np.abs(d - w) <= bound * step + 1e-30), rule
        errs[rule] = np.linalg.norm(d - w) / np.linalg.norm(w)
    assert errs["quark"] < errs["ocp"], errs


# --------------------------------------------------------------------------
# acceptance metrics: hand-computed vectors with closed-form answers
# --------------------------------------------------------------------------
# Reading (the pages name rel_l2 and cosine without defining them): over the
# flattened output, rel_l2 = ||test - ref||_2 / ||ref||_2 and
# cosine = <test, ref> / (||test|| ||ref||).  The vectors below are chosen so
# that the plausible mistakes give other values: a squared norm ratio, a
# missing normalisation, a mean of element-wise relative errors, a norm
# taken per row instead of over the whole array.

def test_rel_l2_closed_forms():
    # 3-4-5: the difference is an eighth of the reference -> exactly 0.125
    # (a squared ratio would give 0.015625, an unnormalised norm 0.625)
    assert oracle.rel_l2(np.array([3.375, 4.5]), np.array([3.0, 4.0])) == 0.125
    # equal arrays -> 0
    assert oracle.rel_l2(np.array([1.5, -2.0, 7.0]), np.array([1.5, -2.0, 7.0])) == 0.0
    # one small element off by 100%, one large exact: 1 / sqrt(1 + 100^2),
    # not the mean element-wise relative error 0.5
    got = oracle.rel_l2(np.array([2.0, 100.0]), np.array([1.0, 100.0]))
    assert got == pytest.approx(1.0 / math.sqrt(10001.0), rel=1e-15)
    # the opposite sign: ||2 ref|| / ||ref|| = 2
    assert oracle.rel_l2(np.array([-3.0, -4.0]), np.array([3.0, 4.0])) == 2.0
    # norms over the whole [T, K] array, not per row: rows [3, 4] (error
    # [0.375, 0.5]) and [0, 0] (exact) -> 0.625 / 5
    t = np.array([[3.375, 4.5], [0.0, 0.0]])
    r = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert oracle.rel_l2(t, r) == 0.125
    # a second row with its own error adds in quadrature:
    # ||[0.375, 0.5, 0, 12]|| / ||[3, 4, 0, 12]|| = sqrt(144.390625) / 13
    t2 = np.array([[3.375, 4.5], [0.0, 24.0]])
    r2 = np.array([[3.0, 4.0], [0.0, 12.0]])
    assert oracle.rel_l2(t2, r2) == pytest.approx(math.sqrt(0.140625 + 0.25 + 144.0) / 13.0, rel=1e-15)


def test_rel_l2_invariances_and_zero_reference():
    rng = np.random.default_rng(5)
    t, r = rng.standard_normal(1000), rng.standard_normal(1000)
    # a power-of-two scale of both arrays changes nothing (exact in binary)
    assert oracle.rel_l2(8.0 * t, 8.0 * r) == oracle.rel_l2(t, r)
    # the reference's norm is the denominator: swapping the arguments changes the value
    assert oracle.rel_l2(2.0 * r, r) == pytest.approx(1.0, rel=1e-15)
    assert oracle.rel_l2(r, 2.0 * r) == pytest.approx(0.5, rel=1e-15)
    # an all-zero reference (a slice with no local route): only an all-zero
    # output scores 0; anything else scores its own norm, far above the bar
    assert oracle.rel_l2(np.zeros(4), np.zeros(4)) == 0.0
    assert oracle.rel_l2(np.array([3.0, 4.0, 0.0]), np.zeros(3)) == 5.0


def test_cosine_closed_forms():
    # parallel, anti-parallel, orthogonal
    assert oracle.cosine(np.array([1.0, 2.0, 2.0]), np.array([2.0, 4.0, 4.0])) == 1.0
    assert oracle.cosine(np.array([1.0, 2.0, 2.0]), np.array([-0.5, -1.0, -1.0])) == -1.0
    assert oracle.cosine(np.array([1.0, 0.0]), np.array([0.0, 3.0])) == 0.0
    # 3-4-5: <[3,4],[4,3]> / 25 = 0.96 (unnormalised: 24)
    assert oracle.cosine(np.array([3.0, 4.0]), np.array([4.0, 3.0])) == pytest.approx(0.96, rel=1e-15)
    # 45 degrees
    assert oracle.cosine(np.array([1.0, 0.0]), np.array([1.0, 1.0])) == pytest.approx(1.0 / math.sqrt(2.0), rel=1e-15)
    # over the whole [T, K] array: rows ([1,0],[0,2]) against ([1,0],[2,0]) ->
    # 1 / (sqrt(5) sqrt(5)) = 0.2 (a mean of per-row cosines would give 0.5)
    assert oracle.cosine(np.array([[1.0, 0.0], [0.0, 2.0]]), np.array([[1.0, 0.0], [2.0, 0.0]])) == \
        pytest.approx(0.2, rel=1e-15)


def test_cosine_invariances_and_zero_vectors():
    rng = np.random.default_rng(6)
    t, r = rng.standard_normal(1000), rng.standard_normal(1000)
    c = oracle.cosine(t, r)
    assert -1.0 <= c <= 1.0
    # scale of either argument and the argument order do not matter
    assert oracle.cosine(5.0 * t, r) == pytest.approx(c, rel=1e-12)
    assert oracle.cosine(r, t) == pytest.approx(c, rel=1e-12)
    # a small perturbation: 1 - cos = |e_perp|^2 / 2 to first order
    e = 1e-3 * rng.standard_normal(1000)
    e_perp = e - (e @ r) / (r @ r) * r
    want = 1.0 - 0.5 * (e_perp @ e_perp) / (r @ r)
    assert oracle.cosine(r + e, r) == pytest.approx(want, abs=1e-9)
    # both all-zero counts as a match; one all-zero is no match
    assert oracle.cosine(np.zeros(3), np.zeros(3)) == 1.0
    assert oracle.cosine(np.zeros(3), np.array([1.0, 2.0, 3.0])) == 0.0


def test_metric_pins_catch_planted_mistakes(monkeypatch):
    real_rel, real_cos = oracle.rel_l2, oracle.cosine

    def squared_rel(t, r):
        return real_rel(t, r) ** 2

    def mean_elementwise_rel(t, r):
        t, r = np.ravel(t).astype(np.float64), np.ravel(r).astype(np.float64)
        nz = r != 0
        return float(np.mean(np.abs(t[nz] - r[nz]) / np.abs(r[nz]))) if nz.any() else float(np.abs(t).sum())

    def unnormalised_cos(t, r):
        return float(np.ravel(t).astype(np.float64) @ np.ravel(r).astype(np.float64))

    def row_mean_cos(t, r):
        t, r = np.atleast_2d(t), np.atleast_2d(r)
        return float(np.mean([real_cos(a, b) for a, b in zip(t, r)]))

    for planted in (squared_rel, mean_elementwise_rel):
        monkeypatch.setattr(oracle, "rel_l2", planted)
        with pytest.raises(AssertionError):
            test_rel_l2_closed_forms()
    monkeypatch.setattr(oracle, "rel_l2", real_rel)
    for planted in (unnormalised_cos, row_mean_cos):
        monkeypatch.setattr(oracle, "cosine", planted)
        with pytest.raises(AssertionError):
            test_cosine_closed_forms()


def test_routing_nan_logits_rank_last():
    # Reading (the pages are silent; finite logits are the precondition): a
    # NaN logit ranks below every number, -inf included, ties to the lower id.
    nan, inf = float("nan"), float("inf")
    row = [nan, 1.0, nan, -inf, 0.5]
    for k, want in ((2, [1, 4]), (3, [1, 4, 3]), (4, [1, 4, 3, 0]), (5, [1, 4, 3, 0, 2])):
        ids, w = oracle.route_topk(np.array([row], np.float32), k, "softmax")
        assert ids[0].tolist() == want
        assert bf.topk_by_argmax(row, k) == want
        # a selected NaN (or -inf next to finite values: exp(-inf) = 0) shapes the weights
        if k == 2:
            assert np.all(np.isfinite(w))
        if k >= 4:
            assert np.all(np.isnan(w))
    # all NaN: ids 0..k-1, weights NaN
    ids, w = oracle.route_topk(np.full((1, 6), np.nan, np.float32), 3, "sigmoid")
    assert ids[0].tolist() == [0, 1, 2] and np.all(np.isnan(w))
    # random rows with NaNs sprinkled in agree with the repeated arg-max
    rng = np.random.default_rng(17)
    for E, k in ((32, 4), (128, 4), (384, 8)):
        logits = (np.round(rng.standard_normal((12, E)) * 4) / 4).astype(np.float32)
        logits[rng.random((12, E)) < 0.2] = np.nan
        logits[3] = np.nan
        ids, _ = oracle.route_topk(logits, k, "softmax")
        for t in range(12):
            assert ids[t].tolist() == bf.topk_by_argmax([float(v) for v in logits[t]], k)
