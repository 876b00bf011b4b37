"""CPU oracle of the routed-expert MXFP4 MoE decode layer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``.  The product (the HIP library and its Python binding) never does,
and nothing here imports the product: both sides take their inputs from the
seeded ``workloads`` generators and share no other code.

It is deliberately plain: every local expert that receives a route is fully
dequantised to a dense matrix, then multiplied with a library matmul; routing
is a full sort; bucketing is a stable sort.  No blocking, fusion or reordering
beyond that.

Sources (page title, then section):

* "GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2", What was built, Byte-exact
  repack: OCP MXFP4 is E2M1 values stored low nibble first, E8M0 scales,
  blocks of 32.  Same page, Why it needed a port, item 1: each expert's fused
  w13 rows are [gate; up]; item 2: experts are sliced by expert-parallel rank;
  item 4: routing ids are int32.  Same page, MXFP4 encoder: E2M1 saturates at 6.
* "MXFP4 MoE decode kernels", The bottleneck: 4-bit E2M1 values, two per byte,
  one E8M0 scale per 32 values.  Design, Read the served layout: w13 u8
  [E, 2I, K/2], s13 u8 [E, 2I, K/32], w2 u8 [E, K, I/2], s2 u8 [E, K, I/32].
  Design, Fused epilogues: bias added in fp32, SwiGLU-OAI = gate capped at the
  limit, up clamped to +-limit, gate*sigmoid(1.702*gate)*(up+1); the w2 stage
  adds the routing-weighted bias once per route and keeps fp32 per-token sums.
  Design, Routing inside the kernel: routes are counting-sorted by local expert,
  routes to other ranks are skipped.  Beyond gpt-oss: the SiLU form without
  bias for [gate; up] rows.  Parity: the reference is CPU fp32 with dequantised
  weights and a bf16 intermediate, rounded to bf16 once.
* "GLM-5.3-Flash on Gaudi 2", Why (model table): top-8 sigmoid scoring.

Readings where the pages are silent:

* E2M1 magnitudes are the OCP table {0, 0.5, 1, 1.5, 2, 3, 4, 6}, bit 3 the
  sign; code 8 decodes to -0.0.
* E8M0 byte s is 2**(s - 127); s = 255 is NaN.  s = 0 gives the fp32
  subnormal 2**-127.  Products overflow to +-inf as IEEE says.
* top-k order: logit descending, ties to the lower expert id, selection on the
  raw logits.  Softmax weights are the softmax of the k selected logits;
  sigmoid weights are sigmoid(logit) renormalised over the k selected.
* a route r = t*top_k + j is local when its global id lies in
  [expert_offset, expert_offset + E_local); weights are not renormalised over
  the local subset; in ids mode the given weights are used as they are.
* the bf16 rounding is round-to-nearest-even.

MXFP4 encoder (``encode_mxfp4``): "GLM-5.2 and GLM-5.3 (744B) in MXFP4 on
Gaudi 2", What was built, MXFP4 encoder: the OCP shared exponent is
floor(log2(amax)) - 2 (values above 6 * 2^X clamp); Quark bumps the exponent
when amax / 2^X >= 7.  Readings where the page is silent: elements round to
the nearest E2M1 value with ties to the even code (round-to-nearest-even,
saturating at 6); the sign bit is the input's sign bit (a negative value that
rounds to zero gives code 8, -0); amax = 0 gives exponent -127 (scale byte 0);
the exponent is clipped to [-127, 127], so scale byte 255 (NaN) never occurs.

Gate/up row order (``w13_order``): "MXFP4 MoE decode kernels", Beyond
gpt-oss, lists a w13 kernel for interleaved gate/up rows next to the
[gate; up] one, and Design, Read the served layout, describes gpt-oss's
served w13 as interleaved (the GLM page's item 1 says gpt-oss's own loader
undoes that).  Reading: interleaved means row 2n is gate row n and row 2n + 1
is up row n, with b13 and the scale rows in the same order; the activation is
chosen independently of the order.

Per-route output (``route_outputs``): the same page's Beyond gpt-oss lists a
down kernel that writes one output row per route for models that apply a
per-route operation before the token sum.  Reading: row r = t*k + j holds
a W2^T (+ b2) in fp32 for a local route, without the routing weight, and
zeros for a route outside the local slice.

The tiled weight layout (``tile16``) is this library's own storage order, not
the pages': the pages' kernels read the served row layout and name a repack
as the next step they chose not to take, to keep one copy of the experts.
Here the repack is an in-place permutation, so there is still one copy.

Precision: ``dtype=np.float32`` (default) is the pages' parity reference.
``dtype=np.float64`` runs the same steps in fp64 to bound the oracle's own
rounding.

Parity pins: every function below is pinned by ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` and ``tests/test_oracle_layer.py``.  The only
unpinned item is the pages' own real-weight rel_l2 table, which needs
checkpoints that are not available ("parity unpinned", context only).
"""

from __future__ import annotations

import numpy as np

# OCP MXFP4 element: E2M1 magnitudes indexed by the low three code bits.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)

MX_BLOCK = 32  # values that share one E8M0 scale

SOFTMAX = "softmax"
SIGMOID = "sigmoid"
SILU_MUL = "silu_mul"
SWIGLU_OAI = "swiglu_oai"
GATE_UP = "gate_up"           # w13 rows [gate; up]
INTERLEAVED = "interleaved"   # w13 row 2n gate n, row 2n + 1 up n


# --------------------------------------------------------------------------
# MXFP4 decoding
# --------------------------------------------------------------------------

def e2m1_to_float(codes: np.ndarray) -> np.ndarray:
    """E2M1 code (0..15) -> float32 value; bit 3 is the sign, code 8 is -0.0."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDE[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag).astype(np.float32)


def e8m0_to_float(s: np.ndarray) -> np.ndarray:
    """E8M0 scale byte -> float32 2**(s - 127); 255 is NaN."""
    s = np.asarray(s).astype(np.int32)
    out = np.ldexp(np.float32(1.0), s - 127).astype(np.float32)
    return np.where(s == 255, np.float32(np.nan), out).astype(np.float32)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., C/2] -> E2M1 codes [..., C]; element 2c is the low nibble of byte c."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    return codes


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed MXFP4 rows [..., C/2] with scales [..., C/32] -> float32 [..., C].

    Value (row n, column c) = E2M1(code of column c) * E8M0(scales[n, c // 32]).
    The product is exact in fp32 except where it overflows.
    """
    values = e2m1_to_float(unpack_codes(packed))
    scale = np.repeat(e8m0_to_float(scales), MX_BLOCK, axis=-1)
    if scale.shape != values.shape:
        raise ValueError(f"scales {scales.shape} do not match packed {packed.shape}")
    with np.errstate(over="ignore", invalid="ignore"):
        return (values * scale).astype(np.float32)


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# MXFP4 encoder
# --------------------------------------------------------------------------

OCP = "ocp"
QUARK = "quark"


def round_to_e2m1(a: np.ndarray) -> np.ndarray:
    """Non-negative float64 -> E2M1 magnitude code 0..7: the nearest grid value,
    ties to the even code (the even codes are the grid values with mantissa 0)."""
    a = np.asarray(a, dtype=np.float64)
    dist = np.abs(a[..., None] - E2M1_MAGNITUDE.astype(np.float64))
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    # among the nearest codes prefer an even one; there are at most two
    even = tied & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, tied)
    return np.argmax(pick, axis=-1).astype(np.uint8)


def encode_mxfp4(values: np.ndarray, rule: str = QUARK):
    """float32/bfloat16-valued array [..., cols] (cols % 32 == 0) -> (packed
    uint8 [..., cols/2], scales uint8 [..., cols/32]).

    Per block of 32: X = floor(log2(amax)) - 2 from the binary exponent of
    amax (exact), plus one under the Quark rule when amax / 2^X >= 7; scale
    byte X + 127; code = sign bit | E2M1 round-to-nearest-even of v / 2^X.
    """
    v = np.asarray(values, dtype=np.float64)
    *lead, cols = v.shape
    assert cols % MX_BLOCK == 0
    b = v.reshape(*lead, cols // MX_BLOCK, MX_BLOCK)
    amax = np.abs(b).max(axis=-1)
    _, e = np.frexp(amax)                       # amax = m * 2^e, 0.5 <= m < 1
    x = e.astype(np.int64) - 1 - 2
    if rule == QUARK:
        x = np.where(np.ldexp(amax, -x) >= 7.0, x + 1, x)
    elif rule != OCP:
        raise ValueError(rule)
    x = np.where(amax == 0, -127, x)
    x = np.clip(x, -127, 127)
    y = np.ldexp(b, -x[..., None])              # exact: a power-of-two scaling
    codes = round_to_e2m1(np.abs(y)) | np.where(np.signbit(y), 8, 0).astype(np.uint8)
    codes = codes.reshape(*lead, cols)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (x + 127).astype(np.uint8)
    return packed, scales


# --------------------------------------------------------------------------
# tiled weight layout
# --------------------------------------------------------------------------

TILE_ROWS = 16    # rows per tile group
PIECE_BYTES = 16  # one MX block of packed codes


def tile16(packed: np.ndarray) -> np.ndarray:
    """Row layout -> tiled layout of packed MXFP4 rows ``[..., rows, cols/2]``.

    In every group of 16 consecutive rows, the 16-byte blocks are stored
    block-major: block b of row r of the group lands at byte 256*b + 16*r of
    the group.  Rows must be a multiple of 16.  A pure byte permutation.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    *lead, rows, rb = packed.shape
    assert rows % TILE_ROWS == 0 and rb % PIECE_BYTES == 0
    g = packed.reshape(*lead, rows // TILE_ROWS, TILE_ROWS, rb // PIECE_BYTES, PIECE_BYTES)
    return np.ascontiguousarray(np.swapaxes(g, -3, -2)).reshape(packed.shape)


def untile16(tiled: np.ndarray) -> np.ndarray:
    """Inverse of ``tile16``."""
    tiled = np.asarray(tiled, dtype=np.uint8)
    *lead, rows, rb = tiled.shape
    assert rows % TILE_ROWS == 0 and rb % PIECE_BYTES == 0
    g = tiled.reshape(*lead, rows // TILE_ROWS, rb // PIECE_BYTES, TILE_ROWS, PIECE_BYTES)
    return np.ascontiguousarray(np.swapaxes(g, -3, -2)).reshape(tiled.shape)


def unpack_bf16(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The prefill unpack ("MXFP4 MoE decode kernels", Prefill: unpack once,
    then the stock op): dequantised values as bf16 bit patterns (uint16).

    An E2M1 value times a power of two has at most two significant bits and
    bf16 keeps fp32's exponent range, so every finite product is a bf16 value:
    the pattern is the upper half of the fp32 dequantisation, exactly.  A NaN
    scale (byte 255) gives a NaN pattern.
    """
    f = dequantize(packed, scales)
    bits = f.view(np.uint32)
    finite = ~np.isnan(f)
    if np.any((bits[finite] & 0xFFFF) != 0):
        raise AssertionError("a dequantised value is not a bf16 value")
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Raw bf16 patterns (uint16) -> float32 (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even; returns the same dtype.

    Works from the float64 value: the quantum is 2**(e - 8) for a value in
    [2**(e-1), 2**e) (8 significant bits), never below the bf16 subnormal
    quantum 2**-133; results beyond the largest bf16 become +-inf.
    """
    v = np.asarray(v)
    out_dtype = v.dtype if v.dtype in (np.float32, np.float64) else np.float64
    x = v.astype(np.float64)
    res = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133).astype(np.float64)
    r = np.rint(np.ldexp(xf, (-q).astype(np.int64))) * np.ldexp(1.0, q.astype(np.int64))
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    res[finite] = r
    return res.astype(out_dtype)


# --------------------------------------------------------------------------
# routing and bucketing
# --------------------------------------------------------------------------

def route_topk(logits: np.ndarray, top_k: int, scoring: str, dtype=np.float32):
    """Router logits [T, E] -> (ids int32 [T, k], weights [T, k]).

    Experts are ordered by (logit descending, id ascending) with a full sort
    and the first k are taken.  Softmax weights: exp(l_j - l_0) / sum over the
    k selected; sigmoid weights: sigmoid(l_j) / sum over the k selected.

    Finite logits are the layer's precondition.  Reading for a NaN logit (the
    pages are silent): it ranks below every number, -inf included, and NaNs
    among themselves go to the lower id; the weights then follow the same
    arithmetic (a selected NaN makes every weight of the token NaN).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k out of range")
    ids = np.empty((T, top_k), dtype=np.int32)
    weights = np.empty((T, top_k), dtype=dtype)
    expert = np.arange(E)
    for t in range(T):
        nan = np.isnan(logits[t])
        neg = np.where(nan, np.float32(0.0), -logits[t])
        order = np.lexsort((expert, neg, nan))  # keys: NaN last, then -logit, then id
        sel = order[:top_k]
        ids[t] = sel
        l = logits[t, sel].astype(dtype)
        with np.errstate(invalid="ignore", over="ignore"):
            if scoring == SOFTMAX:
                p = np.exp(l - l[0])
            elif scoring == SIGMOID:
                p = np.asarray(1.0, dtype) / (np.asarray(1.0, dtype) + np.exp(-l))
            else:
                raise ValueError(f"unknown scoring {scoring!r}")
            weights[t] = p / p.sum(dtype=dtype)
    return ids, weights


def bucket_routes(ids: np.ndarray, E_local: int, expert_offset: int):
    """Stable counting sort of the local routes by local expert.

    Route r = t*k + j (row-major over ids) is local when
    expert_offset <= ids[t, j] < expert_offset + E_local.
    Returns counts int32 [E_local], offsets int32 [E_local + 1] (exclusive
    prefix sum) and routes int32 [R_local], the local route indices grouped by
    expert, ascending r inside each group.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    is_local = (flat >= expert_offset) & (flat < expert_offset + E_local)
    r_local = np.nonzero(is_local)[0]
    e_local = flat[r_local] - expert_offset
    routes = r_local[np.argsort(e_local, kind="stable")].astype(np.int32)
    counts = np.bincount(e_local, minlength=E_local).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return counts, offsets, routes


# --------------------------------------------------------------------------
# activation
# --------------------------------------------------------------------------

def activation(gate: np.ndarray, up: np.ndarray, kind: str, alpha: float = 1.702,
               limit: float = 7.0) -> np.ndarray:
    """SILU_MUL: gate*sigmoid(gate)*up.
    SWIGLU_OAI: g = min(gate, limit), u = clip(up, -limit, limit),
    g*sigmoid(alpha*g)*(u + 1)."""
    dt = gate.dtype
    one = np.asarray(1.0, dt)
    with np.errstate(over="ignore"):
        if kind == SILU_MUL:
            return gate * (one / (one + np.exp(-gate))) * up
        if kind == SWIGLU_OAI:
            L = np.asarray(limit, dt)
            g = np.minimum(gate, L)
            u = np.clip(up, -L, L)
            return g * (one / (one + np.exp(-np.asarray(alpha, dt) * g))) * (u + one)
    raise ValueError(f"unknown activation {kind!r}")


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def moe_forward(*, x_bits, w13_packed, w13_scales, w2_packed, w2_scales, K, I,
                E_global, E_local, top_k, expert_offset=0, scoring=SOFTMAX,
                activation_kind=SILU_MUL, swiglu_alpha=1.702, swiglu_limit=7.0,
                logits=None, topk_ids=None, topk_weights=None, b13=None, b2=None,
                dtype=np.float32, round_intermediate=True, experts_cache=None, w13_order=GATE_UP):
    """One MoE layer call on an expert-parallel slice.

    Inputs are the raw arrays: x as bf16 bits [T, K]; either router logits
    [T, E_global] or (topk_ids [T, k], topk_weights [T, k]); packed weights and
    scales in the served layout; optional bf16-bit biases.

    Steps: (1) x to fp32; (2) route (or take the given ids and weights);
    (3) bucket the local routes; (4) per local expert with routes: dequantise
    w13, H = X_e W13^T (+ b13), activation on the gate and up columns
    ([gate; up] halves, or even and odd columns for ``w13_order``
    "interleaved"), round to bf16; dequantise w2, O = A_e W2^T (+ b2);
    (5) y[t] = sum over token t's local routes j (ascending j) of
    w[t, j] * O[route].

    Returns a dict with y [T, K] and every intermediate: ids, weights, counts,
    offsets, routes, h [R_local, 2I] and a [R_local, I] in route order, o
    [R_local, K].
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    if x_bits.shape != (T, K) or K % MX_BLOCK or I % MX_BLOCK:
        raise ValueError("bad shapes")
    if expert_offset < 0 or expert_offset + E_local > E_global:
        raise ValueError("local slice outside the global experts")
    if w13_order not in (GATE_UP, INTERLEAVED):
        raise ValueError(w13_order)
    x = bf16_bits_to_float(x_bits).astype(dtype)
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")

    if logits is not None:
        if topk_ids is not None or topk_weights is not None:
            raise ValueError("give router logits or top-k ids+weights, not both")
        ids, weights = route_topk(logits, top_k, scoring, dtype=dtype)
    else:
        ids = np.asarray(topk_ids, dtype=np.int32).reshape(T, top_k)
        weights = np.asarray(topk_weights, dtype=np.float32).reshape(T, top_k).astype(dtype)

    counts, offsets, routes = bucket_routes(ids, E_local, expert_offset)
    R = int(offsets[-1])
    h_all = np.zeros((R, 2 * I), dtype=dtype)
    a_all = np.zeros((R, I), dtype=dtype)
    o_all = np.zeros((R, K), dtype=dtype)

    for e in range(E_local):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        tokens = routes[lo:hi] // top_k
        if experts_cache is not None and ("w13", e) in experts_cache:
            w13 = experts_cache[("w13", e)]
            w2 = experts_cache[("w2", e)]
        else:
            w13 = dequantize(w13_packed[e], w13_scales[e]).astype(dtype)   # [2I, K]
            w2 = dequantize(w2_packed[e], w2_scales[e]).astype(dtype)      # [K, I]
            if experts_cache is not None:
                experts_cache[("w13", e)] = w13
                experts_cache[("w2", e)] = w2
        with np.errstate(over="ignore", invalid="ignore"):
            h = x[tokens] @ w13.T
            if b13 is not None:
                h = h + bf16_bits_to_float(b13[e]).astype(dtype)
            if w13_order == GATE_UP:
                gate, up = h[:, :I], h[:, I:]
            else:
                gate, up = h[:, 0::2], h[:, 1::2]
            act = activation(gate, up, activation_kind, swiglu_alpha, swiglu_limit)
            a = round_to_bf16(act) if round_intermediate else act
            o = a @ w2.T
            if b2 is not None:
                o = o + bf16_bits_to_float(b2[e]).astype(dtype)
        h_all[lo:hi] = h
        a_all[lo:hi] = a
        o_all[lo:hi] = o

    position = np.full(T * top_k, -1, dtype=np.int64)
    position[routes] = np.arange(R)
    y = np.zeros((T, K), dtype=dtype)
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(T):
            for j in range(top_k):
                p = position[t * top_k + j]
                if p >= 0:
                    y[t] += weights[t, j] * o_all[p]

    return {"y": y, "ids": ids, "weights": weights, "counts": counts, "offsets": offsets,
            "routes": routes, "h": h_all, "a": a_all, "o": o_all}


def route_outputs(result: dict, T: int, top_k: int) -> np.ndarray:
    """Per-route down-projection rows [T * top_k, K] from a ``moe_forward``
    result: row r = t * top_k + j is O of route r (a W2^T + b2, no routing
    weight) when the route is local, else zeros."""
    o = result["o"]
    out = np.zeros((T * top_k, o.shape[1]), dtype=o.dtype)
    out[result["routes"]] = o
    return out


def moe_forward_cfg(cfg, weights, inputs, **kw):
    """moe_forward with the shape and routing fields taken from a layer config."""
    return moe_forward(
        x_bits=inputs.x, logits=inputs.logits, topk_ids=inputs.topk_ids,
        topk_weights=inputs.topk_weights,
        w13_packed=weights.w13_packed, w13_scales=weights.w13_scales,
        w2_packed=weights.w2_packed, w2_scales=weights.w2_scales,
        b13=weights.b13, b2=weights.b2, K=cfg.K, I=cfg.I, E_global=cfg.E_global,
        E_local=weights.w13_packed.shape[0], top_k=cfg.top_k,
        expert_offset=kw.pop("expert_offset", cfg.expert_offset), scoring=cfg.scoring,
        activation_kind=cfg.activation, swiglu_alpha=cfg.swiglu_alpha,
        swiglu_limit=cfg.swiglu_limit, **kw)


def rel_l2(test: np.ndarray, ref: np.ndarray) -> float:
    """||test - ref||_2 / ||ref||_2 over the flattened arrays (fp64).

    "MXFP4 MoE decode kernels", Parity, reports rel_l2 without defining it;
    the reading is the relative Euclidean error over the whole output.  An
    all-zero reference scores the output's own norm (0 only for an all-zero
    output)."""
    t = np.asarray(test, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(r)
    return float(np.linalg.norm(t - r) / den) if den > 0 else float(np.linalg.norm(t))


def cosine(test: np.ndarray, ref: np.ndarray) -> float:
    """<test, ref> / (||test|| ||ref||) over the flattened arrays (fp64); two
    all-zero arrays count as a match (1.0), one all-zero array as none (0.0)."""
    t = np.asarray(test, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(t) * np.linalg.norm(r)
    return float(t @ r / den) if den > 0 else (1.0 if not t.any() and not r.any() else 0.0)
