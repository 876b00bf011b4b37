"""Brute-force scalar evaluation of the MoE layer, in fp64, for tiny shapes.

TEST INFRASTRUCTURE, used only to pin ``oracle.moe_oracle``.  It shares no
code with ``moe_oracle``: it decodes each weight on the fly from its bit
fields (sign, 2-bit exponent with bias 1, 1-bit mantissa; E8M0 as a power of
two), selects the top-k by repeated arg-max instead of a sort, walks tokens
and routes directly without any permutation, and accumulates every dot
product in a Python float (fp64).  Pure-Python loops: keep K, I <= ~128.

It does not round the intermediate to bf16; compare it with the oracle run
with ``round_intermediate=False``.
"""

from __future__ import annotations

import math


def e2m1_from_bits(code: int) -> float:
    """E2M1 from its bit fields: value = (-1)^s * 2^(e-1) * (1 + m/2) for e > 0,
    (-1)^s * m/2 for e = 0 (subnormal)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    v = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m * 0.5)
    return -v if s else v


def e8m0_from_bits(s: int) -> float:
    return math.nan if s == 255 else math.ldexp(1.0, s - 127)


def weight(packed, scales, e: int, row: int, col: int) -> float:
    byte = int(packed[e][row][col // 2])
    code = (byte & 0x0F) if col % 2 == 0 else (byte >> 4)
    return e2m1_from_bits(code) * e8m0_from_bits(int(scales[e][row][col // 32]))


def bf16_value(bits: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _sigmoid(v: float) -> float:
    if v >= 0:
        return 1.0 / (1.0 + math.exp(-v))
    z = math.exp(v)
    return z / (1.0 + z)


def topk_by_argmax(row, k):
    """Repeated arg-max: the largest remaining logit, ties to the lower id; a
    NaN loses to every number and, among NaNs, the lower id comes first."""
    def beats(v, b):
        if math.isnan(v):
            return False
        return math.isnan(b) or v > b

    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or beats(v, row[best]):
                best = e
        chosen.append(best)
    return chosen


def moe_bruteforce(*, x_bits, w13_packed, w13_scales, w2_packed, w2_scales, K, I,
                   E_global, E_local, top_k, expert_offset=0, scoring="softmax",
                   activation_kind="silu_mul", swiglu_alpha=1.702, swiglu_limit=7.0,
                   logits=None, topk_ids=None, topk_weights=None, b13=None, b2=None,
                   w13_order="gate_up", per_route=False):
    """y [T][K] as nested lists; with per_route, also the per-route rows
    {t * top_k + j: [K]} (a W2^T + b2 of each local route, no routing weight)."""
    T = len(x_bits)
    rows = {}
    x = [[bf16_value(x_bits[t][c]) for c in range(K)] for t in range(T)]
    y = [[0.0] * K for _ in range(T)]
    for t in range(T):
        if logits is not None:
            row = [float(v) for v in logits[t]]
            ids = topk_by_argmax(row, top_k)
            if scoring == "softmax":
                z = [math.exp(row[i] - row[ids[0]]) for i in ids]
            else:
                z = [_sigmoid(row[i]) for i in ids]
            s = sum(z)
            w = [v / s for v in z]
        else:
            ids = [int(v) for v in topk_ids[t]]
            w = [float(v) for v in topk_weights[t]]
        for j in range(top_k):
            if not (expert_offset <= ids[j] < expert_offset + E_local):
                continue
            e = ids[j] - expert_offset
            h = []
            for n in range(2 * I):
                acc = 0.0
                for c in range(K):
                    acc += x[t][c] * weight(w13_packed, w13_scales, e, n, c)
                if b13 is not None:
                    acc += bf16_value(b13[e][n])
                h.append(acc)
            a = []
            for n in range(I):
                if w13_order == "gate_up":
                    g, u = h[n], h[I + n]
                else:                       # interleaved: gate row n is row 2n, up row n is row 2n + 1
                    g, u = h[2 * n], h[2 * n + 1]
                if activation_kind == "silu_mul":
                    a.append(g * _sigmoid(g) * u)
                else:
                    g2 = min(g, swiglu_limit)
                    u2 = max(-swiglu_limit, min(u, swiglu_limit))
                    a.append(g2 * _sigmoid(swiglu_alpha * g2) * (u2 + 1.0))
            for kk in range(K):
                acc = 0.0
                for n in range(I):
                    acc += weight(w2_packed, w2_scales, e, kk, n) * a[n]
                if b2 is not None:
                    acc += bf16_value(b2[e][kk])
                y[t][kk] += w[j] * acc
                rows.setdefault(t * top_k + j, [0.0] * K)[kk] = acc
    return (y, rows) if per_route else y
