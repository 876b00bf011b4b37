"""Seeded generators for layer weights and per-call inputs.

Every array comes from numpy's ``Generator(PCG64(seed))`` drawn in a fixed
order, so the CPU oracle and the device path receive byte-identical inputs.

* weights, seed ``1000*index + replica``: w13 packed bytes, w13 scales, w2
  packed bytes, w2 scales, then (if the layer has them) b13 and b2.
  Packed bytes are uniform over 0..255, i.e. both E2M1 codes of a byte are
  uniform over the 16 codes; scales are uniform integers in
  ``[scale_lo, scale_hi]``; biases are N(0,1) cast to bf16.
* inputs, seed ``1000*index + 100 + 10*t_index + call``: router logits
  N(0, logit_std) in fp32, then x = N(0, x_std) cast to bf16.

bf16 values are carried as their raw 16-bit patterns (``uint16``).  The
fp32 -> bf16 cast of the Gaussian draws is torch's round-to-nearest-even cast;
it only shapes the input distribution.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerConfig


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class LayerWeights:
    w13_packed: np.ndarray            # u8 [E_local, 2I, K/2]
    w13_scales: np.ndarray            # u8 [E_local, 2I, K/32]
    w2_packed: np.ndarray             # u8 [E_local, K, I/2]
    w2_scales: np.ndarray             # u8 [E_local, K, I/32]
    b13: Optional[np.ndarray] = None  # bf16 bits u16 [E_local, 2I]
    b2: Optional[np.ndarray] = None   # bf16 bits u16 [E_local, K]


@dataclass
class LayerInputs:
    x: np.ndarray                     # bf16 bits u16 [T, K]
    logits: Optional[np.ndarray]      # f32 [T, E_global], or None in ids mode
    topk_ids: Optional[np.ndarray] = None      # i32 [T, top_k]
    topk_weights: Optional[np.ndarray] = None  # f32 [T, top_k]


def make_weights(cfg: LayerConfig, replica: int = 0, E_local: Optional[int] = None) -> LayerWeights:
    E = cfg.E_local if E_local is None else E_local
    K, I = cfg.K, cfg.I
    rng = _rng(1000 * cfg.index + replica)
    w13p = rng.integers(0, 256, size=(E, 2 * I, K // 2), dtype=np.uint8)
    w13s = rng.integers(cfg.scale_lo, cfg.scale_hi + 1, size=(E, 2 * I, K // 32), dtype=np.uint8)
    w2p = rng.integers(0, 256, size=(E, K, I // 2), dtype=np.uint8)
    w2s = rng.integers(cfg.scale_lo, cfg.scale_hi + 1, size=(E, K, I // 32), dtype=np.uint8)
    b13 = b2 = None
    if cfg.bias:
        b13 = _to_bf16_bits(rng.standard_normal((E, 2 * I), dtype=np.float32))
        b2 = _to_bf16_bits(rng.standard_normal((E, K), dtype=np.float32))
    return LayerWeights(w13p, w13s, w2p, w2s, b13, b2)


def make_inputs(cfg: LayerConfig, T: int, call: int = 0, t_index: Optional[int] = None,
                x_scale: float = 1.0, all_local_boost: float = 0.0) -> LayerInputs:
    """Router-logits mode inputs for one call of T tokens.

    ``x_scale`` multiplies the activation standard deviation (4 gives the
    RMS-4 activations that drive the SwiGLU clamps).  ``all_local_boost`` is
    added to the logits of the slice's own experts so that every route lands
    locally (the "all local" routing of the per-call tables).
    """
    if t_index is None:
        t_index = cfg.tokens.index(T) if T in cfg.tokens else 9
    rng = _rng(1000 * cfg.index + 100 + 10 * t_index + call)
    logits = (rng.standard_normal((T, cfg.E_global), dtype=np.float32) * np.float32(cfg.logit_std))
    if all_local_boost:
        lo, hi = cfg.expert_offset, cfg.expert_offset + cfg.E_local
        logits[:, lo:hi] += np.float32(all_local_boost)
    x = _to_bf16_bits(rng.standard_normal((T, cfg.K), dtype=np.float32) * np.float32(cfg.x_std * x_scale))
    return LayerInputs(x=x, logits=np.ascontiguousarray(logits, dtype=np.float32))


def make_topk_inputs(cfg: LayerConfig, T: int, seed: int, pad_fraction: float = 0.0,
                     x_scale: float = 1.0) -> LayerInputs:
    """Precomputed-routing inputs: distinct random ids per token, positive weights.

    A fraction ``pad_fraction`` of the slots is set to -1 (padding); ids
    outside the local slice occur naturally when E_local < E_global.
    """
    rng = _rng(seed)
    ids = np.empty((T, cfg.top_k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(cfg.E_global, size=cfg.top_k, replace=False)
    if pad_fraction > 0:
        ids[rng.random(ids.shape) < pad_fraction] = -1
    w = rng.random((T, cfg.top_k), dtype=np.float32) + np.float32(0.05)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    x = _to_bf16_bits(rng.standard_normal((T, cfg.K), dtype=np.float32) * np.float32(cfg.x_std * x_scale))
    return LayerInputs(x=x, logits=None, topk_ids=ids, topk_weights=w)
