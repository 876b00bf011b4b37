"""Layer shapes and value distributions of the synthetic workloads.

Each configuration is one expert-parallel slice of an MXFP4 MoE layer as held
by one GPU.  The shapes follow the models the "MXFP4 MoE decode kernels" page
measures (gpt-oss-20b/120b: K = I = 2880, top-4; GLM-5.x: K 6144, top-8 of
256 with sigmoid scoring; Kimi-K2.7: K 7168, I 2048, 48 of 384 experts, top-8).
Real checkpoints are not available, so weights are uniform random E2M1 codes
with E8M0 scales drawn uniformly from a narrow band, and activations and router
logits are Gaussian.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    description: str
    K: int                      # hidden size (reduction of w13, output rows of w2)
    I: int                      # intermediate size per expert
    E_global: int               # experts scored by the router
    E_local: int                # experts held by this slice
    expert_offset: int          # global id of local expert 0
    top_k: int
    scoring: str                # "softmax" | "sigmoid"
    activation: str             # "silu_mul" | "swiglu_oai"
    bias: bool                  # per-row biases b13 [E,2I], b2 [E,K]
    tokens: Tuple[int, ...]     # token counts T per call
    scale_lo: int               # E8M0 scales uniform in [scale_lo, scale_hi]
    scale_hi: int
    logit_std: float = 1.0
    x_std: float = 1.0
    swiglu_alpha: float = 1.702
    swiglu_limit: float = 7.0
    index: int = 0              # seed namespace

    def bytes_per_expert(self) -> int:
        """Packed + scale bytes of one expert (w13 and w2), plus its biases."""
        K, I = self.K, self.I
        w13 = 2 * I * (K // 2) + 2 * I * (K // 32)
        w2 = K * (I // 2) + K * (I // 32)
        b = 2 * (2 * I + K) if self.bias else 0
        return w13 + w2 + b


CONFIGS = {
    "tiny": LayerConfig(
        name="tiny",
        description="tiny MXFP4 MoE: K=I=256, E=8, top-2 softmax, T=4",
        K=256, I=256, E_global=8, E_local=8, expert_offset=0, top_k=2,
        scoring="softmax", activation="silu_mul", bias=False, tokens=(4,),
        scale_lo=118, scale_hi=130, index=1),
    "gptoss20b": LayerConfig(
        name="gptoss20b",
        description="gpt-oss-20b-shaped: K=I=2880, E=32, top-4 softmax, bias, clamped SwiGLU",
        K=2880, I=2880, E_global=32, E_local=32, expert_offset=0, top_k=4,
        scoring="softmax", activation="swiglu_oai", bias=True, tokens=(1, 4, 16, 32),
        scale_lo=115, scale_hi=127, index=2),
    "gptoss120b": LayerConfig(
        name="gptoss120b",
        description="gpt-oss-120b-shaped: K=I=2880, E=128, top-4 softmax, bias, clamped SwiGLU, logits N(0,2)",
        K=2880, I=2880, E_global=128, E_local=128, expert_offset=0, top_k=4,
        scoring="softmax", activation="swiglu_oai", bias=True, tokens=(1, 4, 8, 16, 32),
        scale_lo=115, scale_hi=127, logit_std=2.0, index=3),
    "glm5_ep": LayerConfig(
        name="glm5_ep",
        description="GLM-5.x EP slice: K=6144, I=2048, 32 of 256 experts, top-8 sigmoid, SiLU*up, no bias",
        K=6144, I=2048, E_global=256, E_local=32, expert_offset=0, top_k=8,
        scoring="sigmoid", activation="silu_mul", bias=False, tokens=(1, 8, 32),
        scale_lo=115, scale_hi=127, index=4),
    "widek": LayerConfig(
        name="widek",
        description="wide-K slice: K=7168, I=2048, 48 of 384 experts, top-8 sigmoid, SiLU*up, no bias",
        K=7168, I=2048, E_global=384, E_local=48, expert_offset=0, top_k=8,
        scoring="sigmoid", activation="silu_mul", bias=False, tokens=(32, 256, 2048),
        scale_lo=115, scale_hi=127, index=5),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
