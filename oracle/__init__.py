"""CPU oracle (test infrastructure only; see ``moe_oracle`` for the rules of use)."""

from .moe_oracle import (  # noqa: F401
    E2M1_MAGNITUDE,
    SIGMOID,
    SILU_MUL,
    SOFTMAX,
    SWIGLU_OAI,
    activation,
    bf16_bits_to_float,
    bucket_routes,
    cosine,
    dequantize,
    e2m1_to_float,
    e8m0_to_float,
    moe_forward,
    moe_forward_cfg,
    rel_l2,
    round_to_bf16,
    route_topk,
    tile16,
    unpack_codes,
    untile16,
)
