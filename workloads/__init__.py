"""Seeded synthetic workloads for the routed-expert MXFP4 MoE decode layer.

This package only draws random numbers and fixes shapes.  It holds none of the
layer's arithmetic (no decoding, routing, activation or rounding rules), so
that the CPU oracle and the HIP path can both take their inputs from it without
sharing any of the method's code.
"""

from .configs import CONFIGS, LayerConfig, get_config
from .generate import (
    LayerWeights,
    LayerInputs,
    make_weights,
    make_inputs,
    make_topk_inputs,
)

__all__ = [
    "CONFIGS",
    "LayerConfig",
    "get_config",
    "LayerWeights",
    "LayerInputs",
    "make_weights",
    "make_inputs",
    "make_topk_inputs",
]
