"""Seeded synthetic workloads for the fused MoE layer forward.

This package only draws inputs: shapes, dtypes, value distributions and the
router-load skew of the five benchmark layers.  It holds none of the layer's
arithmetic (no routing, no alignment, no expert math), so both the CPU oracle's
tests and the GPU path can take their inputs from here without sharing any
computation.
"""
from .configs import LAYERS, LayerShape, layer_shape  # noqa: F401
from .gen import Layer, make_bias, make_layer, make_router, make_tokens, make_topk_ids  # noqa: F401
