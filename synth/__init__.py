"""Seeded synthetic inputs for the decode-time int4 MoE layer.

This package holds only input synthesis (shapes, random draws, storage
layout of the generated weights). It contains none of the layer's
arithmetic: no dequantisation, routing, activation or combine. Both the
fp64 oracle and the HIP path are fed the arrays it produces.
"""
from .configs import Shape, Workload, CONFIGS, shape_of, C0, C1, C2, C3, C4, TINY  # noqa: F401
