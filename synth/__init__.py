"""Seeded synthetic workloads for the Fast-AR codebook decoder.

This package only draws random numbers and lays them out: model shapes,
weights, Slow-AR hidden states, semantic codes, per-request sampling
settings and the caller-side uniforms.  It holds none of the decoder's
arithmetic, so both the oracle and the HIP path can be fed from it without
sharing any computation.
"""
from .inputs import (  # noqa: F401
    ModelShape,
    TINY,
    S2PRO,
    S2PRO_PROJ,
    RAGGED,
    Workload,
    WORKLOADS,
    make_weights,
    make_frames,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    weight_names,
)
