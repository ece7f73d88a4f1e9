"""Seeded synthetic inputs for the MoE expert layer.

This package only draws numbers: counter-based SplitMix64 streams, uniforms,
Box-Muller normals, round-to-nearest-even conversion to bfloat16, and the
per-configuration recipes (shapes, seeds, distributions).  It contains none of
the layer's arithmetic (no router, no dequantisation, no GEMM), so both the
CPU oracle's tests and the HIP path's tests and benchmark can use it without
sharing any of the method's code.
"""

from .gen import (  # noqa: F401
    GAMMA,
    splitmix64_mix,
    stream_key,
    stream_u64,
    uniform,
    normal,
    f64_to_bf16_bits,
    bf16_bits_to_f32,
    random_bytes,
    make_bank,
    make_router,
    make_zipf_bias,
    make_tokens,
)
from .configs import CONFIGS, LayerShape, FULL_SHAPE, TINY_SHAPE, build_config  # noqa: F401
from .gdn import GDN_CONFIGS, GdnShape, build_gdn_config, make_gdn_inputs  # noqa: F401
