"""CPU oracle for the MoE expert layer (test infrastructure only).

A plain, slow float64 C++ implementation (``moe_oracle.cpp``) behind ctypes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP product path never does, and the two share no code.
"""

from .api import (  # noqa: F401
    build,
    lib_path,
    load,
    router_logits,
    router_logits_f64,
    topk,
    route_tables,
    max_blocks,
    block_map,
    dequant,
    f32_to_bf16,
    expert_ffn,
    moe_layer,
    route,
    relative_error,
    relative_error_elementwise,
)
from .gdn import gated_delta_scan  # noqa: F401
