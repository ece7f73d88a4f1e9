"""MI355X (gfx950) sparse MoE expert layer with fused groupwise-affine 4-bit weights.

The compute lives in libmoe_w4.so (hand-written HIP, C ABI in include/moe_w4.h
and include/gdn_scan.h); this package only marshals arguments to it.
"""

from .moe import (  # noqa: F401
    Bank,
    DeviceBank,
    Dims,
    EXPORTED,
    GdnDims,
    LIB_PATH,
    MoeError,
    MoeLayer,
    RouteOut,
    RouteTables,
    STATUS_BAD_INDEX,
    STATUS_BLOCK_OVERFLOW,
    STATUS_NAN_LOGIT,
    gdn_scan,
    gdn_scan_chunked,
    gdn_scan_chunked_ws_bytes,
    lib,
    make_dims,
    moe_abi_version,
    moe_combine,
    moe_w4_ffn_combine,
    moe_grouped_w4_ffn,
    moe_max_blocks,
    moe_route,
    moe_route_no_alloc,
    moe_route_ws_bytes,
    moe_routed_w4_ffn,
    moe_shared_w4_ffn,
    moe_read_probe,
    moe_mfma_probe,
    moe_w4_dequant,
    moe_w4_dequant_packed,
    moe_w4_pack,
    moe_w4_packed_bytes,
    moe_w4_down,
    moe_w4_gate_up,
    strerror,
)

lib()  # load the HIP library now: a missing build is an import error, never a fallback
