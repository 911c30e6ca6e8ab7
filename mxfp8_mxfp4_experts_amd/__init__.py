"""MXFP8 x MXFP4 fused MoE expert layer for AMD Instinct MI355X (gfx950).

The layer is five C calls into ``libmi355moe.so`` (declared in
``include/mi355moe.h``); this package is their thin Python binding plus
``MoELayer``, which issues the calls in order with one workspace (routing,
quantisation and grouping as the one call ``moe_route_quant_permute``; with
given top-k ids, quantisation and grouping as ``moe_quant_permute``).
"""
from ._binding import (  # noqa: F401
    COMBINE_ATOMIC,
    COMBINE_DETERMINISTIC,
    EXPORTS,
    MoEError,
    lib,
    load_library,
    moe_abi_version,
    moe_fc1_situ,
    moe_fc2_combine,
    moe_permute,
    moe_permute_noalloc,
    W13_GATE_UP,
    W13_INTERLEAVED,
    W13_UP_GATE,
    moe_prepack_w13,
    moe_prepack_w13_layout,
    moe_prepack_w2,
    moe_quant_mxfp8,
    moe_quant_permute,
    moe_route,
    moe_route_quant_permute,
    moe_workspace_size,
)
from .layer import MoELayer  # noqa: F401
