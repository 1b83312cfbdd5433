"""HGA routed-attention forward for MI355X (gfx950).

Python binding of the C ABI in include/hga.h; the computation runs in the HIP
kernels of libhga.so (built by ``hierarchical_sparse_attention_hga_amd.build``).
"""
from ._binding import (  # noqa: F401
    EXPORTS, HGA_BF16, HGA_BF16_F32OUT, HGA_ERR_DEVICE, HGA_ERR_INVALID_ARGUMENT, HGA_ERR_UNSUPPORTED,
    HGA_ERR_WORKSPACE, HGA_F32, HGA_OK, HGA_SUMMARY_MEAN, HGA_WS_ATTEND, HGA_WS_ATTEND_TIERED,
    HGA_WS_ATTEND_CACHED, HGA_WS_BACKWARD, HGA_WS_BACKWARD_TIERED, HGA_WS_ROUTE, HGA_TC_GS, HGA_TC_KV, TC_COUNTERS,
    hga_tier_cache, hga_tier_cache_init, hga_tier_cache_min_slots, hga_tier_cache_size, tier_cache, LIB_PATH, HgaError, hga_attend, hga_attend_backward, hga_build_summaries,
    hga_build_summaries_range,
    hga_config, hga_last_error, hga_route, hga_route_attend, hga_route_attend_cached, hga_route_attend_noalloc, hga_status_string, hga_stream_forward,
    hga_tiered, hga_version, hga_workspace_size, load, make_config,
)
