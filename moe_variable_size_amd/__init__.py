"""MI355X-native MoE variable-size grouped GEMM (HIP, gfx950).

The compute lives in libmoe_vs.so behind the C ABI of include/moe_vs.h; the
names below mirror it.  Importing this package does not load the library; the
first call does, and raises if it has not been built.
"""
from .api import (  # noqa: F401
    MOE_BF16, MOE_F32, MOE_LAYOUT_CONTIGUOUS, MOE_LAYOUT_MASKED, MoEFunction, Schedule,
    grouped_gemm, moe, moe_build_schedule, moe_fused_bwd, moe_fused_bwd_workspace_bytes,
    moe_fused_fwd, moe_schedule_workspace_bytes, moe_tile_map, moe_timing_enable, moe_timing_read,
)

__version__ = "0.1.0"
