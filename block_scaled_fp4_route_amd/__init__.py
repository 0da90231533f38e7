"""MI355X (gfx950) routed mixture-of-experts FFN over block-scaled FP4 experts.

The compute runs in the HIP library libmoe_fp4.so (C ABI in
include/moe_fp4.h); this package only loads it and marshals arguments.
Importing fails loudly when the library has not been built.
"""
from .binding import (  # noqa: F401
    EXPORTS, FORMATS, LIB_PATH, ExpertTier, MOE_SCALE_CEIL, MOE_SCALE_FLOOR, MOE_ERR_ARG, MOE_ERR_HIP, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_FMT_MXFP4,
    MOE_FMT_NVFP4, MOE_NOALLOC_SCRATCH_BYTES, MOE_MODE_DECODE, MOE_MODE_PREFILL, MOE_MODE_ROUTE, MOE_OK, MOE_OUT_BF16, MOE_OUT_F32, MoeError,
    alloc_workspace, desc, expert_ptr_table, lib, moe_block_bytes, moe_block_layout, moe_dequant_block,
    moe_act_quant_fp8, moe_expert_decode, moe_expert_prefetch, moe_prefetch_sink_bytes, moe_expert_prefill, moe_gemv_fp8, moe_layer_decode, moe_layer_decode_noalloc, moe_route,
    moe_workspace_bytes,
)
