"""libmiattn: fused exact attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmiattn.so`` (C ABI in
include/libmiattn.h); this package is its ctypes binding.  Build it with
``python -m tiled_attention_fa_amd.build``.
"""
from .binding import (  # noqa: F401
    FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_PARAM,
    FA_ERR_WORKSPACE, FA_ERR_LAUNCH, FA_ERR_SCRATCH, FA_NOALLOC_SCRATCH_BYTES, FA_BF16, FA_F32, FA_BWD_DELTA, FA_BWD_DKDV, FA_BWD_DQ,
    MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT,
    MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_LOCAL_BOOST, MOD_REL_BIAS,
    TILE_EMPTY, TILE_PARTIAL, TILE_FULL, BLOCK, EXPORTED,
    FaMaskParams, FaModParams, FaBlockMask, FaError, BlockMask,
    lib, fa_fwd, fa_bwd, fa_bwd_phase, fa_bwd_noalloc, fa_block_mask_build, fa_bwd_workspace_bytes,
    fa_bwd_ds_workspace_bytes,
    fa_bwd_rel_bias_workspace_bytes, fa_block_mask_bytes, fa_fwd_kv_step,
    fa_status_str, fa_version, default_scale, build_block_mask, forward, backward, attention,
    FP8_BLOCK, quantize_fp8, forward_fp8, FA_WORK_QUEUE_INTS, new_work_queue,
    FA_WG_TRACE_WORDS, new_wg_trace, decode_wg_trace,
)
