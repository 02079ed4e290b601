"""MI355X-native fused multi-tenant LoRA layer over an FP8 / MXFP4 base GEMM.

The compute lives in the HIP library ``liblora_lowp.so`` (gfx950 kernels behind the C
ABI in ``include/lora_lowp.h``); :mod:`precision_gemm_amd.ops` is its Python binding on
torch device tensors.  Build the library with ``python -m precision_gemm_amd.build``.
"""

from .ops import (  # noqa: F401
    LORA_ACT_BF16, LORA_BUILD_SEGMENTS, LORA_FUSE_SHRINK, LORA_W_FP8_E4M3, LORA_W_MXFP4_E2M1, Adapters, LowpWeight, Segments,
    BackwardAdapters, Grads, a_rows, alloc_grads, grads_from, adapter_rows, lora_backward, pack_adapters_bwd, pack_weight_t, alloc_workspace, build_segments, pack_adapter, rank_pad, empty_segments, expand, gemm_lowp_lora_epilogue, gemm_lowp_lora_epilogue_noalloc, merged_layer, pack_weight, plan_info,
    quant_act_mxfp8, shrink, shrink_config_info, shrink_configured, version, workspace_bytes, workspace_segment_error, workspace_status,
)
