"""MI355X-native layer-end KV-eviction compressor (two-pass blockwise scoring,
top-k selection and retained-cache gather) as a C-ABI HIP library, with a thin
Python binding whose functions carry the C entry points' names."""
from ._lib import (  # noqa: F401
    KVC_ERR_ALIGN, KVC_ERR_HIP, KVC_ERR_INVALID_ARG, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE,
    KVC_SCORE_LOGIT, KVC_SCORE_LOGIT_INT8, KVC_SCORE_SOFTMAX, KVC_FLAG_FUSED_SELECT, kvc_overlap_coefficient,
    KVC_MAX_KV_HEADS, KVC_MAX_POOL, KVC_MAX_ROWS, KVC_OK, LIB_PATH, KvcError, LayerDesc,
    LayerOutputs, PreparedLayer, PreparedSweep, SWEEP_STREAMS, alloc_outputs, alloc_sweep_workspace,
    alloc_workspace, compress_layer, desc_for, kvc_budgets_inverse_stability,
    kvc_compress_layer, kvc_compress_layers, kvc_gather_retained, kvc_retained_offsets, kvc_score_pass1,
    kvc_score_layer, kvc_score_pass2, kvc_select_topk, kvc_strerror, kvc_version, kvc_workspace_size, lib,
    make_desc, kvc_chunk_workspace_size, kvc_evict_chunk, kvc_chunked_workspace_size, kvc_compress_chunked,
    kvc_plan_layer, LayerPlan, kvc_compress_layer_noalloc, KVC_NOALLOC_SCRATCH_BYTES, KVC_SCAN_STREAM, KVC_SCAN_PER_HEAD, KVC_SCAN_LOGIT,
    alloc_arena, PreparedChunked, PrefillDesc, kvc_rmsnorm, kvc_rope_append, kvc_chunk_attention, kvc_swiglu,
)
