"""MI355X-native decode hot path of lookahead block scoring with sparse KV
staging (OasisKV, arXiv 2608.08097): block scoring from min/max key summaries,
top-K selection under a token budget, fetch-capped staging from a pinned host
pool into an HBM working set, and sparse GQA decode attention, as HIP kernels
for gfx950 behind the C ABI of liboasis.so (include/oasis.h)."""
from .binding import (  # noqa: F401
    OASIS_COPY_DMA, OASIS_COPY_KERNEL, OASIS_COPY_MIXED, OASIS_EHIP, OASIS_EINVAL, OASIS_ENOSPACE, OASIS_EUNSUPPORTED,
    OASIS_OK, OasisError, dims, library, oasis_append_kv, oasis_attn_launch_shape, oasis_attn_num_splits,
    oasis_block_attention_mass, oasis_block_mass_workspace_bytes,
    oasis_topk_overlap, oasis_attn_workspace_bytes,
    oasis_build_summaries, oasis_fetch_cap_blocks, oasis_host_empty, oasis_last_error, oasis_layer_buffers, oasis_lookahead_attn,
    oasis_lookahead_attn_workspace_bytes,
    oasis_pipeline_copy_host_seconds, oasis_pipeline_create, oasis_pipeline_desc, oasis_pipeline_destroy,
    oasis_pipeline_drain, oasis_pipeline_issue_threads, oasis_pipeline_layer_step, oasis_pipeline_stream,
    oasis_pipeline_timing,
    oasis_pipeline_timing_read, oasis_pipeline_timing_values, oasis_score_blocks, oasis_select_topk, oasis_sparse_decode_attn,
    oasis_sparse_decode_attn_static, oasis_sparse_decode_attn_static_bytes,
    oasis_stage_blocks, oasis_stage_buffer_bytes, oasis_stage_copy, oasis_stage_plan, oasis_stage_plan_bytes,
    oasis_stage_read_stats, oasis_stage_stats, oasis_version)
