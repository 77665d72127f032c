"""MI355X-native mean-pooled Top-K block-routed sparse attention (forward).

The computation lives in ``libsparse_attn.so`` (hand-written HIP for
gfx950, C ABI in ``include/sparse_attn.h``); this package is its thin Python
binding.  Build the library with ``python -m block_sparse_attention_05_amd.build``.
"""
from ._lib import (  # noqa: F401
    BLOCK, HEAD_DIM, VIDEO_TAIL_MODES, SparseAttnError, check_key_bias, dense_sink_fwd, lib,
    routed_attention,
    sa_max_selected, sa_dense_workspace_bytes, sa_device_info, sa_num_blocks, sa_num_query_blocks,
    sa_num_sparse_blocks, sa_route_workspace_bytes, sa_anchor_workspace_bytes, spark_global_anchor,
    spark_reweight, sparse_attn_fwd_spark, routed_attention_spark, sparse_attn_pool,
    sparse_attn_fwd_fused, routed_attention_fused,
    sa_topk_budget,
    sparse_attn_fwd, sparse_attn_route, sparse_attn_route_noalloc,
)
