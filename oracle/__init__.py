"""fp64 CPU oracle for the MSA forward path.  Test infrastructure only: the
product path never imports it."""

from .msa_oracle import (  # noqa: F401
    block_max_pool,
    default_scale,
    dense_gqa,
    index_topk_row,
    msa_forward,
    msa_index_topk,
    msa_sparse_attention,
    select_blocks,
    softmax_attention,
    token_scores,
    visible_positions,
)
