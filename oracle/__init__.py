"""CPU oracle for dynamic sparse attention in causal prefill and decoding (test infrastructure).

Plain, slow NumPy fp64 statements of what the hot path computes. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never imports it.
"""
from .minf_oracle import (  # noqa: F401
    BLOCK,
    topk_lowidx,
    attend_rows,
    dense_attn,
    ashape_mask_row,
    vs_last_query_probs,
    vs_column_diag_sums,
    vs_index,
    vs_block_set,
    vs_column_set,
    vs_mask_block,
    vs_window_set,
    vsw_mask_block,
    vertical_tiles,
    pool_blocks,
    block_scores,
    block_index,
    bs_mask_block,
    ashape_mask_block,
    build_vs_index,
    build_block_index,
    sparse_attn,
    plan_mask_block,
    decode_block_index,
    decode_mask,
    sparse_decode,
    dense_decode,
    plan_blocks,
    pattern_recall,
    candidate_plan,
    search_head_pattern,
    grid_permutation,
    permuted_block_index,
    permuted_block_attn,
)
