"""fp64 CPU oracle (test infrastructure only; see lcv_oracle's header)."""
from .lcv_oracle import (  # noqa: F401
    BLOCK, HEAD_DIM, ROPE_SECTIONS, SOFTMAX_SCALE, attended_pairs, block_mask, block_pairs_attended,
    bsa_backward, bsa_backward_keys, bsa_backward_rows, bsa_forward, bsa_forward_blocks, bsa_forward_cached, cross_attention, cross_attention_backward, csr, masked_attention, merge_partials,
    masked_attention_backward,
    n_blocks_of, qk_norm_rope, qk_norm_rope_backward, rmsnorm, rope3d, rope3d_at, rope3d_transpose, token_coords, token_mask, token_mask_rows,
)
