"""CPU fp64 oracle (test infrastructure only; never used by the product path)."""

from .masked_attention import (  # noqa: F401
    CANDIDATE, EMPTY, FULL, HISTORY, PARTIAL, PROFILE, REALTIME, TILE_K, TILE_Q,
    attention_backward, attention_backward_qk_norm, attention_backward_sampled, attention_forward,
    attention_rows,
    compressed_history_length, count_visible, group_sum_compress, hstu_rab, masked_softmax_attention,
    masked_softmax_attention_backward, pointwise_attention,
    pointwise_attention_forward, pointwise_attention_rows, prune_history, prune_history_keep, prune_history_pooled,
    pruned_history_length, pruned_history_length_exp, qk_rmsnorm,
    qk_rmsnorm_backward,
    rope_frequencies,
    tile_plan, tile_plan_request, time_bucket, time_rope, time_rope_transpose, visibility, visible_rows,
)
