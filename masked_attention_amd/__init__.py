"""Request-centric masked attention (forward and backward) with time RoPE on MI355X.

The computation lives in librk.so (HIP, gfx950); this package holds the
library sources (csrc/), the build step (build.py) and a thin Python binding
(binding.py).  Importing the package does not load the library; the first
call does, and fails loudly if it has not been built.
"""

from .binding import (  # noqa: F401
    Batch, Layout, Plan, prune_params, rk_attn_workspace_size, rk_compress_layout, rk_gather_mean,
    rk_gather_sum, rk_mask_plan, rk_masked_attn_bwd, rk_masked_attn_fwd,
    rk_masked_attn_fwd_noalloc, rk_plan_workspace_size, rk_pointwise_attn_fwd, rk_prune_layout,
    rk_prune_layout_ex, rk_pruned_history_length, rk_pruned_history_length_ex, rk_qk_norm_rope,
    rk_time_rope,
)
