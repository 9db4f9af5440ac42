"""CPU fp64 oracle (test infrastructure only; see mla_oracle)."""
from .mla_oracle import (  # noqa: F401
    RopeConfig, SelectionError, cache_append, decode_attention, decode_attention_absorbed, inv_freq,
    max_rel_l2, rope_cos_sin, rope_rotate, rope_rotate_halves, selection_mask, selection_set, softmax_scale, topk_select,
    yarn_correction_dim,
)
