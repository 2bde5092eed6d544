"""CPU oracle (test infrastructure only; never used by the product path)."""
from .flce_oracle import (  # noqa: F401
    IGNORE_INDEX,
    ce_on_logits,
    decode_e4m3,
    flce_backward_fp8,
    flce_backward_from_lse,
    flce_forward,
    flce_forward_fp8,
    flce_forward_backward,
    flce_dw_rows,
    flce_rows,
    log_sum_exp,
    merge_vocab_shards,
    reduction_scale,
    valid_rows,
    vocab_shard_backward,
    vocab_shard_partials,
)
