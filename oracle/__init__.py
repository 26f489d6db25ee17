"""CPU oracle (test infrastructure only; see fsdp_oracle's header)."""

from .fsdp_oracle import (  # noqa: F401
    AdamW,
    UnitLayout,
    adamw_scalars,
    adamw_step,
    bf16_round_nearest_even,
    bf16_widen,
    cast_unflatten,
    flatten_pad,
    numel,
    persistent_bytes,
    reduce_adamw_shard,
    reduce_adamw_shard_bf16acc,
    reduce_adamw_shard_hybrid,
    reduce_shard,
    reduce_shard_bf16acc,
    reduce_shard_hybrid,
    unflatten,
    unit_layout,
)
