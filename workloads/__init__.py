"""Seeded synthetic inputs for the paged decode-attention workloads.

This package only draws inputs: lengths, block placements, random tensor values (rounded from
fp32 draws to the storage dtype) and the random projections that build the multi-query keys. It
holds none of the attention arithmetic. The oracle tests and the GPU path both consume its arrays
unchanged, so neither side's inputs come from the other.
"""

from .generators import (  # noqa: F401
    PagedCase,
    PaddedCase,
    padded_from_paged,
    MQCase,
    LockstepPlan,
    POISON_BF16,
    POISON_F32,
    poison_value,
    to_storage,
    make_paged_case,
    tiny,
    tiny_edges,
    b16_plan,
    b128,
    long_context,
    shard_share,
    mq,
    mq_tokenizer,
    TokenizerCase,
    fp32_scale,
)
