"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .varlen_oracle import *  # noqa: F401,F403
from .varlen_oracle import (  # noqa: F401
    validate_cu_seqlens, lengths_from_text_mask, image_tokens, cu_seqlens_from_lengths,
    joint_cu_seqlens, pack_by_cu_seqlens, unpack_by_cu_seqlens, tile_order, grid_blocks,
    block_to_logical, block_schedule, varlen_attention, block_local_key_range,
    block_local_attention, dense_masked_attention, block_diagonal_mask, block_difference_mask,
    cfg_combine, mixfusion_chunk_plan, sp_auto_pad, split_plan, split_range, work_items,
    LPT_MAX_REQS, XCDS, MAX_SPLIT, MIN_SPLIT_KEYS,
)
