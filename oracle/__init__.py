"""Plain CPU oracle (fp64) for indexer-selected block-sparse attention.

Test infrastructure only: imported by ``tests/``, by the package smoke check and by
the CPU-baseline leg of ``bench.py``.  Nothing in the library imports it.
"""
from .sparse_attn_oracle import (  # noqa: F401
    SequencePools,
    attend,
    block_scores,
    dequantize_q8_0,
    mask_positions,
    merge_partials,
    pool_blocks,
    quantize_q8_0,
    round_to_storage,
    run_case,
    run_query,
    select_blocks,
    select_positions,
    select_positions_token_expanded,
    visible_tokens,
    window_union,
)
