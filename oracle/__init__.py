"""Float64 CPU oracle (test infrastructure only; never called by the library)."""
from .asa_oracle import *  # noqa: F401,F403
from .asa_oracle import (pool, block_scores, block_softmax, rank_order, adaptive_count,
                         adaptive_set, static_row, static_mask, build_mask, ambiguous_rows,
                         to_csr, density, attention, attention_rows, attention_block, dense_attention,
                         kept_tokens, kept_tile_flops, num_blocks, block_range, text_blocks,
                         attention_lse, attention_bwd, attention_bwd_block, attention_bwd_flops,
                         attention_bwd_terms,
                         pattern_sparsity, pattern_mse, pattern_loss, select_patterns, pattern_search)
