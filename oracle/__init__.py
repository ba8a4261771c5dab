"""CPU fp64 oracle (test infrastructure only; see flashprefill_oracle)."""
from .flashprefill_oracle import *  # noqa: F401,F403
from .flashprefill_oracle import (Selection, block_entries, block_lengths, block_logits,  # noqa: F401
                                  block_means, block_scores, dequantize_blockwise,
                                  flops_executed, num_blocks, select_blocks,
                                  sparse_attention, attention_probabilities, threshold)
