"""The oracle: a plain, slow, obviously correct fp64 CPU attention (forward, backward,
block-sparse pattern).

TEST INFRASTRUCTURE ONLY. It exists to check the HIP library. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.
It imports nothing from the product package and shares no code with it; the only
module both sides use is ``workloads`` (seeded random inputs, no attention math).
"""
from .attention import (KeySets, attention_backward, attention_backward_varlen, attention_forward,
                        attention_forward_varlen, backward_keys_dkdv, backward_rows_dq, forward_row, kv_head,
                        row_probabilities, row_scores)
from .block_rule import allowed_blocks, block_lists, key_mask_from_lists, transpose_lists

__all__ = [
    "KeySets", "attention_forward", "attention_backward", "attention_forward_varlen",
    "attention_backward_varlen", "backward_keys_dkdv", "backward_rows_dq", "forward_row", "kv_head",
    "row_probabilities", "row_scores", "allowed_blocks", "block_lists", "key_mask_from_lists",
    "transpose_lists",
]
