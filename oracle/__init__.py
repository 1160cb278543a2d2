"""Plain fp64 CPU oracle for exact softmax attention (forward and backward), for the
causal / sliding-window block classification, and for the QK RMS-norm + rotary prologue.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library.

Parity status: every function here is pinned by a CPU test against facts the pages or the
mathematics fix (closed forms, invariants, an independent library routine, finite differences,
brute-force masks and the worked mask pictures of the Graphcore page).  No function is
"parity unpinned".
"""
from .attention import (attn_fwd, attn_bwd, attn_probs, attn_fwd_rows, visible_mask,
                        group_of_head)
from .blocks import (classify_blocks, block_keep_mask, partial_offsets_in_loop_order,
                     triu_offset_sequence, kv_block_range, SKIP, FULL, PARTIAL)
from .rope import qk_norm_rope, rms_normalise, swap_pairs

__all__ = ["attn_fwd", "attn_bwd", "attn_probs", "attn_fwd_rows", "visible_mask",
           "group_of_head", "classify_blocks", "block_keep_mask",
           "partial_offsets_in_loop_order", "triu_offset_sequence", "kv_block_range",
           "SKIP", "FULL", "PARTIAL", "qk_norm_rope", "rms_normalise", "swap_pairs"]
