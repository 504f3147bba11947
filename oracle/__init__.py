"""CPU float64 oracle for the FlashAttention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It shares no code with the HIP library or its binding.
"""
from .attention import (NEG_INF, attention_forward, expand_stats, from_bnsd, head_attention,
                        keep_matrix, to_bnsd)

__all__ = ["NEG_INF", "attention_forward", "expand_stats", "from_bnsd", "head_attention",
           "keep_matrix", "to_bnsd"]
