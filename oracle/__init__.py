"""fp64 CPU oracle for exact softmax attention (test infrastructure only).

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .reference import (NEG_INF, EXACT, FP64, LogOf, attention, attention_backward, attention_backward_sampled,
                        attention_kvlens, attention_kvlens_backward, attention_rows, attention_varlen,
                        attention_varlen_backward,
                        block_stats, blocked_single_query, finalize, legal_keys,
                        merge_partials, merge_stats, set_partitions,
                        softmax_rows, split_partials)

__all__ = ["NEG_INF", "EXACT", "FP64", "LogOf", "attention", "attention_backward", "attention_backward_sampled",
           "attention_kvlens", "attention_kvlens_backward", "attention_rows", "attention_varlen",
           "attention_varlen_backward",
           "block_stats", "blocked_single_query", "finalize", "legal_keys",
           "merge_partials", "merge_stats", "set_partitions", "softmax_rows",
           "split_partials"]
