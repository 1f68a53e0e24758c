"""fp64 CPU oracle of the Prefilling-dLLM chunk-sparse attention path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path; see ``oracle/reference.py`` for the definitions and
the passages of the Prefilling-dLLM summary each one follows.

Every function here is pinned by ``-m "not gpu"`` tests to values fixed by
the mathematics (brute force on tiny inputs, closed forms, library routines,
invariants); none is "parity unpinned".
"""
from .reference import (as_f64, kv_head_of, softmax_rows, chunk_prefill_score,
                        select_topb, select_topk, attended_pool_rows, attended_kv,
                        compact_kept_rows, all_rows_kept,
                        split_attn_decode, lse_merge, attention_over_parts,
                        token_log_probs, chunk_scores)

__all__ = ["as_f64", "kv_head_of", "softmax_rows", "chunk_prefill_score",
           "select_topb", "select_topk", "attended_pool_rows", "attended_kv",
           "compact_kept_rows", "all_rows_kept",
           "split_attn_decode", "lse_merge", "attention_over_parts",
           "token_log_probs", "chunk_scores"]
