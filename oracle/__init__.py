"""CPU oracle for Stem's sparse-prefill path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  The product library never uses it.
"""
from .stem_oracle import *  # noqa: F401,F403
from .stem_oracle import (ALPHA_SCALES_KSTART, block_log_value_norm, block_scores,  # noqa: F401
                          block_sparse_attention, decode_e4m3fn, dense_causal_attention,
                          dequantize_blocks, forced_blocks, full_lists, kept_count,
                          schedule_topk, select_row, strided_scores, tpd_budget, value_bonus)
