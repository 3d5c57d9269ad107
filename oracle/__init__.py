"""Float64 CPU oracle (test infrastructure; never imported by the product)."""
from .rkv_oracle import *  # noqa: F401,F403
from .rkv_oracle import (Params, Regions, HeadResult, StepResult,  # noqa: F401
                         bf16_to_f64, logical_kv, block_regions, topk_count,
                         is_dense, block_reps, ip_scores, top_k,
                         selection_gap, merged_blocks, attend, decode_step)
