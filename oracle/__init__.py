"""CPU oracle for the SPRINT block step (test infrastructure only).

Import only from tests, the package's smoke check and the benchmark's CPU
baseline; the product path never touches this package.
"""
from .sprint_oracle import *  # noqa: F401,F403
from .sprint_oracle import (attention, compact, composite_score, fixed_schedule_count,
                            keep_count, key_norm_importance, key_norms, lmhead_confidence,
                            lmhead_top2_gap, min_acceptances, run_block, select_kept,
                            unmask_select, BlockResult, append_block, store_as,
                            run_generation, key_norm_importance_layers,
                            run_block_layers, LayersResult, silu, moe_route,
                            expert_ffn, moe_ffn)
