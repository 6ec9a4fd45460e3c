"""CPU float64 oracle of the LRMoE backward hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg, never by the GPU library.
"""
from .lrm_oracle import *  # noqa: F401,F403
from .lrm_oracle import (compact, dw_rows, dx_rows, f32_to_bf16_rne, forward_layout,  # noqa: F401
                         grouped_dw, grouped_dx, lrm_scores, plan_quotas, routed_counts, run,
                         select_top_quota, widen)
