"""LRMoE backward hot path on MI355X (gfx950): C-ABI library liblrm.so + thin binding.

The library (include/lrm.h) implements routed counting, retention quotas, LRM scoring, per-expert
top-q selection, physical compaction and the grouped FC2 dW / dphi GEMMs of "LRMoE: Demand-Side
Load Re-Calibration for Efficient MoE Training on Memory-Constrained Nodes" as hand-written HIP
kernels.  This package only marshals arguments (lrm.py) and sequences the six calls (path.py).
"""
from . import lrm, path  # noqa: F401
from .lrm import (LRM_BF16, LRM_F32, Admission, LrmError, Problem, QuotaPolicy,  # noqa: F401
                  load_library, lrm_admit_quotas, make_admission,
                  lrm_compact, lrm_gather_tokens, lrm_grouped_dw, lrm_grouped_dw_dx,
                  lrm_grouped_dw_dx_noalloc,
                  lrm_grouped_dx, lrm_grouped_fc1_dw, lrm_grouped_fc1_dw_dx, lrm_grouped_fc1_dx,
                  lrm_plan_quotas, lrm_scatter_tokens, lrm_swiglu_backward,
                  lrm_read_device_error, lrm_score, lrm_score_combine, lrm_score_criterion,
                  lrm_score_norms, lrm_select,
                  lrm_workspace_bytes, make_policy, make_problem)
