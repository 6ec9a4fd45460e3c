"""Device buffers and the call sequences of the hot path (marshalling only).

``DeviceBuffers`` allocates, with PyTorch, every output and the workspace of one problem; ``run``
enqueues lrm_plan_quotas -> lrm_score (or lrm_score_criterion) -> lrm_select -> lrm_compact ->
lrm_grouped_dw_dx (or lrm_grouped_dw -> lrm_grouped_dx) on one stream, or, given a second
stream, runs lrm_score_norms there beside lrm_plan_quotas and lrm_score_combine after both.
``LayerBuffers`` and ``run_layer`` do the same for the rest of the expert backward over the
retained rows:
lrm_swiglu_backward -> lrm_gather_tokens -> lrm_grouped_fc1_dw_dx (or the two FC1 calls) ->
lrm_scatter_tokens.  No step of the path is computed here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import lrm


def storage_dtype(dtype: str):
    return torch.int16 if dtype == "bf16" else torch.float32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a host array; bf16 bit patterns (uint16) travel as int16."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor, bf16: bool = False) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if bf16 else a


class DeviceBuffers:
    """Outputs and workspace of one problem, sized to its capacities."""

    def __init__(self, problem: lrm.Problem, device="cuda"):
        p = problem
        i32 = dict(dtype=torch.int32, device=device)
        st = storage_dtype("bf16" if p.dtype == lrm.LRM_BF16 else "f32")
        self.problem = p
        self.counts = torch.zeros(p.E, **i32)
        self.fwd_off = torch.zeros(p.E_loc + 1, **i32)
        self.row_pair = torch.zeros(p.L_cap, **i32)
        self.quota = torch.zeros(p.E_loc, **i32)
        self.cmp_off = torch.zeros(p.E_loc + 1, **i32)
        self.admitted = torch.full((1,), -2, **i32)
        self.score = torch.zeros(p.L_cap, dtype=torch.float32, device=device)
        self.sel_row = torch.zeros(p.K_cap, **i32)
        self.sel_pair = torch.zeros(p.K_cap, **i32)
        self.Gc = torch.zeros((p.K_cap, p.h), dtype=st, device=device)
        self.Phic = torch.zeros((p.K_cap, p.d), dtype=st, device=device)
        self.dW = torch.zeros((p.E_loc, p.h, p.d), dtype=torch.float32, device=device)
        self.dphi = torch.zeros((p.K_cap, p.d), dtype=torch.float32, device=device)
        nws = lrm.lrm_workspace_bytes(p)
        if nws == 0:
            raise lrm.LrmError("invalid problem")
        self.ws = torch.zeros(nws, dtype=torch.uint8, device=device)


def _torch_stream(stream):
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def run(problem, policy, topk_idx, topk_w, g, phi, W, bufs: DeviceBuffers, stream=None,
        criterion: str = "lrm", keys=None, fused: bool = True, admission=None, side_stream=None):
    """Enqueue the whole hot path on `stream` (default: torch's current stream).  `criterion`
    picks the selection score (lrm_score for "lrm", else lrm_score_criterion; "random" ranks by
    `keys`, one float32 per pair).  `fused` runs both GEMMs as lrm_grouped_dw_dx, else as
    lrm_grouped_dw then lrm_grouped_dx.  With an `admission` (lrm.make_admission), the quotas are
    those of the first feasible candidate (lrm_admit_quotas after lrm_plan_quotas) and
    bufs.admitted receives its index (-1: none, every quota zero).  With a `side_stream` (LRM
    criterion only) the score's norm pass (lrm_score_norms) runs on it, forked from and joined back
    to `stream` with events, while lrm_plan_quotas runs on `stream`; the results are bitwise
    those of the one-stream sequence."""
    b = bufs
    split = criterion == "lrm" and side_stream is not None
    if split:
        main, side = _torch_stream(stream), _torch_stream(side_stream)
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        lrm.lrm_score_norms(problem, g, phi, b.ws, side)
        join.record(side)
    lrm.lrm_plan_quotas(problem, policy, topk_idx, b.counts, b.fwd_off, b.row_pair, b.quota,
                        b.cmp_off, b.ws, stream)
    if admission is not None:
        lrm.lrm_admit_quotas(problem, admission, b.fwd_off, b.quota, b.cmp_off, b.admitted, b.ws,
                             stream)
    if split:
        main.wait_event(join)
        lrm.lrm_score_combine(problem, topk_w, b.row_pair, b.fwd_off, b.score, b.ws, stream)
    elif criterion == "lrm":
        lrm.lrm_score(problem, topk_w, g, phi, b.row_pair, b.fwd_off, b.score, b.ws, stream)
    else:
        lrm.lrm_score_criterion(problem, criterion, topk_w, g, phi, keys, b.row_pair, b.fwd_off,
                                b.score, b.ws, stream)
    lrm.lrm_select(problem, b.score, b.fwd_off, b.quota, b.cmp_off, b.sel_row, b.ws, stream)
    lrm.lrm_compact(problem, b.sel_row, b.row_pair, b.cmp_off, topk_w, g, phi, b.Gc, b.Phic,
                    b.sel_pair, b.ws, stream)
    if fused:
        lrm.lrm_grouped_dw_dx(problem, b.Gc, b.Phic, W, b.cmp_off, b.dW, b.dphi, b.ws, stream)
    else:
        lrm.lrm_grouped_dw(problem, b.Gc, b.Phic, b.cmp_off, b.dW, b.ws, stream)
        lrm.lrm_grouped_dx(problem, b.Gc, W, b.cmp_off, b.dphi, b.ws, stream)


class LayerBuffers:
    """Outputs of the rest of the expert backward, sized to the problem's capacities."""

    def __init__(self, problem: lrm.Problem, device="cuda"):
        p = problem
        st = storage_dtype("bf16" if p.dtype == lrm.LRM_BF16 else "f32")
        f32 = dict(dtype=torch.float32, device=device)
        self.dH = torch.zeros((p.K_cap, 2 * p.d), dtype=st, device=device)
        self.Xc = torch.zeros((p.K_cap, p.h), dtype=st, device=device)
        self.dW1 = torch.zeros((p.E_loc, 2 * p.d, p.h), **f32)
        self.dX = torch.zeros((p.K_cap, p.h), **f32)
        self.dx = torch.zeros((p.T, p.h), **f32)


def run_layer(problem, ac, x, W1, bufs: DeviceBuffers, lay: LayerBuffers, stream=None,
              fused: bool = True):
    """Enqueue the rest of the expert backward after ``run`` on the same buffers: the activation's
    backward from dphi, FC1's input rows, the FC1 gradients and the return to the tokens."""
    b = bufs
    lrm.lrm_swiglu_backward(problem, b.sel_row, b.cmp_off, b.dphi, ac, lay.dH, b.ws, stream)
    lrm.lrm_gather_tokens(problem, b.sel_pair, b.cmp_off, x, lay.Xc, b.ws, stream)
    if fused:
        lrm.lrm_grouped_fc1_dw_dx(problem, lay.dH, lay.Xc, W1, b.cmp_off, lay.dW1, lay.dX, b.ws,
                                  stream)
    else:
        lrm.lrm_grouped_fc1_dw(problem, lay.dH, lay.Xc, b.cmp_off, lay.dW1, b.ws, stream)
        lrm.lrm_grouped_fc1_dx(problem, lay.dH, W1, b.cmp_off, lay.dX, b.ws, stream)
    lrm.lrm_scatter_tokens(problem, b.sel_pair, b.cmp_off, lay.dX, lay.dx, b.ws, stream)
