"""Thin Python binding of liblrm.so (include/lrm.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch only supplies device memory
(tensors passed by data pointer) and the stream.  There is no fallback: if the library is not
built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LRM_LIBRARY") or os.path.join(_PKG, "liblrm.so")

LRM_F32, LRM_BF16 = 0, 1
DEVERR = {1: "EXPERT_ID", 2: "L_CAP", 4: "K_CAP", 8: "QUOTA", 16: "NONFINITE", 32: "INDEX"}

EXPORTS = ("lrm_workspace_bytes", "lrm_plan_quotas", "lrm_admit_quotas", "lrm_score",
           "lrm_score_norms", "lrm_score_combine", "lrm_score_criterion",
           "lrm_select", "lrm_compact", "lrm_grouped_dw", "lrm_grouped_dx", "lrm_grouped_dw_dx",
           "lrm_swiglu_backward", "lrm_gather_tokens", "lrm_grouped_fc1_dw", "lrm_grouped_fc1_dx",
           "lrm_grouped_fc1_dw_dx", "lrm_scatter_tokens", "lrm_read_device_error",
           "lrm_status_string", "lrm_grouped_dw_dx_noalloc")

QUOTA_KINDS = {"cap": 0, "proportional": 1, "waterfill": 2}
CRITERIA = {"lrm": 0, "grad_sq": 1, "grad_abs": 2, "random": 3}


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "k", "E", "e_lo", "E_loc", "h", "d", "dtype", "L_cap", "K_cap")]


class QuotaPolicy(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("full", "rho_num", "rho_den", "cap_abs", "kind")]


MAX_CANDIDATES = 16


class Admission(ctypes.Structure):
    _fields_ = [("n_cand", ctypes.c_int32), ("kind", ctypes.c_int32), ("cap_abs", ctypes.c_int32),
                ("full", ctypes.c_int32 * MAX_CANDIDATES),
                ("rho_num", ctypes.c_int32 * MAX_CANDIDATES),
                ("rho_den", ctypes.c_int32 * MAX_CANDIDATES),
                ("mem_budget", ctypes.c_int64), ("mem_base", ctypes.c_int64),
                ("mem_per_row", ctypes.c_int64), ("comm_budget", ctypes.c_int64),
                ("comm_per_row", ctypes.c_int64)]


def make_admission(candidates, mem_budget, mem_base=0, mem_per_row=0, comm_budget=-1,
                   comm_per_row=0, kind="cap", cap_abs=-1) -> Admission:
    """candidates: list of (full, rho_num, rho_den), tested in that order."""
    a = Admission()
    a.n_cand = len(candidates)
    a.kind = QUOTA_KINDS[kind] if isinstance(kind, str) else int(kind)
    a.cap_abs = cap_abs
    for i, (f, n, d) in enumerate(candidates):
        a.full[i], a.rho_num[i], a.rho_den[i] = int(f), int(n), int(d)
    a.mem_budget, a.mem_base, a.mem_per_row = mem_budget, mem_base, mem_per_row
    a.comm_budget, a.comm_per_row = comm_budget, comm_per_row
    return a


class LrmError(RuntimeError):
    pass


_LIB = None


def load_library(path: Optional[str] = None):
    """Load liblrm.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LrmError(f"{p} is missing: build the HIP library first "
                       "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    PP, QP = ctypes.POINTER(Problem), ctypes.POINTER(QuotaPolicy)
    lib.lrm_workspace_bytes.argtypes = [PP]
    lib.lrm_workspace_bytes.restype = sz
    lib.lrm_plan_quotas.argtypes = [PP, QP] + [vp] * 7 + [sz, vp]
    lib.lrm_admit_quotas.argtypes = [PP, ctypes.POINTER(Admission)] + [vp] * 5 + [sz, vp]
    lib.lrm_score.argtypes = [PP] + [vp] * 7 + [sz, vp]
    lib.lrm_score_norms.argtypes = [PP] + [vp] * 3 + [sz, vp]
    lib.lrm_score_combine.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_score_criterion.argtypes = [PP, i32] + [vp] * 8 + [sz, vp]
    lib.lrm_select.argtypes = [PP] + [vp] * 6 + [sz, vp]
    lib.lrm_compact.argtypes = [PP] + [vp] * 10 + [sz, vp]
    lib.lrm_grouped_dw.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_grouped_dx.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_grouped_dw_dx.argtypes = [PP] + [vp] * 7 + [sz, vp]
    lib.lrm_grouped_dw_dx_noalloc.argtypes = [PP] + [vp] * 6 + [vp]
    lib.lrm_swiglu_backward.argtypes = [PP] + [vp] * 6 + [sz, vp]
    lib.lrm_gather_tokens.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_grouped_fc1_dw.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_grouped_fc1_dx.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_grouped_fc1_dw_dx.argtypes = [PP] + [vp] * 7 + [sz, vp]
    lib.lrm_scatter_tokens.argtypes = [PP] + [vp] * 5 + [sz, vp]
    lib.lrm_read_device_error.argtypes = [vp, ctypes.POINTER(i32), i32, vp]
    for f in EXPORTS:
        if f not in ("lrm_workspace_bytes", "lrm_status_string"):
            getattr(lib, f).restype = ctypes.c_int
    lib.lrm_status_string.argtypes = [ctypes.c_int]
    lib.lrm_status_string.restype = ctypes.c_char_p
    if path is None:
        _LIB = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(lib, status: int, what: str):
    if status != 0:
        raise LrmError(f"{what}: {lib.lrm_status_string(status).decode()} (status {status})")


def make_problem(T, k, E, e_lo, E_loc, h, d, dtype, L_cap, K_cap) -> Problem:
    dt = {"f32": LRM_F32, "bf16": LRM_BF16}.get(dtype, dtype)
    return Problem(T, k, E, e_lo, E_loc, h, d, dt, L_cap, K_cap)


def make_policy(full=0, rho_num=1, rho_den=1, cap_abs=-1, kind="cap") -> QuotaPolicy:
    kd = QUOTA_KINDS[kind] if isinstance(kind, str) else int(kind)
    return QuotaPolicy(int(full), int(rho_num), int(rho_den), int(cap_abs), kd)


def lrm_workspace_bytes(problem: Problem) -> int:
    return int(load_library().lrm_workspace_bytes(ctypes.byref(problem)))


def lrm_plan_quotas(problem, policy, topk_idx, counts, fwd_off, row_pair, quota, cmp_off, ws,
                    stream=None):
    lib = load_library()
    _check(lib, lib.lrm_plan_quotas(ctypes.byref(problem), ctypes.byref(policy), _ptr(topk_idx),
                                    _ptr(counts), _ptr(fwd_off), _ptr(row_pair), _ptr(quota),
                                    _ptr(cmp_off), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "lrm_plan_quotas")


def lrm_score(problem, topk_w, g, phi, row_pair, fwd_off, score, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_score(ctypes.byref(problem), _ptr(topk_w), _ptr(g), _ptr(phi),
                              _ptr(row_pair), _ptr(fwd_off), _ptr(score), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "lrm_score")


def lrm_score_norms(problem, g, phi, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_score_norms(ctypes.byref(problem), _ptr(g), _ptr(phi), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "lrm_score_norms")


def lrm_score_combine(problem, topk_w, row_pair, fwd_off, score, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_score_combine(ctypes.byref(problem), _ptr(topk_w), _ptr(row_pair),
                                      _ptr(fwd_off), _ptr(score), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "lrm_score_combine")


def lrm_score_criterion(problem, criterion, topk_w, g, phi, keys, row_pair, fwd_off, score, ws,
                        stream=None):
    lib = load_library()
    crit = CRITERIA[criterion] if isinstance(criterion, str) else int(criterion)
    _check(lib, lib.lrm_score_criterion(ctypes.byref(problem), crit, _ptr(topk_w), _ptr(g),
                                        _ptr(phi), _ptr(keys), _ptr(row_pair), _ptr(fwd_off),
                                        _ptr(score), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)), "lrm_score_criterion")


def lrm_select(problem, score, fwd_off, quota, cmp_off, sel_row, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_select(ctypes.byref(problem), _ptr(score), _ptr(fwd_off), _ptr(quota),
                               _ptr(cmp_off), _ptr(sel_row), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "lrm_select")


def lrm_compact(problem, sel_row, row_pair, cmp_off, topk_w, g, phi, Gc, Phic, sel_pair, ws,
                stream=None):
    lib = load_library()
    _check(lib, lib.lrm_compact(ctypes.byref(problem), _ptr(sel_row), _ptr(row_pair),
                                _ptr(cmp_off), _ptr(topk_w), _ptr(g), _ptr(phi), _ptr(Gc),
                                _ptr(Phic), _ptr(sel_pair), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "lrm_compact")


def lrm_grouped_dw(problem, Gc, Phic, cmp_off, dW, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_dw(ctypes.byref(problem), _ptr(Gc), _ptr(Phic), _ptr(cmp_off),
                                   _ptr(dW), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "lrm_grouped_dw")


def lrm_grouped_dx(problem, Gc, W, cmp_off, dphi, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_dx(ctypes.byref(problem), _ptr(Gc), _ptr(W), _ptr(cmp_off),
                                   _ptr(dphi), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "lrm_grouped_dx")


def lrm_grouped_dw_dx(problem, Gc, Phic, W, cmp_off, dW, dphi, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_dw_dx(ctypes.byref(problem), _ptr(Gc), _ptr(Phic), _ptr(W),
                                      _ptr(cmp_off), _ptr(dW), _ptr(dphi), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "lrm_grouped_dw_dx")


def lrm_grouped_dw_dx_noalloc(problem, Gc, Phic, W, cmp_off, dW, dphi, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_dw_dx_noalloc(ctypes.byref(problem), _ptr(Gc), _ptr(Phic), _ptr(W),
                                              _ptr(cmp_off), _ptr(dW), _ptr(dphi),
                                              _stream(stream)),
           "lrm_grouped_dw_dx_noalloc")


def lrm_admit_quotas(problem, admission, fwd_off, quota, cmp_off, admitted, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_admit_quotas(ctypes.byref(problem), ctypes.byref(admission), _ptr(fwd_off),
                                     _ptr(quota), _ptr(cmp_off), _ptr(admitted),
                                     _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "lrm_admit_quotas")


def _ws(ws):
    return _ptr(ws), ws.numel() * ws.element_size()


def lrm_swiglu_backward(problem, sel_row, cmp_off, dphi, ac, dH, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_swiglu_backward(ctypes.byref(problem), _ptr(sel_row), _ptr(cmp_off),
                                        _ptr(dphi), _ptr(ac), _ptr(dH), *_ws(ws),
                                        _stream(stream)), "lrm_swiglu_backward")


def lrm_gather_tokens(problem, sel_pair, cmp_off, x, Xc, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_gather_tokens(ctypes.byref(problem), _ptr(sel_pair), _ptr(cmp_off),
                                      _ptr(x), _ptr(Xc), *_ws(ws), _stream(stream)),
           "lrm_gather_tokens")


def lrm_grouped_fc1_dw(problem, dH, Xc, cmp_off, dW1, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_fc1_dw(ctypes.byref(problem), _ptr(dH), _ptr(Xc), _ptr(cmp_off),
                                       _ptr(dW1), *_ws(ws), _stream(stream)), "lrm_grouped_fc1_dw")


def lrm_grouped_fc1_dx(problem, dH, W1, cmp_off, dX, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_fc1_dx(ctypes.byref(problem), _ptr(dH), _ptr(W1), _ptr(cmp_off),
                                       _ptr(dX), *_ws(ws), _stream(stream)), "lrm_grouped_fc1_dx")


def lrm_grouped_fc1_dw_dx(problem, dH, Xc, W1, cmp_off, dW1, dX, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_grouped_fc1_dw_dx(ctypes.byref(problem), _ptr(dH), _ptr(Xc), _ptr(W1),
                                          _ptr(cmp_off), _ptr(dW1), _ptr(dX), *_ws(ws),
                                          _stream(stream)), "lrm_grouped_fc1_dw_dx")


def lrm_scatter_tokens(problem, sel_pair, cmp_off, dX, dx, ws, stream=None):
    lib = load_library()
    _check(lib, lib.lrm_scatter_tokens(ctypes.byref(problem), _ptr(sel_pair), _ptr(cmp_off),
                                       _ptr(dX), _ptr(dx), *_ws(ws), _stream(stream)),
           "lrm_scatter_tokens")


def lrm_read_device_error(ws, clear: bool = False, stream=None) -> int:
    lib = load_library()
    code = ctypes.c_int32(0)
    _check(lib, lib.lrm_read_device_error(_ptr(ws), ctypes.byref(code), int(clear),
                                          _stream(stream)), "lrm_read_device_error")
    return int(code.value)


def deverr_names(code: int):
    return [name for bit, name in DEVERR.items() if code & bit]
