"""Shared helpers of the parity tests: upload synthetic inputs, run the GPU path through the
C ABI, run the oracle, compare."""
from __future__ import annotations

import functools

import numpy as np

import oracle as O
import synth


def caps(sp, K_cap=None):
    L_cap = max(1, sp.T * min(sp.k, sp.E_loc))
    return L_cap, (K_cap if K_cap is not None else L_cap)


def problem(sp, K_cap=None):
    from backward_token_expert_amd import lrm
    L_cap, Kc = caps(sp, K_cap)
    return lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, Kc)


def policy_obj(pol):
    from backward_token_expert_amd import lrm
    return lrm.make_policy(pol["full"], pol["rho_num"], pol["rho_den"], pol["cap_abs"],
                           pol.get("kind", "cap"))


@functools.lru_cache(maxsize=4)
def workload(cfg, **over):
    return synth.make(cfg, **dict(over))


def oracle_run(w, pol, gemms=True, criterion="lrm", keys=None):
    sp = w.spec
    return O.run(w.topk_idx, w.topk_w, w.g, w.phi, w.W, T=sp.T, k=sp.k, E=sp.E, e_lo=sp.e_lo,
                 E_loc=sp.E_loc, dtype=sp.dtype, policy=pol, gemms=gemms, criterion=criterion,
                 keys=keys)


def upload(w, device="cuda"):
    from backward_token_expert_amd.path import to_device
    sp = w.spec
    L_cap, _ = caps(sp)
    phi = w.phi
    if phi.shape[0] < L_cap:  # pad to the row capacity the problem declares
        pad = np.zeros((L_cap - phi.shape[0], sp.d), phi.dtype)
        phi = np.concatenate([phi, pad])
    return dict(topk_idx=to_device(w.topk_idx, device), topk_w=to_device(w.topk_w, device),
                g=to_device(w.g, device), phi=to_device(phi, device), W=to_device(w.W, device))


def rel_fro(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt((ref * ref).sum())
    num = np.sqrt(((x - ref) ** 2).sum())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def tol_for(dtype):
    return 1e-5 if dtype == "f32" else 2e-3
