"""GPU parity of forward-time admission (lrm_admit_quotas) through the C ABI: the admitted
candidate, its quotas and offsets are bit-exact with the oracle's candidate descent, and the rest
of the path then runs on the admitted quotas exactly as under that candidate's policy."""
import numpy as np
import pytest

import oracle as O
import synth
from tests import _common as C
from tests.test_gpu_parity import (check_compact, check_gemms, check_scores,
                                   check_selection_valid, gate_compact_gemms, host)

pytestmark = pytest.mark.gpu

RATES = [(1, 1, 1), (0, 1, 1), (0, 3, 4), (0, 1, 2), (0, 1, 4), (0, 1, 8)]   # (full, num, den)


def _policies(kind, cap):
    return [{"full": f, "rho_num": a, "rho_den": b, "cap_abs": cap, "kind": kind}
            for f, a, b in RATES]


def _row_bytes(sp):
    b = 2 if sp.dtype == "bf16" else 4
    return (sp.h + sp.d) * b + 4 * sp.d + 8      # Gc, Phic, dphi, sel_row/sel_pair


def _budgets(n_loc, sp, kind, cap, K_cap):
    """Budgets that admit each candidate in turn, and one that admits none."""
    row = _row_bytes(sp)
    Ks = [int(O.plan_quotas(n_loc, p)[1][-1]) for p in _policies(kind, cap)]
    base = 1 << 30
    out = []
    for K in sorted(set(Ks), reverse=True):
        out.append(dict(mem_budget=base + K * row, mem_base=base, mem_per_row=row,
                        comm_budget=-1, comm_per_row=0))
    # the communication window alone binds: room for the smallest total only
    out.append(dict(mem_budget=1 << 50, mem_base=base, mem_per_row=row,
                    comm_budget=min(Ks) * sp.h * 2, comm_per_row=sp.h * 2))
    out.append(dict(mem_budget=base + min(Ks) * row - 1, mem_base=base, mem_per_row=row,
                    comm_budget=-1, comm_per_row=0))
    return out


CASES = [(1, "cap", None), (3, "cap", None), (4, "waterfill", "spec"), (1, "proportional", -1),
         (0, "cap", None)]


@pytest.mark.parametrize("cfg,kind,cap", CASES, ids=[f"cfg{c}-{k}" for c, k, _ in CASES])
def test_admission_descent(cfg, kind, cap):
    torch = pytest.importorskip("torch")
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_host
    w = C.workload(cfg)
    sp = w.spec
    cap = sp.cap_abs if cap in (None, "spec") else cap
    if kind == "proportional":
        cap = -1
    P = C.problem(sp)
    inp = C.upload(w)
    n_loc = O.routed_counts(w.topk_idx, sp.E)[sp.e_lo:sp.e_lo + sp.E_loc]
    pols = _policies(kind, cap)
    for bi, bud in enumerate(_budgets(n_loc, sp, kind, cap, P.K_cap)):
        want_c, want_q, want_off = O.admit_quotas(n_loc, pols, bud, P.K_cap)
        adm = lrm.make_admission(RATES, kind=kind, cap_abs=cap, **bud)
        print(f"[case] admission cfg{cfg} {kind} budget {bi} -> candidate {want_c}", flush=True)
        b = path.DeviceBuffers(P)
        path.run(P, C.policy_obj(pols[0]), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
                 inp["W"], b, admission=adm)
        torch.cuda.synchronize()
        assert lrm.lrm_read_device_error(b.ws) == 0
        assert int(to_host(b.admitted)[0]) == want_c
        np.testing.assert_array_equal(to_host(b.quota), want_q)
        np.testing.assert_array_equal(to_host(b.cmp_off), want_off)
        K = int(want_off[-1])
        if want_c < 0:
            assert K == 0 and not to_host(b.dW).any()
            continue
        # the rest of the path on the admitted quotas equals the path under that policy
        o = C.oracle_run(w, pols[want_c], gemms=False)
        g = host(b, sp)
        if np.array_equal(g["sel_row"], o["sel_row"]):
            check_compact(g, o)
            if bi == 0:                          # the products once per workload (host time)
                check_gemms(g, o, w.W, sp.dtype)
        else:
            # the selections may differ only where the float32 scores differ in bits; then the
            # admitted selection must still be the valid top-q under the GPU's own scores, and
            # the GPU's compaction and GEMMs on the oracle's selection must match the oracle
            assert not np.array_equal(g["score"].view(np.uint32), o["score32"].view(np.uint32))
            check_scores(g, o)
            check_selection_valid(g, o)
            gate_compact_gemms(P, b, inp, o, w.W, sp.dtype)
