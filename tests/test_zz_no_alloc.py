"""The allocation-free FC2 GEMM entry point, lrm_grouped_dw_dx_noalloc, through the C ABI against
lrm_grouped_dw_dx (the same products with a caller workspace) on the same compacted inputs.

dphi must be equal bit for bit (its schedule does not depend on the workspace).  dW must be equal
bit for bit per expert, or, where lrm_grouped_dw_dx split an expert's rows into partial sums added
afterwards (the allocation-free call never splits), within the path's relative Frobenius bound
(1e-5 for fp32 inputs, 2e-3 for bf16).  Each case makes two calls in a row on one GPU, the second
on a smaller input, so the second call runs on the static schedule buffer the first one left.
"""
import numpy as np
import pytest

import synth
from tests import _common as C

pytestmark = pytest.mark.gpu


def _compacted(cfg, T, full):
    """Run the path once (lrm_grouped_dw_dx included) and return its buffers."""
    import torch
    from backward_token_expert_amd import lrm, path
    w = C.workload(cfg, T=T)
    sp = w.spec
    pol = synth.policy(sp, full=full)
    P = C.problem(sp)
    b = path.DeviceBuffers(P)
    inp = C.upload(w)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"],
             b)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws) == 0
    return sp, P, b, inp


def _check_pair(sp, P, b, inp):
    import torch
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_host
    dW = torch.full_like(b.dW, float("nan"))
    dphi = torch.full_like(b.dphi, float("nan"))
    lrm.lrm_grouped_dw_dx_noalloc(P, b.Gc, b.Phic, inp["W"], b.cmp_off, dW, dphi)
    torch.cuda.synchronize()
    co = to_host(b.cmp_off)
    K = int(co[-1])
    want_w, got_w = to_host(b.dW), to_host(dW)
    assert to_host(dphi)[:K].tobytes() == to_host(b.dphi)[:K].tobytes()
    tol = C.tol_for(sp.dtype)
    same = 0
    for e in range(sp.E_loc):
        if co[e + 1] == co[e]:
            assert not got_w[e].any(), f"expert {e} has no rows but nonzero dW"
            continue
        if got_w[e].tobytes() == want_w[e].tobytes():
            same += 1
            continue
        err = C.rel_fro(got_w[e], want_w[e])
        assert err <= tol, f"dW expert {e}: rel fro {err}"
    return same


# (workload, T of the first call, T of the second call, full retention).  The whole layer (4) is
# store-bound: the workspace call runs it dphi-first with dW units claimed from one counter, the
# allocation-free call in the common order, so the two orders are checked against each other.
CASES = [(1, 4096, 1024, False), (0, 4096, 1024, False), (3, 8192, 2048, True),
         (2, 1024, 512, False), (4, 4096, 1024, False),
         # fp32 at full retention: the workspace call splits the largest experts along K, the
         # allocation-free one never does
         (0, 4096, 2048, True)]


@pytest.mark.parametrize("cfg,T1,T2,full", CASES,
                         ids=[f"cfg{c[0]}{'-full' if c[3] else ''}" for c in CASES])
def test_noalloc_equals_workspace_call_twice(cfg, T1, T2, full):
    for T in (T1, T2):
        sp, P, b, inp = _compacted(cfg, T, full)
        print(f"[case] noalloc cfg{cfg} T={T} full={full}", flush=True)
        same = _check_pair(sp, P, b, inp)
        print(f"  experts with dW equal bit for bit: {same} of {sp.E_loc}", flush=True)
