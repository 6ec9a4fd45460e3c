"""GPU parity of the rest of the expert backward over the retained rows, through the C ABI:
lrm_swiglu_backward, lrm_gather_tokens, lrm_grouped_fc1_dw / _dx / _dw_dx, lrm_scatter_tokens.

Each stage is compared with the oracle fed the GPU's own input to that stage (the FC2 input
gradient dphi the GPU computed, its selection and compaction), so every gate is that stage's:
  * dH (the activation's cotangent): both sides evaluate the same float64 expression in the same
    order and round once; the only possible difference is the last bit of exp(), so at most one
    unit in the last place of the storage type, in a vanishing fraction of elements;
  * Xc (FC1's input rows) and dx (the token rows, a float64 sum in slot order rounded once):
    bit-exact;
  * dW1 and dX (the FC1 gradients): relative Frobenius error per expert <= 1e-5 (fp32) or 2e-3
    (bf16); experts without retained rows exactly zero.
The chain is also compared end to end with the oracle's own chain from its float64 dphi.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests import _common as C

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _layer_device(w, li):
    from backward_token_expert_amd.path import to_device
    L_cap, _ = C.caps(w.spec)
    ac = li.ac
    if ac.shape[0] < L_cap:
        ac = np.concatenate([ac, np.zeros((L_cap - ac.shape[0], ac.shape[1]), ac.dtype)])
    return to_device(ac), to_device(li.x), to_device(li.W1)


def run_layer_gpu(w, pol, fused=True):
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    P = C.problem(w.spec)
    bufs = path.DeviceBuffers(P)
    inp = C.upload(w)
    li = synth.layer_inputs(w)
    ac, x, W1 = _layer_device(w, li)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
             inp["W"], bufs)
    lay = path.LayerBuffers(P)
    path.run_layer(P, ac, x, W1, bufs, lay, fused=fused)
    torch.cuda.synchronize()
    err = lrm.lrm_read_device_error(bufs.ws)
    return P, bufs, lay, li, (ac, x, W1), err


def host_layer(bufs, lay, sp):
    from backward_token_expert_amd.path import to_host
    bf = sp.dtype == "bf16"
    co = to_host(bufs.cmp_off)
    K = int(co[-1])
    return dict(cmp_off=co, sel_row=to_host(bufs.sel_row)[:K], sel_pair=to_host(bufs.sel_pair)[:K],
                dphi=to_host(bufs.dphi)[:K], dH=to_host(lay.dH, bf)[:K], Xc=to_host(lay.Xc, bf)[:K],
                dW1=to_host(lay.dW1), dX=to_host(lay.dX)[:K], dx=to_host(lay.dx))


def check_dH(got, want, dtype, rows=None):
    """Equal, or one unit apart in the last place in at most a vanishing fraction of elements."""
    g, o = np.asarray(got), np.asarray(want)
    if rows is not None:
        g, o = g[rows], o[rows]
    if dtype == "bf16":
        gi, oi = g.astype(np.int32), o.astype(np.int32)
    else:
        gi, oi = g.view(np.int32).astype(np.int64), o.view(np.int32).astype(np.int64)
    diff = gi != oi
    n = int(diff.sum())
    if n:
        assert np.all(np.abs(gi[diff] - oi[diff]) == 1), "dH differs by more than one ulp"
    assert n <= max(2, g.size // 1_000_000), f"{n} dH elements differ in the last bit"
    return n


def check_fc1_full(g, o, dtype):
    tol = C.tol_for(dtype)
    co = g["cmp_off"]
    for e in range(len(co) - 1):
        if co[e + 1] == co[e]:
            assert not g["dW1"][e].any(), f"expert {e} has no rows but nonzero dW1"
            continue
        err = C.rel_fro(g["dW1"][e], o["dW1"][e])
        assert err <= tol, f"dW1 expert {e}: rel fro {err}"
        errx = C.rel_fro(g["dX"][co[e]:co[e + 1]], o["dX"][co[e]:co[e + 1]])
        assert errx <= tol, f"dX expert {e}: rel fro {errx}"


def check_stages_full(w, g, li, dtype):
    """Every stage against the oracle on the GPU's own inputs to that stage (small sizes)."""
    sp = w.spec
    dH = O.swiglu_backward(g["dphi"], li.ac, g["sel_row"], dtype)
    nd = check_dH(g["dH"], dH, dtype)
    Xc = O.gather_tokens(li.x, g["sel_pair"], sp.k)
    assert g["Xc"].tobytes() == Xc.tobytes()
    o = dict(dW1=O.fc1_grouped_dw(g["dH"], g["Xc"], g["cmp_off"], dtype),
             dX=O.fc1_grouped_dx(g["dH"], li.W1, g["cmp_off"], dtype))
    check_fc1_full(g, o, dtype)
    dx = O.scatter_with_zeros(g["dX"], g["sel_pair"], sp.T, sp.k).astype(np.float32)
    assert g["dx"].tobytes() == dx.tobytes()
    return nd


def check_end_to_end(w, g, o_path, li, dtype):
    """The GPU chain against the oracle's chain from its own float64 dphi.  Two products compound
    here (FC2's input gradient, then FC1's), so the bound is twice a single product's."""
    sp = w.spec
    lay = O.run_layer(o_path, o_path["dphi"], li.ac, li.x, li.W1, T=sp.T, k=sp.k, dtype=dtype)
    tol = 2 * C.tol_for(dtype)
    co = g["cmp_off"]
    for e in range(len(co) - 1):
        if co[e + 1] > co[e]:
            err = C.rel_fro(g["dW1"][e], lay["dW1"][e])
            assert err <= tol, f"end to end dW1 expert {e}: rel fro {err}"
    err = C.rel_fro(g["dx"], lay["dx"])
    assert err <= tol, f"end to end dx: rel fro {err}"


SMALL = [
    ("tiny-fp32", 0, {}),
    ("qwen3-T2048", 1, {"T": 2048}),
    ("glm45-T512", 2, {"T": 512}),
    ("deepseek-v2-T512", 5, {"T": 512}),
    ("skew-T4096", 3, {"T": 4096}),
    ("layer-T2048", 4, {"T": 2048}),
]


@pytest.mark.parametrize("full", [False, True], ids=["cfg-rho", "rho1"])
@pytest.mark.parametrize("name,cfg,over", SMALL, ids=[s[0] for s in SMALL])
def test_layer_small(name, cfg, over, full):
    w = C.workload(cfg, **over)
    sp = w.spec
    pol = synth.policy(sp, full=full)
    print(f"[case] layer backward {name} full={full}", flush=True)
    P, bufs, lay, li, _, err = run_layer_gpu(w, pol)
    assert err == 0, f"device error {err}"
    g = host_layer(bufs, lay, sp)
    o_path = C.oracle_run(w, pol)
    np.testing.assert_array_equal(g["sel_row"], o_path["sel_row"])
    nd = check_stages_full(w, g, li, sp.dtype)
    print(f"  dH elements one ulp from the oracle: {nd}", flush=True)
    check_end_to_end(w, g, o_path, li, sp.dtype)


def test_layer_fc1_one_launch_equals_two_calls_and_is_deterministic():
    w = C.workload(1, T=2048)
    sp = w.spec
    pol = synth.policy(sp)
    print("[case] layer backward fused vs separate FC1 GEMMs", flush=True)
    outs = []
    for fused in (True, True, False):
        P, bufs, lay, li, _, err = run_layer_gpu(w, pol, fused=fused)
        assert err == 0
        outs.append(host_layer(bufs, lay, sp))
    for key in ("dH", "Xc", "dW1", "dX", "dx"):
        assert outs[0][key].tobytes() == outs[1][key].tobytes(), ("repeat", key)
        assert outs[0][key].tobytes() == outs[2][key].tobytes(), ("separate calls", key)


def test_layer_stale_map_entries_and_zero_tokens():
    """A second selection on the same workspace: the pair -> row map still holds the first call's
    entries, which must be ignored; tokens whose pairs are all dropped get exact zeros."""
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    w = C.workload(1, T=2048)
    sp = w.spec
    P = C.problem(sp)
    bufs = path.DeviceBuffers(P)
    lay = path.LayerBuffers(P)
    inp = C.upload(w)
    li = synth.layer_inputs(w)
    ac, x, W1 = _layer_device(w, li)
    print("[case] layer backward: second selection on one workspace", flush=True)
    for rho in ((1, 1), (1, 4)):
        pol = synth.policy(sp, rho=rho)
        path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
                 inp["W"], bufs)
        path.run_layer(P, ac, x, W1, bufs, lay)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(bufs.ws) == 0
    g = host_layer(bufs, lay, sp)
    check_stages_full(w, g, li, sp.dtype)
    kept_tok = np.zeros(sp.T, bool)
    kept_tok[g["sel_pair"] // sp.k] = True
    assert (~kept_tok).any()
    assert not g["dx"][~kept_tok].any()


def test_layer_out_of_range_indices_set_error_word():
    """Out-of-range selected rows and pair ids are refused by the kernels' own bounds checks: the
    error word says INDEX, the rows concerned are zero or skipped, the rest is still right."""
    torch = _torch()
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_host
    w = C.workload(1, T=1024)
    sp = w.spec
    pol = synth.policy(sp)
    P, bufs, lay, li, (ac, x, W1), err = run_layer_gpu(w, pol)
    assert err == 0
    K = int(to_host(bufs.cmp_off)[-1])
    assert K > 4
    print("[case] layer backward: out-of-range indices", flush=True)
    good = host_layer(bufs, lay, sp)
    bufs.sel_row[1] = P.L_cap + 5                  # outside [0, L_cap)
    lrm.lrm_swiglu_backward(P, bufs.sel_row, bufs.cmp_off, bufs.dphi, ac, lay.dH, bufs.ws)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(bufs.ws, clear=True) & 32
    dH = to_host(lay.dH, True)[:K]
    assert not dH[1].any()
    assert dH[0].tobytes() == good["dH"][0].tobytes() and dH[2:].tobytes() == good["dH"][2:].tobytes()
    bufs.sel_pair[3] = sp.T * sp.k                 # outside [0, T*k)
    lrm.lrm_scatter_tokens(P, bufs.sel_pair, bufs.cmp_off, lay.dX, lay.dx, bufs.ws)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(bufs.ws, clear=True) & 32
    lrm.lrm_gather_tokens(P, bufs.sel_pair, bufs.cmp_off, x, lay.Xc, bufs.ws)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(bufs.ws, clear=True) & 32
    # every token except the one that lost its row is unchanged
    t_lost = int(good["sel_pair"][3]) // sp.k
    dx = to_host(lay.dx)
    others = np.arange(sp.T) != t_lost
    assert dx[others].tobytes() == good["dx"][others].tobytes()


def check_fc1_each_expert(g, W1, dtype):
    """dW1_e and the dX segment of every expert in full against the oracle's float64 products of
    the GPU's own FC1 inputs (dH, Xc, already checked against the oracle), formed one expert at
    a time so that host memory stays at one expert's operands."""
    tol = C.tol_for(dtype)
    co = g["cmp_off"]
    for e in range(len(co) - 1):
        s, t = int(co[e]), int(co[e + 1])
        if t == s:
            assert not g["dW1"][e].any(), f"expert {e} has no rows but nonzero dW1"
            continue
        ref_w = O.fc1_grouped_dw(g["dH"][s:t], g["Xc"][s:t], [0, t - s], dtype)[0]
        err = C.rel_fro(g["dW1"][e], ref_w)
        assert err <= tol, f"dW1 expert {e}: rel fro {err}"
        ref_x = O.fc1_grouped_dx(g["dH"][s:t], W1[e:e + 1], [0, t - s], dtype)
        errx = C.rel_fro(g["dX"][s:t], ref_x)
        assert errx <= tol, f"dX expert {e}: rel fro {errx}"


# (workload, full retention): every workload at its own retention, and the extreme skew (empty
# experts, experts split along K in the FC1 weight-gradient schedule) at full retention too
FULL = [(0, False), (1, False), (2, False), (3, False), (3, True), (4, False), (5, False)]


@pytest.mark.parametrize("cfg,full", FULL, ids=[f"cfg{c}-{'rho1' if f else 'cfg-rho'}" for c, f in FULL])
def test_layer_full_size(cfg, full):
    """Full-size workloads in the launch configuration bench.py times, every output in full: dH
    (within one last-place unit), Xc and dx bit-exact, dW1 and dX per expert."""
    w = C.workload(cfg)
    sp = w.spec
    pol = synth.policy(sp, full=full)
    print(f"[case] layer backward full-size cfg{cfg} full={full}", flush=True)
    P, bufs, lay, li, _, err = run_layer_gpu(w, pol)
    assert err == 0, f"device error {err}"
    g = host_layer(bufs, lay, sp)
    nd = check_dH(g["dH"], O.swiglu_backward(g["dphi"], li.ac, g["sel_row"], sp.dtype), sp.dtype)
    print(f"  dH elements one ulp from the oracle: {nd}", flush=True)
    assert g["Xc"].tobytes() == O.gather_tokens(li.x, g["sel_pair"], sp.k).tobytes()
    check_fc1_each_expert(g, li.W1, sp.dtype)
    dx = O.scatter_with_zeros(g["dX"], g["sel_pair"], sp.T, sp.k).astype(np.float32)
    assert g["dx"].tobytes() == dx.tobytes()


def test_layer_graph_replay_equals_eager():
    """The path and the rest of the expert backward captured in one HIP graph: every replay gives
    the eager result bit for bit (no call allocates, synchronises or records a memset)."""
    torch = _torch()
    from backward_token_expert_amd import path
    w = C.workload(1, T=2048)
    sp = w.spec
    pol = synth.policy(sp)
    P, bufs, lay, li, (ac, x, W1), err = run_layer_gpu(w, pol)
    assert err == 0
    want = host_layer(bufs, lay, sp)
    inp = C.upload(w)
    b = path.DeviceBuffers(P)
    ly = path.LayerBuffers(P)
    print("[case] layer backward graph replay", flush=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
                 inp["W"], b, s)
        path.run_layer(P, ac, x, W1, b, ly, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
                     inp["W"], b, s)
            path.run_layer(P, ac, x, W1, b, ly, s)
    for rep in range(3):
        ly.dx.fill_(5.0)
        ly.dW1.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host_layer(b, ly, sp)
        for key in ("dH", "Xc", "dW1", "dX", "dx"):
            assert got[key].tobytes() == want[key].tobytes(), (rep, key)


def test_layer_more_than_64_slots_per_token():
    """k = 70 experts per token, so the per-token passes (gradient compaction, FC1 input gather,
    return to the tokens) walk a token's slots in two 64-lane blocks."""
    from tests.test_gpu_parity import custom
    rng = np.random.default_rng(4)
    T, k, E = 96, 70, 80
    rows = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    w = custom(rows, E=E, e_lo=3, E_loc=72, h=64, d=32, dtype="bf16")
    sp = w.spec
    pol = {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1, "kind": "cap"}
    print(f"[case] layer backward k={k}", flush=True)
    P, bufs, lay, li, _, err = run_layer_gpu(w, pol)
    assert err == 0
    g = host_layer(bufs, lay, sp)
    o_path = C.oracle_run(w, pol)
    np.testing.assert_array_equal(g["sel_row"], o_path["sel_row"])
    check_stages_full(w, g, li, sp.dtype)
