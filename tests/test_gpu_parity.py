"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar (per the contract of the path):
  * counts, forward layout, quotas, offsets, selected rows, compacted buffers and pair ids:
    bit-exact;
  * scores: |s - R| <= 1e-5 * R against the oracle's float64 R;
  * dW and dphi: relative Frobenius error per expert <= 1e-5 (fp32 inputs) or 2e-3 (bf16
    inputs); experts without retained rows must be exactly zero.
Selection is also gated in reverse: the GPU select applied to the oracle's float32 scores must
reproduce the oracle's selection exactly (both decide on the same float32 values).
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import synth
from tests import _common as C

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def run_gpu(w, pol, K_cap=None, overlap=False):
    """The path as bench.py runs it by default, on one stream (overlap=True: the score's norm half
    on a second stream beside the plan, as bench.py --overlap)."""
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    P = C.problem(w.spec, K_cap)
    bufs = path.DeviceBuffers(P)
    inp = C.upload(w)
    side = torch.cuda.Stream() if overlap else None
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"],
             bufs, side_stream=side)
    torch.cuda.synchronize()
    err = lrm.lrm_read_device_error(bufs.ws)
    return P, bufs, inp, err


def host(bufs, sp):
    from backward_token_expert_amd.path import to_host
    bf = sp.dtype == "bf16"
    fo = to_host(bufs.fwd_off)
    co = to_host(bufs.cmp_off)
    L, K = int(fo[-1]), int(co[-1])
    return dict(counts=to_host(bufs.counts), fwd_off=fo, row_pair=to_host(bufs.row_pair)[:L],
                quota=to_host(bufs.quota), cmp_off=co, score=to_host(bufs.score)[:L],
                sel_row=to_host(bufs.sel_row)[:K], sel_pair=to_host(bufs.sel_pair)[:K],
                Gc=to_host(bufs.Gc, bf)[:K], Phic=to_host(bufs.Phic, bf)[:K],
                dW=to_host(bufs.dW), dphi=to_host(bufs.dphi)[:K])


def check_plan(g, o):
    np.testing.assert_array_equal(g["counts"], o["counts"])
    np.testing.assert_array_equal(g["fwd_off"], o["fwd_off"])
    np.testing.assert_array_equal(g["row_pair"], o["row_pair"])
    np.testing.assert_array_equal(g["quota"], o["quota"])
    np.testing.assert_array_equal(g["cmp_off"], o["cmp_off"])


def check_scores(g, o):
    R = o["score64"]
    s = g["score"].astype(np.float64)
    bad = np.abs(s - R) > 1e-5 * R
    assert not bad.any(), f"{int(bad.sum())} scores off, worst rel {np.max(np.abs(s - R) / np.maximum(R, 1e-300))}"
    return int((g["score"].view(np.uint32) != o["score32"].view(np.uint32)).sum())


def check_selection_valid(g, o):
    """GPU selection from the GPU's own scores: bit-exact with the oracle wherever the two float32
    score vectors agree bitwise; otherwise the kept set must be the unique top-q under the GPU's
    scores and every disagreement must sit on a boundary that the 1e-5 score tolerance reaches."""
    s_bits = g["score"].view(np.uint32).astype(np.int64)
    fo, co, q = g["fwd_off"], g["cmp_off"], g["quota"]
    rp = g["row_pair"]
    for e in range(len(q)):
        rows = np.arange(fo[e], fo[e + 1])
        kept = g["sel_row"][co[e]:co[e + 1]]
        assert kept.size == q[e]
        assert np.all(np.diff(kept) > 0)
        if kept.size == 0 or kept.size == rows.size:
            continue
        dropped = np.setdiff1d(rows, kept)
        # rank key: higher score first, then lower pair index
        kk = s_bits[kept] * (1 << 32) - rp[kept]
        kd = s_bits[dropped] * (1 << 32) - rp[dropped]
        assert kk.min() > kd.max()
    same = np.array_equal(g["score"].view(np.uint32), o["score32"].view(np.uint32))
    if same:
        np.testing.assert_array_equal(g["sel_row"], o["sel_row"])
    else:
        diff = np.setxor1d(g["sel_row"], o["sel_row"])
        R = o["score64"]
        for r in diff:
            e = np.searchsorted(fo, r, side="right") - 1
            seg = np.arange(fo[e], fo[e + 1])
            kept_o = o["sel_row"][o["cmp_off"][e]:o["cmp_off"][e + 1]]
            drop_o = np.setdiff1d(seg, kept_o)
            lo = R[kept_o].min() if kept_o.size else 0.0
            hi = R[drop_o].max() if drop_o.size else 0.0
            assert abs(R[r] - lo) <= 2e-5 * lo or abs(R[r] - hi) <= 2e-5 * hi


def check_compact(g, o, bit_exact=True):
    np.testing.assert_array_equal(g["sel_row"], o["sel_row"])
    np.testing.assert_array_equal(g["sel_pair"], o["sel_pair"])
    assert g["Gc"].tobytes() == o["Gc"].tobytes()
    assert g["Phic"].tobytes() == o["Phic"].tobytes()


def check_gemms(g, o, W, dtype):
    """Every expert's dW_e and every row of its dphi segment against the oracle's float64
    products, in full: relative Frobenius error per expert within the dtype's bound, experts
    without retained rows exactly zero.  Where the oracle run holds no GEMM results (full-size
    workloads), they are formed here one expert at a time from the oracle's own compacted buffers
    (which the caller has already found byte-equal to the GPU's), so host memory stays at one
    expert's operands."""
    tol = C.tol_for(dtype)
    co = o["cmp_off"]
    for e in range(len(co) - 1):
        s, t = int(co[e]), int(co[e + 1])
        if t == s:
            assert not g["dW"][e].any(), f"expert {e} has no rows but nonzero dW"
            continue
        if "dW" in o:
            ref_w, ref_x = o["dW"][e], o["dphi"][s:t]
        else:
            ref_w = O.grouped_dw(o["Gc"][s:t], o["Phic"][s:t], [0, t - s], dtype)[0]
            ref_x = O.grouped_dx(o["Gc"][s:t], W[e:e + 1], [0, t - s], dtype)
        err = C.rel_fro(g["dW"][e], ref_w)
        assert err <= tol, f"dW expert {e}: rel fro {err}"
        errx = C.rel_fro(g["dphi"][s:t], ref_x)
        assert errx <= tol, f"dphi expert {e}: rel fro {errx}"


def gate_select(P, bufs, o):
    """GPU select on the oracle's float32 scores and offsets must equal the oracle's selection."""
    torch = _torch()
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_device, to_host
    L = int(o["fwd_off"][-1])
    score = torch.zeros_like(bufs.score)
    score[:L] = to_device(o["score32"])
    fo = to_device(o["fwd_off"].astype(np.int32))
    q = to_device(o["quota"].astype(np.int32))
    co = to_device(o["cmp_off"].astype(np.int32))
    sel = torch.full_like(bufs.sel_row, -1)
    lrm.lrm_select(P, score, fo, q, co, sel, bufs.ws)
    torch.cuda.synchronize()
    K = int(o["cmp_off"][-1])
    np.testing.assert_array_equal(to_host(sel)[:K], o["sel_row"])


def gate_compact_gemms(P, bufs, inp, o, W, dtype):
    """GPU compaction of the oracle's selection, then the GPU GEMMs on those buffers."""
    torch = _torch()
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_device, to_host
    K = int(o["cmp_off"][-1])
    L = int(o["fwd_off"][-1])
    sel = torch.zeros_like(bufs.sel_row)
    sel[:K] = to_device(o["sel_row"].astype(np.int32))
    rp = torch.zeros_like(bufs.row_pair)
    rp[:L] = to_device(o["row_pair"].astype(np.int32))
    co = to_device(o["cmp_off"].astype(np.int32))
    lrm.lrm_compact(P, sel, rp, co, inp["topk_w"], inp["g"], inp["phi"], bufs.Gc, bufs.Phic,
                    bufs.sel_pair, bufs.ws)
    lrm.lrm_grouped_dw(P, bufs.Gc, bufs.Phic, co, bufs.dW, bufs.ws)
    lrm.lrm_grouped_dx(P, bufs.Gc, inp["W"], co, bufs.dphi, bufs.ws)
    torch.cuda.synchronize()
    bf = dtype == "bf16"
    g = dict(sel_row=o["sel_row"], sel_pair=to_host(bufs.sel_pair)[:K],
             Gc=to_host(bufs.Gc, bf)[:K], Phic=to_host(bufs.Phic, bf)[:K],
             dW=to_host(bufs.dW), dphi=to_host(bufs.dphi)[:K])
    check_compact(g, o)
    check_gemms(g, o, W, dtype)


# ------------------------------------------------------------------------------------------------
# small workloads: full oracle, everything compared
# ------------------------------------------------------------------------------------------------

SMALL = [
    ("tiny-fp32", 0, {}),
    ("qwen3-T2048", 1, {"T": 2048}),
    ("glm45-T1024", 2, {"T": 1024}),
    ("deepseek-v2-T1024", 5, {"T": 1024}),
    ("skew-T4096", 3, {"T": 4096}),
    ("layer-T2048", 4, {"T": 2048}),
]


@pytest.mark.parametrize("full", [False, True], ids=["cfg-rho", "rho1"])
@pytest.mark.parametrize("name,cfg,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_end_to_end(name, cfg, over, full):
    w = C.workload(cfg, **over)
    sp = w.spec
    pol = synth.policy(sp, full=full)
    print(f"[case] {name} full={full}", flush=True)
    P, bufs, inp, err = run_gpu(w, pol)
    assert err == 0, f"device error {err}"
    o = C.oracle_run(w, pol)
    g = host(bufs, sp)
    check_plan(g, o)
    check_scores(g, o)
    check_selection_valid(g, o)
    gate_select(P, bufs, o)
    if np.array_equal(g["sel_row"], o["sel_row"]):
        check_compact(g, o)
        check_gemms(g, o, w.W, sp.dtype)
    else:
        gate_compact_gemms(P, bufs, inp, o, w.W, sp.dtype)


@pytest.mark.parametrize("rho", synth.RHO_SWEEP_3, ids=["1.0", "0.75", "0.5", "0.25"])
def test_small_skew_rho_sweep(rho):
    w = C.workload(3, T=4096)
    pol = synth.policy(w.spec, rho=rho)
    print(f"[case] skew-T4096 rho={rho}", flush=True)
    P, bufs, inp, err = run_gpu(w, pol)
    assert err == 0
    o = C.oracle_run(w, pol)
    g = host(bufs, w.spec)
    check_plan(g, o)
    check_scores(g, o)
    check_selection_valid(g, o)
    gate_select(P, bufs, o)
    check_compact(g, o)
    check_gemms(g, o, w.W, w.spec.dtype)


# ------------------------------------------------------------------------------------------------
# hand-built edge cases
# ------------------------------------------------------------------------------------------------

def custom(idx_rows, E, e_lo, E_loc, h, d, dtype, seed=7, weights=None):
    """Workload from explicit routing (rows of expert ids per token) with seeded values."""
    idx = np.asarray(idx_rows, np.int32)
    T, k = idx.shape
    rng = np.random.default_rng(seed)
    if weights is None:
        a = rng.random((T, k)) + 0.05
        weights = (a / a.sum(1, keepdims=True)).astype(np.float32)
    sp = dataclasses.replace(synth.SPECS[1], name="custom", T=T, k=k, E=E, e_lo=e_lo, E_loc=E_loc,
                             h=h, d=d, dtype=dtype, seed=seed)
    flat = idx.reshape(-1)
    loc = (flat >= e_lo) & (flat < e_lo + E_loc)
    lp = np.flatnonzero(loc)
    layout = lp[np.argsort(flat[loc], kind="stable")]
    g = synth.rows(seed, synth.S_G, T, h, kind=dtype)
    phi = synth.swiglu_rows(seed, layout, d, kind=dtype)
    W = synth.rows(seed, synth.S_W, E_loc * h, d, scale=d ** -0.5, kind=dtype).reshape(E_loc, h, d)
    return synth.Workload(sp, flat.copy(), np.asarray(weights, np.float32).reshape(-1).copy(), g,
                          phi, W, layout, np.zeros(E), np.arange(T))


def full_compare(w, pol, expect_err=0):
    P, bufs, inp, err = run_gpu(w, pol)
    assert err == expect_err, f"device error {err}"
    o = C.oracle_run(w, pol)
    g = host(bufs, w.spec)
    check_plan(g, o)
    check_scores(g, o)
    check_selection_valid(g, o)
    gate_select(P, bufs, o)
    check_compact(g, o)
    check_gemms(g, o, w.W, w.spec.dtype)
    return g, o


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segment_sizes_and_ragged_tiles(dtype):
    # local segments of 0, 1, 63, 64, 65 and 4097 rows; h and d multiples of 8 but not of 128
    sizes = [0, 1, 63, 64, 65, 4097]
    rows = []
    for e, n in enumerate(sizes):
        rows += [[e]] * n
    rows += [[6]] * 50 + [[7]] * 30            # non-local experts
    rng = np.random.default_rng(3)
    rows = np.asarray(rows)[rng.permutation(len(rows))]
    w = custom(rows, E=8, e_lo=0, E_loc=6, h=200, d=72, dtype=dtype)
    print(f"[case] segment sizes {sizes} dtype={dtype}", flush=True)
    for pol in ({"full": 1, "rho_num": 1, "rho_den": 1, "cap_abs": -1},
                {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1},
                {"full": 0, "rho_num": 0, "rho_den": 1, "cap_abs": -1},     # q = 0 everywhere
                {"full": 0, "rho_num": 4, "rho_den": 1, "cap_abs": 64}):    # cap binds
        full_compare(w, pol)


def test_select_segments_ending_at_the_row_capacity():
    # every pair local, so the last segment ends exactly at L_cap = 4099 (not a multiple of 4, so
    # the score, phi and row buffers end mid-16-byte chunk); segment starts 0, 1000, 1001, 3001
    # take every offset modulo 4
    sizes = [1000, 1, 2000, 1098]
    rows = []
    for e, n in enumerate(sizes):
        rows += [[e]] * n
    rows = np.asarray(rows)[np.random.default_rng(5).permutation(len(rows))]
    w = custom(rows, E=4, e_lo=0, E_loc=4, h=64, d=64, dtype="bf16")
    assert C.caps(w.spec)[0] == w.L == 4099
    print("[case] segments ending at L_cap = 4099", flush=True)
    for pol in ({"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1},
                {"full": 0, "rho_num": 3, "rho_den": 1, "cap_abs": 777}):
        full_compare(w, pol)


@pytest.mark.parametrize("h,d", [(512, 384), (256, 512), (384, 1408), (2048, 200)])
def test_gemm_tile_shapes(h, d):
    # column tiles of 192 (d % 192 == 0), 256 (d % 256 == 0) and 128 (otherwise, ragged edge)
    rng = np.random.default_rng(9)
    rows = np.stack([rng.permutation(6)[:2] for _ in range(1500)])
    w = custom(rows, E=6, e_lo=1, E_loc=4, h=h, d=d, dtype="bf16")
    print(f"[case] tile shapes h={h} d={d}", flush=True)
    full_compare(w, {"full": 0, "rho_num": 2, "rho_den": 3, "cap_abs": -1})


def test_single_local_expert_and_no_local_pairs():
    rng = np.random.default_rng(4)
    rows = np.stack([rng.permutation(6)[:2] for _ in range(300)])
    w = custom(rows, E=6, e_lo=2, E_loc=1, h=64, d=128, dtype="bf16")
    print("[case] E_loc=1", flush=True)
    full_compare(w, {"full": 0, "rho_num": 1, "rho_den": 3, "cap_abs": -1})
    rows = np.stack([rng.permutation([0, 1, 2])[:2] for _ in range(100)])
    w = custom(rows, E=6, e_lo=3, E_loc=3, h=64, d=64, dtype="bf16")
    print("[case] L=0", flush=True)
    g, o = full_compare(w, {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1})
    assert g["fwd_off"][-1] == 0 and not g["dW"].any()


def test_plan_with_wide_tables():
    # 4096 experts (the per-chunk table is 4097 columns wide, more than a workgroup's threads),
    # 1024 of them local (one summing thread per local expert), 21 chunks of pairs (a full and a
    # partial placing workgroup)
    rng = np.random.default_rng(21)
    T, k = 10390, 2
    rows = np.stack([rng.choice(4096, k, replace=False) for _ in range(T)])
    w = custom(rows, E=4096, e_lo=2000, E_loc=1024, h=64, d=64, dtype="bf16")
    print("[case] E=4096, E_loc=1024, 21 chunks", flush=True)
    for pol in ({"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1},
                {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1, "kind": "waterfill"}):
        full_compare(w, pol)


def test_row_and_retained_capacities_truncate_and_flag():
    # L > L_cap and K > K_cap: the forward segments end at L_cap, the quotas are those of the
    # truncated segments, the compacted ones end at K_cap, and both capacity bits are set
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    w = C.workload(1, T=1024)
    sp = w.spec
    pol = synth.policy(sp)
    L_cap, K_cap = 5000, 500          # truncated segments 1024, 1015, 971, 875, 791, 324, 0, ...
    assert w.L > L_cap                # keep 156 each under rho = 1/2: K = 936 > K_cap
    P = lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, K_cap)
    b = path.DeviceBuffers(P)
    inp = C.upload(w)
    print(f"[case] L={w.L} > L_cap={L_cap}, K_cap={K_cap}", flush=True)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"],
             b)
    torch.cuda.synchronize()
    err = lrm.lrm_read_device_error(b.ws)
    assert err == lrm_bits("L_CAP", "K_CAP"), lrm.deverr_names(err)
    from backward_token_expert_amd.path import to_host
    counts = O.routed_counts(w.topk_idx, sp.E)
    row_pair, fwd = O.forward_layout(w.topk_idx, sp.e_lo, sp.E_loc)
    fwd_c = np.minimum(fwd, L_cap)
    q = O.plan_quotas(np.diff(fwd_c), pol)[0]
    pre = np.concatenate([[0], np.cumsum(q)])
    o0 = np.minimum(pre[:-1], K_cap)
    o1 = np.minimum(pre[1:], K_cap)
    np.testing.assert_array_equal(to_host(b.counts), counts)
    np.testing.assert_array_equal(to_host(b.fwd_off), fwd_c)
    np.testing.assert_array_equal(to_host(b.row_pair)[:L_cap], row_pair[:L_cap])
    np.testing.assert_array_equal(to_host(b.quota), o1 - o0)
    np.testing.assert_array_equal(to_host(b.cmp_off), np.concatenate([o0, [min(pre[-1], K_cap)]]))
    # the kept rows: each truncated segment's own top quota, from the GPU's float32 scores
    score = to_host(b.score)[:L_cap]
    want = O.select_top_quota(score, fwd_c, o1 - o0, row_pair[:L_cap])
    np.testing.assert_array_equal(to_host(b.sel_row)[:K_cap], want)


def test_nonfinite_scores_are_flagged_and_ranked_as_zero():
    # A NaN phi row gives a NaN score and a +inf in g infinite scores: lrm_score sets NONFINITE,
    # lrm_select ranks NaN (and any pattern with the sign bit) as +0 and +inf above every finite
    # score, and flags the NaN.  The same holds for caller keys of the random criterion, with a
    # negative and a NaN key.
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_host, to_device
    w = C.workload(1, T=512)
    sp = w.spec
    pol = synth.policy(sp)
    P = C.problem(sp)
    inp = dict(C.upload(w))
    r_nan = 5
    t_inf = int(w.layout_pairs[r_nan]) // sp.k + 1   # a token that does not own row r_nan
    inp["phi"][r_nan] = 0x7FC0                   # bf16 NaN
    inp["g"][t_inf, 3] = 0x7F80                  # bf16 +inf
    print("[case] NaN phi row, +inf in g", flush=True)
    b = path.DeviceBuffers(P)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
             inp["W"], b)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws) & lrm_bits("NONFINITE")
    fo, rp = to_host(b.fwd_off), to_host(b.row_pair)[:w.L]
    score = to_host(b.score)[:w.L]
    assert np.isnan(score[r_nan])
    inf_rows = np.flatnonzero(rp // sp.k == t_inf)
    assert inf_rows.size and np.all(np.isposinf(score[inf_rows]))
    ranked = np.where(np.isnan(score), np.float32(0), score)
    want = O.select_top_quota(ranked, fo, to_host(b.quota), rp)
    np.testing.assert_array_equal(to_host(b.sel_row)[:want.size], want)
    assert np.isin(inf_rows, want).all()          # +inf ranks first: always kept

    keys = synth.pair_keys(sp).copy()
    p_neg, p_nan = int(rp[fo[1]]), int(rp[fo[2] + 1])   # a pair of experts 1 and 2
    keys[p_neg], keys[p_nan] = -1.0, np.nan
    print("[case] random criterion with a negative and a NaN key", flush=True)
    b = path.DeviceBuffers(P)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
             inp["W"], b, criterion="random", keys=to_device(keys))
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws) & lrm_bits("NONFINITE")
    kr = keys[rp].astype(np.float32)
    kr = np.where(np.isnan(kr) | (kr < 0), np.float32(0), kr)
    want = O.select_top_quota(kr, fo, to_host(b.quota), rp)
    np.testing.assert_array_equal(to_host(b.sel_row)[:want.size], want)


def test_select_clamps_quotas_outside_the_segment_and_flags():
    # quota above n (clamped to n: every row kept) and below 0 (clamped to 0: none kept) set
    # QUOTA; an offset that would run past K_cap truncates that segment at K_cap and sets K_CAP
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_host, to_device
    w = C.workload(1, T=512)
    sp = w.spec
    pol = synth.policy(sp)
    P = C.problem(sp)
    inp = C.upload(w)
    b = path.DeviceBuffers(P)
    path.run(P, C.policy_obj(pol), inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"],
             inp["W"], b)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws) == 0
    fo, rp = to_host(b.fwd_off), to_host(b.row_pair)
    n = np.diff(fo)
    score = to_host(b.score)[:fo[-1]]
    q = to_host(b.quota).astype(np.int64)
    q_bad = q.copy()
    q_bad[0], q_bad[1] = n[0] + 5, -3
    q_eff = np.clip(q_bad, 0, n)
    off = np.concatenate([[0], np.cumsum(q_eff)])
    print("[case] quotas n+5 and -3", flush=True)
    b.sel_row.fill_(-7)
    lrm.lrm_select(P, b.score, b.fwd_off, to_device(q_bad.astype(np.int32)),
                   to_device(off.astype(np.int32)), b.sel_row, b.ws)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws, clear=True) & lrm_bits("QUOTA")
    want = O.select_top_quota(score, fo, q_eff, rp)
    np.testing.assert_array_equal(to_host(b.sel_row)[:off[-1]], want)
    assert want[:n[0]].tolist() == list(range(fo[0], fo[1]))      # expert 0 keeps every row

    # K_cap below the end of the last segment: the segment that crosses it keeps only its top
    # K_cap - offset rows, the ones after it none
    K = int(off[-1])
    K_cap = K - 10
    Ps = C.problem(sp, K_cap=K_cap)
    b.sel_row.fill_(-7)
    print(f"[case] K_cap = {K_cap} < K = {K}", flush=True)
    lrm.lrm_select(Ps, b.score, b.fwd_off, to_device(q_eff.astype(np.int32)),
                   to_device(off.astype(np.int32)), b.sel_row, b.ws)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws, clear=True) & lrm_bits("K_CAP")
    q_cut = np.clip(np.minimum(q_eff, K_cap - off[:-1]), 0, None)
    got = to_host(b.sel_row)
    np.testing.assert_array_equal(got[:K_cap], O.select_top_quota(score, fo, q_cut, rp))
    assert np.all(got[K_cap:K] == -7)


def test_score_flags_row_pairs_out_of_range():
    # a row whose pair id lies outside [0, T*k) scores 0 and sets INDEX, in lrm_score and in the
    # split form alike; every other row keeps its score
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_host
    w = C.workload(1, T=512)
    sp = w.spec
    P = C.problem(sp)
    inp = C.upload(w)
    b = path.DeviceBuffers(P)
    path.run(P, C.policy_obj(synth.policy(sp)), inp["topk_idx"], inp["topk_w"], inp["g"],
             inp["phi"], inp["W"], b)
    torch.cuda.synchronize()
    want = to_host(b.score)[:w.L].copy()
    b.row_pair[3] = sp.T * sp.k + 5
    b.row_pair[4] = -2
    want[3] = want[4] = 0.0
    print("[case] row_pair entries out of range", flush=True)
    for split in (False, True):
        b.score.fill_(-1.0)
        lrm.lrm_read_device_error(b.ws, clear=True)
        if split:
            lrm.lrm_score_norms(P, inp["g"], inp["phi"], b.ws)
            lrm.lrm_score_combine(P, inp["topk_w"], b.row_pair, b.fwd_off, b.score, b.ws)
        else:
            lrm.lrm_score(P, inp["topk_w"], inp["g"], inp["phi"], b.row_pair, b.fwd_off, b.score,
                          b.ws)
        torch.cuda.synchronize()
        assert lrm.lrm_read_device_error(b.ws) == lrm_bits("INDEX"), split
        assert to_host(b.score)[:w.L].tobytes() == want.tobytes(), split


def lrm_bits(*names):
    from backward_token_expert_amd import lrm
    return sum(bit for bit, n in lrm.DEVERR.items() if n in names)


def test_all_equal_scores_keep_first_rows():
    T = 500
    rows = np.zeros((T, 1), np.int32)
    w = custom(rows, E=2, e_lo=0, E_loc=1, h=64, d=64, dtype="bf16",
               weights=np.full((T, 1), 0.5, np.float32))
    w.g[:] = w.g[0]
    w.phi[:] = w.phi[0]
    print("[case] all-equal scores", flush=True)
    g, o = full_compare(w, {"full": 0, "rho_num": 1, "rho_den": 3, "cap_abs": -1})
    assert g["sel_row"].tolist() == list(range(T // 3))


def test_ties_straddling_the_boundary():
    rng = np.random.default_rng(5)
    rows = np.stack([rng.permutation(8)[:2] for _ in range(3000)])
    w = custom(rows, E=8, e_lo=0, E_loc=8, h=128, d=64, dtype="bf16")
    pol = {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1}
    o = C.oracle_run(w, pol, gemms=False)
    k = w.spec.k
    # in every expert, copy the q-th ranked pair's (alpha, g, phi) onto the next two ranked pairs
    for e in range(8):
        r0, r1 = o["fwd_off"][e], o["fwd_off"][e + 1]
        q = o["quota"][e]
        if q == 0 or q + 2 > r1 - r0:
            continue
        seg = np.arange(r0, r1)
        order = seg[np.lexsort((o["row_pair"][seg], -o["score32"][seg].astype(np.float64)))]
        src = order[q - 1]
        ps = o["row_pair"][src]
        for dst in order[q:q + 2]:
            pd = o["row_pair"][dst]
            w.topk_w[pd] = w.topk_w[ps]
            w.g[pd // k] = w.g[ps // k]
            w.phi[dst] = w.phi[src]
    o2 = C.oracle_run(w, pol, gemms=False)
    n_ties = 0
    for e in range(8):
        r0, r1 = o2["fwd_off"][e], o2["fwd_off"][e + 1]
        kept = o2["sel_row"][o2["cmp_off"][e]:o2["cmp_off"][e + 1]]
        dropped = np.setdiff1d(np.arange(r0, r1), kept)
        if kept.size and dropped.size:
            n_ties += int(o2["score32"][kept].min() == o2["score32"][dropped].max())
    assert n_ties >= 4, "fixture must put ties on the boundary"
    print(f"[case] boundary ties in {n_ties} experts", flush=True)
    full_compare(w, pol)


def test_segment_longer_than_lds_stage():
    T = 40000
    rows = np.zeros((T, 1), np.int32)
    rows[::7] = 1
    w = custom(rows, E=2, e_lo=0, E_loc=2, h=64, d=64, dtype="bf16")
    print("[case] segment of 34285 rows (global-memory select)", flush=True)
    full_compare(w, {"full": 0, "rho_num": 1, "rho_den": 3, "cap_abs": -1})


def test_out_of_range_expert_id_sets_error_word():
    rng = np.random.default_rng(6)
    rows = np.stack([rng.permutation(4)[:2] for _ in range(200)])
    w = custom(rows, E=4, e_lo=0, E_loc=4, h=64, d=64, dtype="bf16")
    w.topk_idx[5] = 9     # invalid id: skipped and flagged, never dereferenced
    print("[case] invalid expert id", flush=True)
    P, bufs, inp, err = run_gpu(w, {"full": 1, "rho_num": 1, "rho_den": 1, "cap_abs": -1})
    assert err & 1
    from backward_token_expert_amd.path import to_host
    cnt = to_host(bufs.counts)
    valid = np.delete(w.topk_idx, 5)
    np.testing.assert_array_equal(cnt, np.bincount(valid, minlength=4))


def _compact_with(P, bufs, inp, sel_host, rp_host, K):
    """lrm_compact on a host-given selection / row map (the rest from the workload)."""
    torch = _torch()
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_device
    sel = torch.zeros_like(bufs.sel_row)
    sel[:K] = to_device(np.asarray(sel_host, np.int32))
    rp = torch.zeros_like(bufs.row_pair)
    rp[:len(rp_host)] = to_device(np.asarray(rp_host, np.int32))
    co = torch.zeros_like(bufs.cmp_off)
    co[-1] = K
    lrm.lrm_read_device_error(bufs.ws, clear=True)
    lrm.lrm_compact(P, sel, rp, co, inp["topk_w"], inp["g"], inp["phi"], bufs.Gc, bufs.Phic,
                    bufs.sel_pair, bufs.ws)
    torch.cuda.synchronize()
    return lrm.lrm_read_device_error(bufs.ws)


GEMM_SHAPES = [
    # (retained rows per expert, h, d): tile widths 192 / 256 / 384 (with a partial column tile),
    # one or several row tiles, an empty expert, and a full round of dphi units followed by a
    # partial one (130 row tiles x 2 column tiles = 260 units on 256 workgroups)
    ([32], 256, 192),
    ([300], 512, 768),
    ([100], 256, 1408),
    ([70, 0, 130], 4096, 1408),
    ([40, 0, 0, 200], 256, 256),
    ([16500, 16524], 256, 768),
    # many small experts on 256 x 384 tiles: store-bound (the jobs' K steps sum to less than their
    # fixed costs), so the one-launch form starts with dphi units and claims dW units from one
    # counter; empty experts write zeros
    ([2000, 1500, 0, 3, 40, 700, 1] + [5] * 40 + [0] * 10, 2048, 768),
    ([2500, 30, 0, 1200, 64, 0] + [33] * 20, 2048, 768),
    # one expert far above the fair share, not store-bound: the dW schedule's contiguous fill
    # splits it along K into partial slots that the one-launch form's second launch adds up
    ([12000] + [40] * 15, 2048, 768),
    # a few large experts whose dphi units fit in one round of the grid (90 units on 256
    # workgroups): the schedule estimates that starting them first ends sooner, so the one-launch
    # form takes the dphi-first order with dW tiles claimed largest expert first, unsplit
    ([1568] * 5 + [702, 250, 76, 14, 10, 2, 3, 1, 0, 0, 0], 2048, 768),
    # many short experts, more dphi units than workgroups (280 on 256) and every dW job cheaper
    # than a dphi unit: the dphi-first order again, now over more than one round
    ([300] * 70, 2048, 768),
]


@pytest.mark.parametrize("Ke,h,d", GEMM_SHAPES,
                         ids=[f"E{len(k)}-K{sum(k)}-h{h}-d{d}" for k, h, d in GEMM_SHAPES])
def test_grouped_gemms_shapes(Ke, h, d):
    """lrm_grouped_dw / lrm_grouped_dx on seeded bf16 segments against the float64 oracle."""
    _check_grouped_gemms(Ke, h, d)


def _seeded_shape(seed):
    """Retained rows per expert (1-40 experts: a power-law skew, near-uniform, a few large experts
    over a tail, or mostly empty) and a product shape, drawn from `seed`."""
    r = np.random.default_rng(seed)
    E = int(r.integers(1, 41))
    h = int(r.choice([256, 512, 1024, 2048]))
    d = int(r.choice([192, 256, 384, 768]))
    kind = int(r.integers(0, 4))
    if kind == 0:
        w = 1.0 / np.arange(1, E + 1) ** r.uniform(0.5, 2.0)
    elif kind == 1:
        w = r.uniform(0.5, 1.5, E)
    elif kind == 2:
        nb = int(r.integers(1, min(E, 5) + 1))
        w = np.concatenate([r.uniform(5, 10, nb), r.uniform(0, 0.3, E - nb)])
    else:
        w = r.uniform(0, 1, E) * (r.uniform(0, 1, E) < 0.3)
    K = int(r.integers(200, 24000 // max(1, h // 512)))
    if w.sum() == 0:
        w[0] = 1.0
    return np.floor(w / w.sum() * K).astype(int).tolist(), h, d


# Seeds whose shapes take each order of the one-launch form under its schedule's rules: dphi
# first after an estimate (0, 14, 21), dW first with experts split along K (1, 11), store-bound
# (4, 5).
SEEDED_SHAPES = [0, 1, 4, 5, 11, 14, 21]


@pytest.mark.parametrize("seed", SEEDED_SHAPES)
def test_grouped_gemms_seeded_shapes(seed):
    """The grouped GEMMs on seeded random segment sizes: both forms give the same bits, and both
    match the float64 oracle."""
    Ke, h, d = _seeded_shape(seed)
    _check_grouped_gemms(Ke, h, d)


def _check_grouped_gemms(Ke, h, d):
    torch = _torch()
    from backward_token_expert_amd import lrm
    from backward_token_expert_amd.path import to_device, to_host
    rng = np.random.default_rng(sum(Ke) + h + d)
    K, E_loc = sum(Ke), len(Ke)
    co = np.concatenate([[0], np.cumsum(Ke)]).astype(np.int32)
    Gc = O.f32_to_bf16_rne(rng.standard_normal((K, h)).astype(np.float32))
    Ph = O.f32_to_bf16_rne(rng.standard_normal((K, d)).astype(np.float32))
    W = O.f32_to_bf16_rne((rng.standard_normal((E_loc, h, d)) / np.sqrt(d)).astype(np.float32))
    P = lrm.make_problem(max(K, 1), 1, E_loc, 0, E_loc, h, d, "bf16", max(K, 1), max(K, 1))
    ws = torch.zeros(lrm.lrm_workspace_bytes(P), dtype=torch.uint8, device="cuda")
    dW = torch.full((E_loc, h, d), 7.0, device="cuda")
    dphi = torch.zeros((K, d), device="cuda")
    print(f"[case] grouped GEMMs Ke={Ke} h={h} d={d}", flush=True)
    cod = to_device(co)
    Gd, Pd, Wd = to_device(Gc), to_device(Ph), to_device(W)
    lrm.lrm_grouped_dw(P, Gd, Pd, cod, dW, ws)
    lrm.lrm_grouped_dx(P, Gd, Wd, cod, dphi, ws)
    # the one-launch form must give the same bits
    dW2 = torch.full((E_loc, h, d), -3.0, device="cuda")
    dphi2 = torch.full((K, d), -3.0, device="cuda")
    lrm.lrm_grouped_dw_dx(P, Gd, Pd, Wd, cod, dW2, dphi2, ws)
    torch.cuda.synchronize()
    gW, gx = to_host(dW), to_host(dphi)
    assert to_host(dW2).tobytes() == gW.tobytes()
    assert to_host(dphi2).tobytes() == gx.tobytes()
    rW = O.grouped_dw(Gc, Ph, co, "bf16")
    rx = O.grouped_dx(Gc, W, co, "bf16")
    tol = C.tol_for("bf16")
    for e in range(E_loc):
        if Ke[e] == 0:
            assert not gW[e].any(), f"expert {e} has no rows but nonzero dW"
            continue
        assert C.rel_fro(gW[e], rW[e]) <= tol, (e, C.rel_fro(gW[e], rW[e]))
        s, t = co[e], co[e + 1]
        assert C.rel_fro(gx[s:t], rx[s:t]) <= tol, (e, C.rel_fro(gx[s:t], rx[s:t]))


def test_compaction_ignores_map_entries_of_earlier_calls():
    """The pair -> row map in the workspace is never cleared: calls with different selections on
    one workspace must each match the oracle's compaction of their own selection."""
    from backward_token_expert_amd import path
    from backward_token_expert_amd.path import to_host
    w = C.workload(1, T=2048)
    sp = w.spec
    P = C.problem(sp)
    bufs = path.DeviceBuffers(P)
    inp = C.upload(w)
    for full, rho in ((False, (1, 2)), (False, (1, 8)), (True, None), (False, (1, 3))):
        pol = synth.policy(sp, full=full, rho=rho)
        print(f"[case] compaction on a reused workspace, full={full} rho={rho}", flush=True)
        o = C.oracle_run(w, pol, gemms=False)
        K = int(o["cmp_off"][-1])
        err = _compact_with(P, bufs, inp, o["sel_row"], o["row_pair"], K)
        assert err == 0
        bf = sp.dtype == "bf16"
        g = dict(sel_row=o["sel_row"], sel_pair=to_host(bufs.sel_pair)[:K],
                 Gc=to_host(bufs.Gc, bf)[:K], Phic=to_host(bufs.Phic, bf)[:K])
        check_compact(g, o)


def test_compaction_flags_unordered_or_shared_pairs():
    from backward_token_expert_amd import path
    from backward_token_expert_amd.path import to_host
    w = C.workload(1, T=1024)
    sp = w.spec
    P = C.problem(sp)
    bufs = path.DeviceBuffers(P)
    inp = C.upload(w)
    o = C.oracle_run(w, synth.policy(sp), gemms=False)
    K = int(o["cmp_off"][-1])
    sel, rp = o["sel_row"].copy(), o["row_pair"].copy()
    print("[case] compaction of an in-order selection", flush=True)
    assert _compact_with(P, bufs, inp, sel, rp, K) == 0
    print("[case] compaction of a selection with two rows swapped", flush=True)
    bad = sel.copy()
    bad[[10, 11]] = bad[[11, 10]]
    assert _compact_with(P, bufs, inp, bad, rp, K) & 32
    print("[case] compaction with two selected rows naming one pair", flush=True)
    rp2 = rp.copy()
    rp2[sel[20]] = rp2[sel[21]]
    assert _compact_with(P, bufs, inp, sel, rp2, K) & 32
    print("[case] compaction with a selected row out of range", flush=True)
    bad = sel.copy()
    bad[-1] = P.L_cap
    assert _compact_with(P, bufs, inp, bad, rp, K) & 32
    assert to_host(bufs.sel_pair)[K - 1] == -1


# ------------------------------------------------------------------------------------------------
# determinism and graph capture
# ------------------------------------------------------------------------------------------------

def test_bitwise_determinism_and_graph_replay():
    torch = _torch()
    from backward_token_expert_amd import path
    w = C.workload(1, T=2048)
    sp = w.spec
    pol = C.policy_obj(synth.policy(sp))
    P = C.problem(sp)
    inp = C.upload(w)
    outs = []
    for fused in (True, True, False):
        b = path.DeviceBuffers(P)
        path.run(P, pol, inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"], b,
                 fused=fused)
        torch.cuda.synchronize()
        outs.append(host(b, sp))
    for key in outs[0]:
        assert outs[0][key].tobytes() == outs[2][key].tobytes(), ("separate GEMM calls", key)
    for key in outs[0]:
        assert outs[0][key].tobytes() == outs[1][key].tobytes(), key
    # capture the six calls in a graph and replay it; every replay must equal the eager result
    b = path.DeviceBuffers(P)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        path.run(P, pol, inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"], b, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            path.run(P, pol, inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"], b, s)
    for rep in range(3):
        b.dW.fill_(7.0)
        b.sel_row.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(b, sp)
        for key in got:
            assert got[key].tobytes() == outs[0][key].tobytes(), (rep, key)


def test_score_halves_on_a_side_stream():
    """lrm_score_norms on a second stream beside lrm_plan_quotas, then lrm_score_combine, gives
    every output of the one-stream sequence bit for bit; phi rows past L (NaN here) reach no score
    and set no error; the forked sequence captures into one HIP graph whose replays (with eager
    work between them) equal the eager result."""
    torch = _torch()
    from backward_token_expert_amd import lrm, path
    w = C.workload(3, T=2048)          # extreme skew: empty experts, L well below L_cap
    sp = w.spec
    pol = C.policy_obj(synth.policy(sp))
    P = C.problem(sp)
    inp = dict(C.upload(w))
    L = w.phi.shape[0]
    assert L < P.L_cap
    nan = 0x7FC0 if sp.dtype == "bf16" else float("nan")
    inp["phi"][L:] = nan
    args = (P, pol, inp["topk_idx"], inp["topk_w"], inp["g"], inp["phi"], inp["W"])
    ref = path.DeviceBuffers(P)
    path.run(*args, ref)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(ref.ws) == 0
    want = host(ref, sp)
    side = torch.cuda.Stream()
    b = path.DeviceBuffers(P)
    path.run(*args, b, side_stream=side)
    torch.cuda.synchronize()
    assert lrm.lrm_read_device_error(b.ws) == 0
    got = host(b, sp)
    for key in want:
        assert got[key].tobytes() == want[key].tobytes(), key
    # the two halves back to back on one stream
    b.score.fill_(-1.0)
    lrm.lrm_score_norms(P, inp["g"], inp["phi"], b.ws)
    lrm.lrm_score_combine(P, inp["topk_w"], b.row_pair, b.fwd_off, b.score, b.ws)
    torch.cuda.synchronize()
    assert host(b, sp)["score"].tobytes() == want["score"].tobytes()
    # the forked sequence in one graph
    g = path.DeviceBuffers(P)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        path.run(*args, g, s, side_stream=side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            path.run(*args, g, s, side_stream=side)
    for rep in range(3):
        g.score.fill_(-1.0)
        g.dW.fill_(7.0)
        g.sel_row.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(g, sp)
        for key in got:
            assert got[key].tobytes() == want[key].tobytes(), (rep, key)
        assert lrm.lrm_read_device_error(g.ws) == 0


def test_full_size_score_halves_on_a_side_stream_match_one_stream():
    # the Qwen3 share at full size: the forked sequence (bench.py --overlap) against the one-stream
    # sequence bench.py times by default, every output bit for bit
    w = C.workload(1)
    sp = w.spec
    pol = synth.policy(sp)
    print("[case] full-size cfg1, score halves on a side stream", flush=True)
    _, b1, _, e1 = run_gpu(w, pol)
    _, b2, _, e2 = run_gpu(w, pol, overlap=True)
    assert e1 == 0 and e2 == 0
    h1, h2 = host(b1, sp), host(b2, sp)
    for key in h1:
        assert h1[key].tobytes() == h2[key].tobytes(), key


# ------------------------------------------------------------------------------------------------
# full-size workloads (the launch configuration bench.py times): every output compared in full
# ------------------------------------------------------------------------------------------------

FULL = [(0, None), (1, None), (2, None), (3, (1, 1)), (3, (3, 4)), (3, (1, 2)), (3, (1, 4)),
        (4, None), (5, None)]
# every workload at its own retention (the extreme skew at each sweep point), and once per
# workload at full retention
FULL_CASES = sorted([(c, r, False) for c, r in FULL] +
                    [(c, r, True) for c, r in FULL if r in (None, (1, 2))], key=lambda x: x[0])


@pytest.mark.parametrize("cfg,rho,full", FULL_CASES,
                         ids=[f"cfg{c}-{r}-{'rho1' if f else 'cfg-rho'}" for c, r, f in FULL_CASES])
def test_full_size(cfg, rho, full):
    w = C.workload(cfg)
    sp = w.spec
    pol = synth.policy(sp, full=full, rho=rho)
    print(f"[case] full-size cfg{cfg} rho={rho} full={full}", flush=True)
    P, bufs, inp, err = run_gpu(w, pol)
    assert err == 0, f"device error {err}"
    o = C.oracle_run(w, pol, gemms=False)
    g = host(bufs, sp)
    check_plan(g, o)
    nd = check_scores(g, o)
    print(f"  scores differing in float32 bits from the oracle's rounding: {nd}", flush=True)
    check_selection_valid(g, o)
    gate_select(P, bufs, o)
    if np.array_equal(g["sel_row"], o["sel_row"]):
        check_compact(g, o)
        check_gemms(g, o, w.W, sp.dtype)
    else:
        gate_compact_gemms(P, bufs, inp, o, w.W, sp.dtype)
