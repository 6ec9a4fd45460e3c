"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something the pages or mathematics fix independently: the
pages' worked examples (golden files), closed forms (the rank-one identity, the Gram identity,
the exact derivative of a linear loss), invariants, a library routine (torch's float->bfloat16
rounding), and brute force over all subsets in exact rational arithmetic.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16_bits(x):
    return O.f32_to_bf16_rne(np.asarray(x, np.float32))


def _tiny_problem(rng, T=40, k=3, E=6, e_lo=1, E_loc=4, h=8, d=8, dtype="bf16"):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(-1)
    w = rng.random((T, k)).astype(np.float32)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)
    row_pair, fwd_off = O.forward_layout(idx, e_lo, E_loc)
    L = row_pair.size
    g32 = rng.standard_normal((T, h)).astype(np.float32)
    p32 = rng.standard_normal((L, d)).astype(np.float32)
    W32 = (rng.standard_normal((E_loc, h, d)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        g, phi, W = _bf16_bits(g32), _bf16_bits(p32), _bf16_bits(W32)
    else:
        g, phi, W = g32, p32, W32
    return dict(idx=idx, w=w, g=g, phi=phi, W=W, row_pair=row_pair, fwd_off=fwd_off, T=T, k=k,
                E=E, e_lo=e_lo, E_loc=E_loc, h=h, d=d, dtype=dtype)


# ---------------------------------------------------------------------------------------------
# counts, layout, quotas: the pages' worked examples
# ---------------------------------------------------------------------------------------------

def test_expert_parallel_math_worked_example():
    gx = _gold("expert_parallel_math_worked_example.json")
    E, k, T = gx["E"], gx["k"], gx["T"]
    n = np.asarray(gx["n"])
    idx = np.repeat(np.arange(E), n)
    np.random.default_rng(0).shuffle(idx)
    cnt = O.routed_counts(idx, E)
    assert cnt.tolist() == gx["n"]
    assert cnt.sum() == T * k                      # sum_i n_i = T*k
    pol = {"full": 0, "rho_num": gx["capacity_factor_num"], "rho_den": gx["capacity_factor_den"],
           "cap_abs": -1}
    q, off = O.plan_quotas(cnt, pol)
    assert int(q.max()) == gx["C"]                 # C = CF * T*k/E = 20480
    assert q.tolist() == [min(v, gx["C"]) for v in gx["n"]]
    assert int(q.sum()) == gx["real_carried"]
    assert int((cnt - q).sum()) == gx["dropped"]
    assert round(100.0 * gx["dropped"] / (T * k), 2) == gx["drop_rate_percent_rounded"]
    assert E * gx["C"] == gx["slots_moved"]
    assert round(100.0 * int(q.sum()) / gx["slots_moved"]) == gx["utilization_percent_rounded"]
    assert off.tolist() == [0] + np.cumsum(q).tolist()


def test_fig4_counts_layout_offsets():
    gx = _gold("lrmoe_fig4_pack.json")
    idx = np.asarray(gx["pre_drop_experts"], np.int32)
    cnt = O.routed_counts(idx, 3)
    assert cnt.tolist() == gx["loads"]
    row_pair, fwd_off = O.forward_layout(idx, 0, 3)
    assert fwd_off.tolist() == [0, 4, 6, 9]
    assert row_pair.tolist() == [0, 2, 5, 8, 3, 6, 1, 4, 7]
    q, off = O.plan_quotas(np.asarray(gx["retained"]), {"full": 1})
    assert q.tolist() == gx["retained"] and off.tolist() == gx["offsets"]


def test_counts_reject_bad_ids():
    with pytest.raises(ValueError):
        O.routed_counts(np.array([0, 3]), 3)
    with pytest.raises(ValueError):
        O.routed_counts(np.array([-1, 0]), 3)


def test_layout_is_stable_permutation():
    rng = np.random.default_rng(1)
    P = _tiny_problem(rng, T=300, k=4, E=10, e_lo=3, E_loc=5)
    idx, rp, off = P["idx"], P["row_pair"], P["fwd_off"]
    local = np.flatnonzero((idx >= 3) & (idx < 8))
    assert sorted(rp.tolist()) == local.tolist()
    for i in range(5):
        seg = rp[off[i]:off[i + 1]]
        assert np.all(idx[seg] == 3 + i)
        assert np.all(np.diff(seg) > 0)
    assert off[-1] == local.size


def test_quota_integer_floor_and_caps():
    # floor(29*100/(100*1)) = 29 exactly; 0.29*100 in binary floating point is 28.999...
    q, _ = O.plan_quotas(np.array([100]), {"full": 0, "rho_num": 29, "rho_den": 100, "cap_abs": -1})
    assert q.tolist() == [29]
    # tiny fp32 workload recipe: floor(0.6 * 8192/8) = 614
    q, _ = O.plan_quotas(np.array([3556, 2100, 1114, 529, 355, 237, 165, 136]),
                         {"full": 0, "rho_num": 3, "rho_den": 5, "cap_abs": -1})
    assert q.tolist() == [614, 614, 614, 529, 355, 237, 165, 136]
    # an absolute cap binds below the proportional one
    q, off = O.plan_quotas(np.array([50, 5, 0, 45]), {"full": 0, "rho_num": 1, "rho_den": 1,
                                                      "cap_abs": 10})
    assert q.tolist() == [10, 5, 0, 10] and off.tolist() == [0, 10, 15, 15, 25]
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = rng.integers(0, 1000, size=rng.integers(1, 20))
        num, den = int(rng.integers(0, 9)), int(rng.integers(1, 9))
        q, off = O.plan_quotas(n, {"full": 0, "rho_num": num, "rho_den": den, "cap_abs": -1})
        assert np.all(q >= 0) and np.all(q <= n)
        assert np.all(q == np.minimum(n, (num * int(n.sum())) // (den * n.size)))
        qf, _ = O.plan_quotas(n, {"full": 1})
        assert np.array_equal(qf, n)


def test_fig4_proportional_quotas():
    # Fig. 4: loads [4, 2, 3] reduced to [3, 1, 2]; a retained total of 6 of 9 (rho = 2/3) split
    # in proportion to the loads gives exactly that, and no cap C reproduces it
    gx = _gold("lrmoe_fig4_pack.json")
    loads = np.asarray(gx["loads"])
    q, off = O.plan_quotas(loads, {"full": 0, "kind": "proportional", "rho_num": 2, "rho_den": 3,
                                   "cap_abs": -1})
    assert q.tolist() == gx["retained"] and off.tolist() == gx["offsets"]
    for c in range(0, 5):
        assert np.minimum(loads, c).tolist() != gx["retained"]
    with pytest.raises(ValueError):
        O.plan_quotas(loads, {"kind": "proportional", "rho_num": 1, "rho_den": 2, "cap_abs": 3})


def _brute_split(bounds, total, cost):
    """All integer vectors 0 <= q <= bounds with sum(q) == total; minimise cost(q) exactly, ties
    to the lexicographically largest q (the lower expert first)."""
    best = None
    for q in itertools.product(*(range(b + 1) for b in bounds)):
        if sum(q) != total:
            continue
        key = (cost(q), tuple(-v for v in q))
        if best is None or key < best[0]:
            best = (key, list(q))
    return best[1]


def test_proportional_quotas_are_closest_integer_split():
    # largest remainder = the integer split with sum B closest (in squared distance) to the exact
    # shares B*n_e/L; brute force over every split in exact rationals
    rng = np.random.default_rng(21)
    for trial in range(150):
        n = [int(v) for v in rng.integers(0, 7, size=int(rng.integers(1, 5)))]
        L = sum(n)
        num, den = int(rng.integers(0, 5)), int(rng.integers(1, 5))
        B = min(L, num * L // den)
        pol = {"full": 0, "kind": "proportional", "rho_num": num, "rho_den": den, "cap_abs": -1}
        q, off = O.plan_quotas(np.asarray(n), pol)
        assert int(q.sum()) == B and off[-1] == B
        if L == 0:
            assert not q.any()
            continue
        share = [Fraction(B * v, L) for v in n]
        ref = _brute_split(n, B, lambda qq: sum((a - b) ** 2 for a, b in zip(qq, share)))
        assert q.tolist() == ref, (n, B)
        for v, x in zip(q.tolist(), share):              # quota property: floor <= q <= ceil
            assert x - 1 < v < x + 1


def test_waterfill_quotas_are_most_level_split():
    # water-fill = the split of min(B, sum m) with 0 <= q <= m = min(n, cap) that minimises the
    # sum of squares (the most level one); brute force over every split
    rng = np.random.default_rng(22)
    for trial in range(150):
        n = [int(v) for v in rng.integers(0, 8, size=int(rng.integers(1, 5)))]
        cap = int(rng.choice([-1, 2, 4]))
        num, den = int(rng.integers(0, 5)), int(rng.integers(1, 5))
        L = sum(n)
        B = min(L, num * L // den)
        m = [v if cap < 0 else min(v, cap) for v in n]
        pol = {"full": 0, "kind": "waterfill", "rho_num": num, "rho_den": den, "cap_abs": cap}
        q, _ = O.plan_quotas(np.asarray(n), pol)
        ref = _brute_split(m, min(B, sum(m)), lambda qq: sum(v * v for v in qq))
        assert q.tolist() == ref, (n, cap, B)
    # a level below the cap, and the cap binding with budget to spare
    pol = {"full": 0, "kind": "waterfill", "rho_num": 1, "rho_den": 2, "cap_abs": -1}
    assert O.plan_quotas(np.array([50, 5, 0, 45]), pol)[0].tolist() == [23, 5, 0, 22]
    pol = {"full": 0, "kind": "waterfill", "rho_num": 1, "rho_den": 1, "cap_abs": 30}
    assert O.plan_quotas(np.array([50, 5, 0, 45]), pol)[0].tolist() == [30, 5, 0, 30]


# ---------------------------------------------------------------------------------------------
# scores: rank-one identity (Prop. 3.1 / Appendix 7.1 Eq. (11)-(12))
# ---------------------------------------------------------------------------------------------

def test_bf16_widen_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F], np.uint16)
    v = O.widen(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 1.0 + 2.0 ** -7 and v[3] == 0.0
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scores_equal_frobenius_norm_of_materialised_contribution(dtype):
    rng = np.random.default_rng(3)
    P = _tiny_problem(rng, dtype=dtype)
    R = O.lrm_scores(P["w"], P["g"], P["phi"], P["row_pair"], P["k"], dtype)
    gw, pw = O.widen(P["g"], dtype), O.widen(P["phi"], dtype)
    for r, p in enumerate(P["row_pair"]):
        t, j = divmod(int(p), P["k"])                     # p = t*k + j
        alpha = float(np.float32(P["w"][t * P["k"] + j]))
        G = np.outer(alpha * gw[t], pw[r])               # G_u = (alpha_u g_t) phi_u^T
        fro2 = float((G * G).sum())
        assert abs(R[r] - fro2) <= 1e-12 * fro2


def test_scores_scale_homogeneity_and_token_sharing():
    rng = np.random.default_rng(4)
    P = _tiny_problem(rng, dtype="f32")
    args = (P["w"], P["g"], P["phi"], P["row_pair"], P["k"], "f32")
    R = O.lrm_scores(*args)
    R_a = O.lrm_scores(P["w"] * np.float32(2), *args[1:])
    R_g = O.lrm_scores(P["w"], P["g"] * np.float32(4), *args[2:])
    R_p = O.lrm_scores(P["w"], P["g"], P["phi"] * np.float32(0.5), *args[3:])
    np.testing.assert_allclose(R_a, 4 * R, rtol=1e-14)
    np.testing.assert_allclose(R_g, 16 * R, rtol=1e-14)
    np.testing.assert_allclose(R_p, 0.25 * R, rtol=1e-14)
    # pairs of one token share ||g_t||^2: R / (alpha^2 ||phi||^2) depends on t only
    rp = P["row_pair"]
    a = P["w"][rp].astype(np.float64)
    pn = (P["phi"].astype(np.float64) ** 2).sum(1)
    gn = R / (a * a * pn)
    gt = (P["g"].astype(np.float64) ** 2).sum(1)[rp // P["k"]]
    np.testing.assert_allclose(gn, gt, rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# Table 2's alternative criteria
# ---------------------------------------------------------------------------------------------

def test_gradient_criteria_closed_forms():
    # rows of known norms: (3, -4, 0...) -> ||.||_2^2 = 25, ||.||_1 = 7; a constant row of +-c
    # reaches ||g||_1^2 = h ||g||_2^2; one non-zero entry gives ||g||_1 = ||g||_2
    h, k = 16, 2
    g = np.zeros((4, h), np.float32)
    g[0, :2] = [3, -4]
    g[1] = 0.5 * np.where(np.arange(h) % 2 == 0, 1.0, -1.0)
    g[2, 7] = -2.0
    row_pair = np.array([0, 1, 2, 3, 4, 5, 6, 7])
    sq = O.grad_sq_scores(g, row_pair, k, "f32")
    ab = O.grad_abs_scores(g, row_pair, k, "f32")
    assert sq.tolist() == [25, 25, 4, 4, 4, 4, 0, 0]
    assert ab.tolist() == [7, 7, 8, 8, 2, 2, 0, 0]
    assert ab[2] ** 2 == h * sq[2] and ab[4] ** 2 == sq[4]
    gb = _bf16_bits(g)                                    # exact in bf16 as well
    assert O.grad_sq_scores(gb, row_pair, k, "bf16").tolist() == sq.tolist()
    assert O.grad_abs_scores(gb, row_pair, k, "bf16").tolist() == ab.tolist()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_criteria_ignore_weight_and_activation(dtype):
    # gradient-only rules (Sec. 4.7): independent of alpha and phi; norm inequalities
    # ||g||_2 <= ||g||_1 <= sqrt(h) ||g||_2; ||g||_2^2 is the LRM score at alpha = 1, ||phi|| = 1
    rng = np.random.default_rng(23)
    P = _tiny_problem(rng, dtype=dtype)
    rp, k, h = P["row_pair"], P["k"], P["h"]
    for crit in ("grad_sq", "grad_abs"):
        a = O.scores(crit, P["w"], P["g"], P["phi"], rp, k, dtype)
        b = O.scores(crit, P["w"] * np.float32(3), P["g"], P["phi"][::-1].copy(), rp, k, dtype)
        np.testing.assert_array_equal(a, b)
    sq = O.grad_sq_scores(P["g"], rp, k, dtype)
    ab = O.grad_abs_scores(P["g"], rp, k, dtype)
    assert np.all(np.sqrt(sq) <= ab * (1 + 1e-15)) and np.all(ab <= np.sqrt(h * sq) * (1 + 1e-15))
    unit = np.zeros_like(P["phi"])
    unit[:, 0] = _bf16_bits([1.0])[0] if dtype == "bf16" else 1.0
    R = O.lrm_scores(np.ones_like(P["w"]), P["g"], unit, rp, k, dtype)
    np.testing.assert_array_equal(R, sq)
    t = rp // k                                           # pairs of one token share the score
    for tt in np.unique(t):
        assert np.unique(sq[t == tt]).size == 1


def test_random_criterion_keeps_uniform_subsets():
    # random drop: with independent uniform keys, each of an expert's n rows is kept with
    # probability q/n; over 4000 draws every row's count stays within 5 sigma of 4000 q/n, and
    # the kept set never depends on g or phi
    rng = np.random.default_rng(24)
    n_e, q_e = [10, 7], [3, 6]
    off = [0, 10, 17]
    rp = np.arange(17) * 2
    hits = np.zeros(17)
    draws = 4000
    for _ in range(draws):
        keys = rng.random(40).astype(np.float32)
        s = O.random_scores(keys, rp).astype(np.float32)
        sel = O.select_top_quota(s, off, q_e, rp)
        hits[sel] += 1
    for e in range(2):
        pr = q_e[e] / n_e[e]
        sd = np.sqrt(draws * pr * (1 - pr))
        assert np.all(np.abs(hits[off[e]:off[e + 1]] - draws * pr) <= 5 * sd)
    P = _tiny_problem(rng, dtype="bf16")
    keys = rng.random(P["T"] * P["k"]).astype(np.float32)
    a = O.scores("random", P["w"], P["g"], P["phi"], P["row_pair"], P["k"], "bf16", keys)
    b = O.scores("random", P["w"], P["g"][::-1].copy(), P["phi"] * 0, P["row_pair"], P["k"], "bf16",
                 keys)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a.astype(np.float32), keys[P["row_pair"]])
    with pytest.raises(ValueError):
        O.scores("random", P["w"], P["g"], P["phi"], P["row_pair"], P["k"], "bf16")


# ---------------------------------------------------------------------------------------------
# selection: Prop. 7.1 and brute force over all subsets (exact rationals)
# ---------------------------------------------------------------------------------------------

def _brute_select(score32, pairs, q):
    """All q-subsets; maximise the exact sum, break ties by the lexicographically smallest
    ascending pair list (the pair-index-ascending tie-break)."""
    vals = [Fraction(float(s)) for s in np.asarray(score32, np.float32)]
    best = None
    for sub in itertools.combinations(range(len(vals)), q):
        s = sum((vals[i] for i in sub), Fraction(0))
        key = (-s, sorted(int(pairs[i]) for i in sub))
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1])


def test_select_matches_exhaustive_search():
    rng = np.random.default_rng(5)
    for trial in range(120):
        n = int(rng.integers(0, 12))
        q = int(rng.integers(0, n + 1))
        if trial % 3 == 0:      # heavy ties, straddling the boundary
            s = rng.choice(np.float32([0.5, 1.0, 1.0, 2.0, 0.0]), size=n).astype(np.float32)
        else:
            s = (rng.random(n) * rng.choice([1e-3, 1.0, 1e3])).astype(np.float32)
        pairs = np.sort(rng.choice(1000, size=n, replace=False))   # ascending within an expert
        sel = O.select_top_quota(s, [0, n], [q], pairs)
        assert sel.tolist() == _brute_select(s, pairs, q)


def test_select_exchange_optimality_and_special_cases():
    rng = np.random.default_rng(6)
    n_e = [0, 1, 7, 64, 65, 300]
    off = np.concatenate([[0], np.cumsum(n_e)])
    L = int(off[-1])
    rp = np.arange(L) * 3 + 1                   # ascending pair ids
    s = rng.random(L).astype(np.float32)
    s[off[4]:off[5]] = np.float32(0.25)         # an all-equal segment
    q = [0, 1, 3, 64, 10, 150]
    sel = O.select_top_quota(s, off, q, rp)
    assert sel.size == sum(q)
    pos = 0
    for e in range(len(n_e)):
        rows = np.arange(off[e], off[e + 1])
        kept = sel[pos:pos + q[e]]
        pos += q[e]
        assert np.all(np.diff(kept) > 0)
        dropped = np.setdiff1d(rows, kept)
        if kept.size and dropped.size:          # Prop. 7.1: min kept >= max dropped
            assert s[kept].min() >= s[dropped].max()
    seg4 = sel[sum(q[:4]):sum(q[:5])]
    assert seg4.tolist() == list(range(off[4], off[4] + 10))    # all equal -> first q rows
    assert sel[sum(q[:3]):sum(q[:4])].tolist() == list(range(off[3], off[4]))  # q = n
    with pytest.raises(ValueError):
        O.select_top_quota(s, off, [0, 2, 0, 0, 0, 0], rp)      # q > n


# ---------------------------------------------------------------------------------------------
# compaction: byte-exact against a naive per-row gather with torch's bf16 rounding
# ---------------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_and_ties_to_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.4028235e38, 0.0, -0.0,
                    1e-40, 2 ** -133]),
    ]).astype(np.float32)
    ours = O.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-8] == 0x3F80 and ours[-7] == 0x3F82          # ties go to the even mantissa
    assert ours[-5] == 0x7F80                                 # rounds up to infinity


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compact_matches_naive_gather(dtype):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    P = _tiny_problem(rng, T=60, dtype=dtype)
    n = O.routed_counts(P["idx"], P["E"])[P["e_lo"]:P["e_lo"] + P["E_loc"]]
    q, off = O.plan_quotas(n, {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1})
    R = O.lrm_scores(P["w"], P["g"], P["phi"], P["row_pair"], P["k"], dtype).astype(np.float32)
    sel = O.select_top_quota(R, P["fwd_off"], q, P["row_pair"])
    Gc, Phic, sp = O.compact(sel, P["row_pair"], P["w"], P["g"], P["phi"], P["k"], dtype)
    assert Gc.shape[0] == int(off[-1]) == sel.size
    for i, r in enumerate(sel):
        p = int(P["row_pair"][r])
        t = p // P["k"]
        assert sp[i] == p
        assert Phic[i].tobytes() == P["phi"][r].tobytes()
        a = torch.tensor(float(P["w"][p]), dtype=torch.float32)
        if dtype == "f32":
            ref = (a * torch.from_numpy(P["g"][t])).numpy()
            assert Gc[i].tobytes() == ref.tobytes()
        else:
            g32 = torch.from_numpy(P["g"][t].view(np.int16)).view(torch.bfloat16).float()
            ref = (a * g32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert Gc[i].tobytes() == ref.tobytes()


# ---------------------------------------------------------------------------------------------
# gradients: zero-masked equivalence, Gram identity, exact derivative of a linear loss
# ---------------------------------------------------------------------------------------------

def _path(P, pol):
    n = O.routed_counts(P["idx"], P["E"])[P["e_lo"]:P["e_lo"] + P["E_loc"]]
    q, off = O.plan_quotas(n, pol)
    R = O.lrm_scores(P["w"], P["g"], P["phi"], P["row_pair"], P["k"], P["dtype"]).astype(np.float32)
    sel = O.select_top_quota(R, P["fwd_off"], q, P["row_pair"])
    Gc, Phic, sp = O.compact(sel, P["row_pair"], P["w"], P["g"], P["phi"], P["k"], P["dtype"])
    return q, off, sel, Gc, Phic


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compact_gemm_equals_zero_masked_gemm(dtype):
    # Sec. 3.4: the compacted GEMM equals the zero-masked full-size GEMM for the same retained set.
    rng = np.random.default_rng(9)
    P = _tiny_problem(rng, T=80, h=16, d=12, dtype=dtype)
    q, off, sel, Gc, Phic = _path(P, {"full": 0, "rho_num": 1, "rho_den": 3, "cap_abs": -1})
    dW = O.grouped_dw(Gc, Phic, off, dtype)
    dX = O.grouped_dx(Gc, P["W"], off, dtype)
    # full-size tensors over every forward row, dropped rows masked to zero
    allrows = np.arange(P["row_pair"].size)
    Gf, Pf, _ = O.compact(allrows, P["row_pair"], P["w"], P["g"], P["phi"], P["k"], dtype)
    mask = np.zeros(allrows.size)
    mask[sel] = 1.0
    Gm = O.widen(Gf, dtype) * mask[:, None]
    Pm = O.widen(Pf, dtype)
    fo = P["fwd_off"]
    for e in range(P["E_loc"]):
        ref = Gm[fo[e]:fo[e + 1]].T @ Pm[fo[e]:fo[e + 1]]
        np.testing.assert_allclose(dW[e], ref, rtol=1e-12, atol=1e-12)
        refx = Gm[fo[e]:fo[e + 1]] @ O.widen(P["W"][e], dtype)
        kept = sel[(sel >= fo[e]) & (sel < fo[e + 1])]
        np.testing.assert_allclose(dX[off[e]:off[e + 1]], refx[kept - fo[e]], rtol=1e-12, atol=1e-12)


def test_gram_identity_and_rank_one_expert():
    # Appendix 7.3, Eq. (19): ||sum_u G_u||^2 = sum_{u,v} <G_u, G_v> with <G_u,G_v> = (d_u.d_v)(p_u.p_v)
    rng = np.random.default_rng(10)
    P = _tiny_problem(rng, T=50, h=10, d=6, dtype="f32")
    q, off, sel, Gc, Phic = _path(P, {"full": 1})
    dW = O.grouped_dw(Gc, Phic, off, "f32")
    D, Ph = Gc.astype(np.float64), Phic.astype(np.float64)
    for e in range(P["E_loc"]):
        s, t = off[e], off[e + 1]
        gram = sum(float(D[u] @ D[v]) * float(Ph[u] @ Ph[v]) for u in range(s, t) for v in range(s, t))
        fro2 = float((dW[e] ** 2).sum())
        assert abs(fro2 - gram) <= 1e-11 * max(gram, 1e-300)
    # one retained row: ||dW_e||^2 = ||delta||^2 ||phi||^2 (Eq. (11))
    one = O.grouped_dw(Gc[:1], Phic[:1], [0, 1], "f32")[0]
    assert abs((one ** 2).sum() - (D[0] @ D[0]) * (Ph[0] @ Ph[0])) <= 1e-12 * (one ** 2).sum()
    # no retained rows: exact zeros
    z = O.grouped_dw(Gc[:0], Phic[:0], [0, 0], "f32")
    assert z.shape == (1, Gc.shape[1], Phic.shape[1]) and not z.any()


@pytest.mark.parametrize("hd", [(8, 8), (12, 5)])
def test_gradients_are_exact_derivatives_of_linear_loss(hd):
    # Appendix 7.1, Eq. (6)-(8): with y_u = W_e phi_u weighted by delta_u, the loss
    # F(W, phi) = sum_u <delta_u, W_e phi_u> has dF/dW_e = sum_u delta_u phi_u^T and
    # dF/dphi_u = W_e^T delta_u.  F is linear in each argument, so F(W+V) - F(W) = <V, dW> exactly.
    h, d = hd
    rng = np.random.default_rng(11)
    P = _tiny_problem(rng, T=64, h=h, d=d, dtype="f32")
    q, off, sel, Gc, Phic = _path(P, {"full": 0, "rho_num": 2, "rho_den": 3, "cap_abs": -1})
    W = P["W"].astype(np.float64)
    D, Ph = Gc.astype(np.float64), Phic.astype(np.float64)
    e_of = np.searchsorted(off, np.arange(D.shape[0]), side="right") - 1

    def F(Wm, Phm):
        return sum(float(D[i] @ (Wm[e_of[i]] @ Phm[i])) for i in range(D.shape[0]))

    V = rng.standard_normal(W.shape)
    dW = O.grouped_dw(Gc, Phic, off, "f32")
    lhs = F(W + V, Ph) - F(W, Ph)
    assert abs(lhs - float((V * dW).sum())) <= 1e-9 * (abs(lhs) + 1)
    Psi = rng.standard_normal(Ph.shape)
    dX = O.grouped_dx(Gc, P["W"], off, "f32")
    lhs = F(W, Ph + Psi) - F(W, Ph)
    assert abs(lhs - float((Psi * dX).sum())) <= 1e-9 * (abs(lhs) + 1)
    # cross identity <W_e, dW_e> = sum_u <phi_u, dphi_u> per expert
    for e in range(P["E_loc"]):
        s, t = off[e], off[e + 1]
        a = float((W[e] * dW[e]).sum())
        b = float((Ph[s:t] * dX[s:t]).sum())
        assert abs(a - b) <= 1e-10 * (abs(a) + 1)


def test_dropped_mass_bound():
    # Appendix 7.3, Eq. (20): ||Delta_D||^2 <= (sum_D sqrt(R_u))^2 <= |D| sum_D R_u, where R_u is
    # the squared norm of the dropped rank-one contribution.
    rng = np.random.default_rng(12)
    P = _tiny_problem(rng, T=90, h=9, d=7, dtype="f32")
    qf, offf, self_, Gf, Pf = _path(P, {"full": 1})
    q, off, sel, Gc, Phic = _path(P, {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1})
    dWf = O.grouped_dw(Gf, Pf, offf, "f32")
    dW = O.grouped_dw(Gc, Phic, off, "f32")
    D, Ph = Gf.astype(np.float64), Pf.astype(np.float64)
    fo = P["fwd_off"]
    for e in range(P["E_loc"]):
        rows = np.arange(fo[e], fo[e + 1])
        dropped = np.setdiff1d(rows, sel)
        Ru = (D[dropped] ** 2).sum(1) * (Ph[dropped] ** 2).sum(1)
        lhs = float(((dWf[e] - dW[e]) ** 2).sum())
        assert lhs <= float(np.sqrt(Ru).sum()) ** 2 * (1 + 1e-12) + 1e-300
        assert float(np.sqrt(Ru).sum()) ** 2 <= dropped.size * float(Ru.sum()) * (1 + 1e-12) + 1e-300


def test_sampled_helpers_agree_with_full_products():
    rng = np.random.default_rng(13)
    P = _tiny_problem(rng, T=70, h=16, d=24, dtype="bf16")
    q, off, sel, Gc, Phic = _path(P, {"full": 0, "rho_num": 3, "rho_den": 4, "cap_abs": -1})
    dW = O.grouped_dw(Gc, Phic, off, "bf16")
    dX = O.grouped_dx(Gc, P["W"], off, "bf16")
    for e in range(P["E_loc"]):
        np.testing.assert_array_equal(O.dw_rows(Gc, Phic, off, e, [0, 5, 15], "bf16"), dW[e][[0, 5, 15]])
    rows = np.arange(0, Gc.shape[0], 3)
    np.testing.assert_allclose(O.dx_rows(Gc, P["W"], off, rows, "bf16"), dX[rows], rtol=1e-14)


def test_run_end_to_end_small():
    rng = np.random.default_rng(14)
    P = _tiny_problem(rng, T=100, dtype="bf16")
    out = O.run(P["idx"], P["w"], P["g"], P["phi"], P["W"], T=P["T"], k=P["k"], E=P["E"],
                e_lo=P["e_lo"], E_loc=P["E_loc"], dtype="bf16",
                policy={"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1})
    assert out["counts"].sum() == P["T"] * P["k"]
    assert np.array_equal(out["sel_pair"], out["row_pair"][out["sel_row"]])
    assert out["Gc"].shape[0] == out["cmp_off"][-1] == out["dphi"].shape[0]
    retained = out["cmp_off"][1:] - out["cmp_off"][:-1]
    n_loc = out["fwd_off"][1:] - out["fwd_off"][:-1]
    assert np.array_equal(retained, np.minimum(out["quota"], n_loc))


# ------------------------------------------------------------------------------------------------
# forward-time admission (candidate descent against one GPU's budgets)
# ------------------------------------------------------------------------------------------------

def _budget(mem_budget, mem_base=0, mem_per_row=1, comm_budget=-1, comm_per_row=0):
    return dict(mem_budget=mem_budget, mem_base=mem_base, mem_per_row=mem_per_row,
                comm_budget=comm_budget, comm_per_row=comm_per_row)


def test_admission_worked_example():
    # The page-2 worked example: full retention carries all 131072 routed rows, the capacity rule
    # with CF = 5/4 carries 118032.  A budget between the two admits the capacity candidate.
    gx = _gold("expert_parallel_math_worked_example.json")
    n = np.asarray(gx["n"])
    full = {"full": 1, "rho_num": 1, "rho_den": 1, "cap_abs": -1}
    cf = {"full": 0, "rho_num": gx["capacity_factor_num"], "rho_den": gx["capacity_factor_den"],
          "cap_abs": -1}
    row = 2 * 4096                                   # bytes per retained row
    for mem, want in ((int(n.sum()) * row, 0), (gx["real_carried"] * row, 1),
                      (gx["real_carried"] * row - 1, -1)):
        c, q, off = O.admit_quotas(n, [full, cf], _budget(mem, mem_per_row=row))
        assert c == want
        if c == 1:
            assert int(off[-1]) == gx["real_carried"] and int(q.max()) == gx["C"]
        if c == -1:
            assert not q.any() and not off.any()


def test_admission_is_first_feasible_and_largest_rate():
    rng = np.random.default_rng(3)
    for trial in range(200):
        E_loc = int(rng.integers(1, 9))
        n = rng.integers(0, 60, E_loc)
        kind = ["cap", "proportional", "waterfill"][trial % 3]
        cap = -1 if kind == "proportional" else int(rng.integers(-1, 40))
        rates = [(1, 1), (7, 8), (3, 4), (1, 2), (1, 4), (1, 8), (0, 1)]
        cands = [{"full": 1, "rho_num": 1, "rho_den": 1, "cap_abs": cap, "kind": kind}] + \
                [{"full": 0, "rho_num": a, "rho_den": b, "cap_abs": cap, "kind": kind}
                 for a, b in rates]
        Ks = [int(O.plan_quotas(n, p)[1][-1]) for p in cands]
        # the retained total never grows as the rate decreases (so the first feasible candidate
        # in decreasing order is the largest feasible rate)
        assert all(Ks[i] >= Ks[i + 1] for i in range(len(Ks) - 1)), (kind, n, cap, Ks)
        b = _budget(int(rng.integers(0, 400)), mem_base=int(rng.integers(0, 50)),
                    mem_per_row=int(rng.integers(1, 4)), comm_budget=int(rng.integers(-1, 200)),
                    comm_per_row=int(rng.integers(0, 3)))
        K_cap = int(rng.integers(1, 400))
        c, q, off = O.admit_quotas(n, cands, b, K_cap)
        ok = [K <= K_cap and b["mem_base"] + K * b["mem_per_row"] <= b["mem_budget"] and
              (b["comm_budget"] < 0 or K * b["comm_per_row"] <= b["comm_budget"]) for K in Ks]
        want = ok.index(True) if any(ok) else -1
        assert c == want
        if c >= 0:
            assert int(off[-1]) == Ks[c] and np.all(q <= n)
