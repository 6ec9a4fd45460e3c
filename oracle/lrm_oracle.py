"""CPU oracle of the LRMoE backward hot path, in float64.

TEST INFRASTRUCTURE ONLY.  This package is the independent reference that the GPU library is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the GPU product path never calls, links or executes anything here, and
this package imports nothing from the GPU library.

Sources (cited by page title and section/equation):
  [LRMoE]  "LRMoE: Demand-Side Load Re-Calibration for Efficient MoE Training on
           Memory-Constrained Nodes" (Hu et al., arXiv 2610.37720): Sec. 3.1 design overview,
           Sec. 3.2 Load Recalibration Metric (Prop. 3.1, Eq. (1)-(3)), Sec. 3.3 layerwise load
           calibration (Algorithm 1, Fig. 4), Sec. 3.4 repacking GEMM, Appendix 7.1 (Eq. (4)-(12)),
           Appendix 7.2 (Prop. 7.1, Eq. (13)-(16)).
  [EPMath] "Expert Parallel Math Deep": "Routing as an expectation over a batch" (counts, sum of
           n_i = T*k) and "Capacity and the exact drop-rate formula" (C = CF*T*k/E).

Every function computes the plain definition: fp64 arithmetic on the exact stored input values
(bf16 inputs are given as uint16 bit patterns and widened exactly).  Readings where the pages
leave a step open:
  * pair index p = t*k + j, slot j in descending-logit order; token t = p // k;
  * the forward layout of the saved activations phi is expert-major with p ascending inside each
    expert (Sec. 3.1/3.3 keep one fixed pair order);
  * quota policy q_e = n_e (full retention) or min(n_e, floor(num*L / (den*E_loc)), cap) in
    integer arithmetic, where L is the number of local routed pairs (the pages leave open how the
    retained total is split across experts, Sec. 3.2; this is the capacity form of [EPMath]);
    two further policies split a retained total B = min(L, floor(num*L/den)) across experts:
    proportional shares B*n_e/L rounded by largest remainder (lower expert first on equal
    remainders), the split that turns Fig. 4's loads [4,2,3] into [3,1,2] at B = 6, and a
    water-fill min(n_e, cap, level) whose leftover units go to the lowest-indexed experts above
    the level;
  * Table 2's alternative criteria: "L-2 norm for grad" is ||g_t||_2^2 and "absolute value for
    grad" is ||g_t||_1 = sum_i |g_t,i|, both of the upstream gradient without the routing weight
    (Sec. 4.7: a gradient-only rule sees neither the routing weight nor the saved activation);
    "random drop" ranks by keys drawn by the caller, one per pair;
  * selection is decided on float32 scores (the precision the GPU stores), ranking by score
    descending and then pair index ascending; kept rows are written in ascending forward-row
    order;
  * the compacted weighted cotangent is delta = RNE_dtype(fl32(alpha * g)): one IEEE float32
    product, then round-to-nearest-even to the storage type (Appendix 7.1, Eq. (5) allows exposing
    delta instead of g, applying alpha only once);
  * dW and dphi are produced in float64 here (fp32 on the GPU);
  * the rest of the expert backward (Sec. 3.1: FC2, the activation function, FC1 and the backward
    dispatch use the same retained identities; Sec. 3.4: all four expert-backward GEMMs shrink):
    phi = SiLU(a) * c with a, c the gate and up halves of the saved FC1 output; the activation's
    cotangent dH = (dphi * c * SiLU'(a), dphi * SiLU(a)) is computed in float64 and rounded once,
    to nearest even, to the storage type; FC1 maps the token input x (h) to the 2d-wide [a; c];
    input-gradient rows return to their tokens as a float64 sum over the token's retained slots
    in slot order, rounded once to float32, and tokens without a retained pair get zeros.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# ------------------------------------------------------------------------------------------------
# element types
# ------------------------------------------------------------------------------------------------


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements (dtype "f32" or "bf16" given as uint16 bits)."""
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    bf16 keeps the upper 16 bits of the float32 pattern.  Adding 0x7FFF plus the lowest kept bit
    and truncating rounds the dropped 16 bits to nearest with ties to the even kept value; a carry
    out of the mantissa correctly increments the exponent (up to infinity).  Finite inputs only
    (the largest finite pattern 0xFF7FFFFF plus 0x8000 still fits in 32 bits).
    """
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    one, half = np.uint32(1), np.uint32(0x7FFF)
    u = u + half + ((u >> np.uint32(16)) & one)
    return (u >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------------------------------------------------------
# a1: routed counts and forward layout
# ------------------------------------------------------------------------------------------------


def routed_counts(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """n_e = |P_e|, the number of routed pairs of every expert e in [0, E).

    [LRMoE] Algorithm 1, its count of each expert's pairs (N_{l,e} <- |P_{l,e}|); [EPMath] "Routing as an expectation over
    a batch": each token makes k dispatches, so the counts sum to T*k.
    """
    idx = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert id out of range")
    n = np.zeros(E, np.int64)
    np.add.at(n, idx, 1)
    return n


def forward_layout(topk_idx: np.ndarray, e_lo: int, E_loc: int):
    """Forward dispatch layout of the local pairs.

    Returns (row_pair, fwd_off): row_pair lists, expert by expert for e in [e_lo, e_lo+E_loc),
    the pair indices routed to e in ascending order ([LRMoE] Sec. 3.1 and 3.3: rows are kept in a
    consistent pair order, grouped by expert); fwd_off[i] is the first row of local expert i and
    fwd_off[E_loc] = L.
    """
    idx = np.asarray(topk_idx).reshape(-1)
    segs, off = [], [0]
    for e in range(e_lo, e_lo + E_loc):
        ps = np.flatnonzero(idx == e).astype(np.int64)        # ascending pair index
        segs.append(ps)
        off.append(off[-1] + ps.size)
    row_pair = np.concatenate(segs) if segs else np.zeros(0, np.int64)
    return row_pair, np.asarray(off, np.int64)


# ------------------------------------------------------------------------------------------------
# a2: quotas and compacted offsets
# ------------------------------------------------------------------------------------------------


QUOTA_KINDS = ("cap", "proportional", "waterfill")


def retained_total(L: int, num: int, den: int) -> int:
    """B = min(L, floor(num*L/den)): the retained count K = rho*N of [LRMoE] Sec. 3.1 for a
    retention fraction rho = num/den, in integers."""
    if den <= 0 or num < 0:
        raise ValueError("bad retention fraction")
    return min(L, (num * L) // den)


def proportional_quotas(n, B: int):
    """Split B retained rows across experts in proportion to their loads (largest remainder).

    [LRMoE] Sec. 3.3 asks for quotas with 0 <= K_e <= N_e summing to the retained count and
    leaves the split open; Fig. 4 reduces loads [4,2,3] to [3,1,2], which is the proportional
    split of B = 6: exact shares B*n_e/L are rounded down and the B - sum of floors leftover rows
    go to the experts with the largest fractional parts, the lower expert index first on equal
    fractions.
    """
    L = sum(n)
    if L == 0:
        return [0] * len(n)
    share = [Fraction(B * v, L) for v in n]
    q = [int(x) for x in share]                          # floor (shares are non-negative)
    left = B - sum(q)
    order = sorted(range(len(n)), key=lambda e: (-(share[e] - q[e]), e))
    for e in order[:left]:
        q[e] += 1
    return q


def waterfill_quotas(n, B: int, cap: int):
    """Water-fill B retained rows: q_e = min(n_e, cap, level) at the highest integer level whose
    total stays within B, then one more row each to the lowest-indexed experts still above the
    level until the total is B (or q_e = min(n_e, cap) everywhere when that total is <= B).

    The reading of a retained total B with a per-expert cap ([LRMoE] Sec. 3.1/3.3 quotas
    0 <= K_e <= N_e; the cap of [EPMath] "Capacity and the exact drop-rate formula"): experts
    below the level keep every row, the others are levelled.
    """
    m = [v if cap < 0 else min(v, cap) for v in n]
    if sum(m) <= B:
        return m

    def total(level):
        return sum(min(v, level) for v in m)

    lo, hi = 0, max(m)                  # total(lo) <= B < total(hi); bisect for the last level
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if total(mid) <= B:
            lo = mid
        else:
            hi = mid
    q = [min(v, lo) for v in m]
    left = B - sum(q)
    for e in range(len(m)):
        if left == 0:
            break
        if m[e] > lo:
            q[e] += 1
            left -= 1
    return q


def plan_quotas(n_loc: np.ndarray, policy: dict):
    """Retention quotas q_e and compacted-segment offsets.

    [LRMoE] Sec. 3.1/3.3: quotas satisfy 0 <= K_e <= N_e and are fixed for the invocation;
    the admission search begins at full retention, K_e = N_e.  The cap form (policy kind "cap", the
    default) follows [EPMath] "Capacity and the exact drop-rate formula": an expert keeps
    min(n_e, C) rows with C = CF * (mean load), here C = floor(num*L / (den*E_loc)) computed
    exactly in integers, optionally also capped at an absolute cap.  Kinds "proportional" and
    "waterfill" split B = retained_total(L, num, den) (see proportional_quotas, waterfill_quotas;
    "proportional" takes no cap).  cmp_off is the exclusive prefix sum of q with the total
    appended, so segment e occupies rows [cmp_off[e], cmp_off[e+1]) ([LRMoE] Fig. 4: counts
    R=[3,1,2] give offsets [0,3,4,6]).
    """
    n = [int(v) for v in np.asarray(n_loc).reshape(-1)]
    E_loc = len(n)
    L = sum(n)
    kind = policy.get("kind", "cap")
    if kind not in QUOTA_KINDS:
        raise ValueError(f"unknown quota policy kind {kind!r}")
    cap = int(policy.get("cap_abs", -1))
    if policy.get("full", 0):
        q = list(n)
    elif kind == "cap":
        num, den = int(policy["rho_num"]), int(policy["rho_den"])
        if den <= 0 or num < 0:
            raise ValueError("bad retention fraction")
        c = (num * L) // (den * E_loc) if E_loc > 0 else 0
        q = [min(v, c) if cap < 0 else min(v, c, cap) for v in n]
    elif kind == "proportional":
        if cap >= 0:
            raise ValueError("the proportional policy takes no cap")
        q = proportional_quotas(n, retained_total(L, int(policy["rho_num"]), int(policy["rho_den"])))
    else:
        q = waterfill_quotas(n, retained_total(L, int(policy["rho_num"]), int(policy["rho_den"])),
                             cap)
    off = [0]
    for v in q:
        off.append(off[-1] + v)
    return np.asarray(q, np.int64), np.asarray(off, np.int64)


def admission_feasible(K: int, budget: dict, K_cap=None) -> bool:
    """Whether a retained total K fits one GPU's resources: its row capacity K_cap, the HBM budget
    (mem_base bytes needed whatever the retention -- the complete forward workload and its saved
    state -- plus mem_per_row bytes per retained row) and the bytes the backward dispatch may move
    inside the overlap window (comm_budget = B_eff * T_ovlp, comm_per_row bytes per retained row;
    comm_budget < 0: no limit)."""
    if K_cap is not None and K > K_cap:
        return False
    if budget["mem_base"] + K * budget["mem_per_row"] > budget["mem_budget"]:
        return False
    if budget["comm_budget"] >= 0 and K * budget["comm_per_row"] > budget["comm_budget"]:
        return False
    return True


def admit_quotas(n_loc: np.ndarray, candidates, budget: dict, K_cap=None):
    """Forward-time admission on one GPU: the candidate retention rates are tested in the given
    order (decreasing, starting with full retention), each candidate's quotas come from
    plan_quotas, and the first candidate whose retained total K = sum of its quotas is feasible
    fixes the quotas; if none is, admission fails ([LRMoE] Algorithm 1, its admission loop over candidate policies; Sec. 3.3:
    candidates are tested in decreasing order starting with full retention, the first feasible one
    fixes the quotas, and admission fails when none is feasible).

    Returns (index of the admitted candidate or -1, quotas, offsets); a failed admission keeps no
    row (all quotas zero).  The replica placement the pages plan jointly needs several GPUs and is
    not part of one GPU's admission.
    """
    n_loc = np.asarray(n_loc)
    for c, pol in enumerate(candidates):
        q, off = plan_quotas(n_loc, pol)
        if admission_feasible(int(off[-1]), budget, K_cap):
            return c, q, off
    E_loc = n_loc.size
    return -1, np.zeros(E_loc, np.int64), np.zeros(E_loc + 1, np.int64)


# ------------------------------------------------------------------------------------------------
# a3: Load Recalibration Metric
# ------------------------------------------------------------------------------------------------


def lrm_scores(topk_w, g, phi, row_pair, k: int, dtype: str, chunk: int = 65536) -> np.ndarray:
    """R_r = alpha_p^2 * ||g_t||_2^2 * ||phi_r||_2^2 for every local forward row r, in float64.

    [LRMoE] Sec. 3.2, Prop. 3.1, Eq. (3) (and Algorithm 1's score): the squared Frobenius norm of
    the pair's FC2 weight-gradient contribution G_u = (alpha_u g_t) phi_u^T, factorised with the
    rank-one identity of Appendix 7.1, Eq. (11)-(12).  p = row_pair[r], t = p // k.
    """
    row_pair = np.asarray(row_pair, np.int64)
    a = np.asarray(topk_w, np.float32).astype(np.float64)[row_pair]
    t = row_pair // k
    gsq = np.empty(g.shape[0], np.float64)
    for s in range(0, g.shape[0], chunk):
        gw = widen(g[s:s + chunk], dtype)
        gsq[s:s + chunk] = (gw * gw).sum(axis=1)
    psq = np.empty(row_pair.shape[0], np.float64)
    for s in range(0, row_pair.shape[0], chunk):
        pw = widen(phi[s:s + chunk], dtype)
        psq[s:s + chunk] = (pw * pw).sum(axis=1)
    return a * a * gsq[t] * psq


def _token_rows(g, dtype, chunk, f):
    """f(widened rows) for every token row of g, in float64, chunk by chunk."""
    out = np.empty(g.shape[0], np.float64)
    for s in range(0, g.shape[0], chunk):
        out[s:s + chunk] = f(widen(g[s:s + chunk], dtype))
    return out


def grad_sq_scores(g, row_pair, k: int, dtype: str, chunk: int = 65536) -> np.ndarray:
    """||g_t||_2^2 of the pair's token for every local forward row ([LRMoE] Table 2, "L-2 norm
    for grad"; the upstream gradient alone, Sec. 4.7)."""
    t = np.asarray(row_pair, np.int64) // k
    return _token_rows(g, dtype, chunk, lambda x: (x * x).sum(axis=1))[t]


def grad_abs_scores(g, row_pair, k: int, dtype: str, chunk: int = 65536) -> np.ndarray:
    """||g_t||_1 = sum_i |g_t,i| of the pair's token for every local forward row ([LRMoE]
    Table 2, "absolute value for grad")."""
    t = np.asarray(row_pair, np.int64) // k
    return _token_rows(g, dtype, chunk, lambda x: np.abs(x).sum(axis=1))[t]


def random_scores(keys, row_pair) -> np.ndarray:
    """keys[p] for every local forward row ([LRMoE] Table 2, "random drop"): with independent
    uniform keys per pair, the top-q of each expert is a uniformly random q-subset."""
    return np.asarray(keys, np.float32).astype(np.float64)[np.asarray(row_pair, np.int64)]


CRITERIA = ("lrm", "grad_sq", "grad_abs", "random")


def scores(criterion: str, topk_w, g, phi, row_pair, k: int, dtype: str, keys=None) -> np.ndarray:
    """Selection score of every local forward row under one of [LRMoE] Table 2's criteria."""
    if criterion == "lrm":
        return lrm_scores(topk_w, g, phi, row_pair, k, dtype)
    if criterion == "grad_sq":
        return grad_sq_scores(g, row_pair, k, dtype)
    if criterion == "grad_abs":
        return grad_abs_scores(g, row_pair, k, dtype)
    if criterion == "random":
        if keys is None:
            raise ValueError("the random criterion needs one key per pair")
        return random_scores(keys, row_pair)
    raise ValueError(f"unknown criterion {criterion!r}")


# ------------------------------------------------------------------------------------------------
# a4: per-expert top-q selection
# ------------------------------------------------------------------------------------------------


def select_top_quota(score32: np.ndarray, fwd_off, quota, row_pair) -> np.ndarray:
    """Forward rows kept by per-expert TopK(q_e), ascending within each expert, experts in order.

    [LRMoE] Algorithm 1's per-expert TopK and Sec. 3.3: within each logical expert keep the q_e
    highest-scoring pairs; Appendix 7.2, Prop. 7.1: keeping the largest scores is optimal, and ties
    at the boundary admit several optimal sets.  The set is made unique by ranking on
    (score descending, pair index ascending).  Scores are the float32 values the decision is taken
    on.
    """
    s = np.asarray(score32, np.float32).astype(np.float64)
    row_pair = np.asarray(row_pair, np.int64)
    out = []
    for e in range(len(quota)):
        r0, r1 = int(fwd_off[e]), int(fwd_off[e + 1])
        q = int(quota[e])
        if q < 0 or q > r1 - r0:
            raise ValueError("quota outside [0, n_e]")
        rows = np.arange(r0, r1, dtype=np.int64)
        order = np.lexsort((row_pair[rows], -s[rows]))      # primary: -score; then pair index
        out.append(np.sort(rows[order[:q]]))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


# ------------------------------------------------------------------------------------------------
# a5: physical compaction
# ------------------------------------------------------------------------------------------------


def compact(sel_row, row_pair, topk_w, g, phi, k: int, dtype: str, chunk: int = 8192):
    """Gather the retained rows into contiguous expert-major buffers.

    [LRMoE] Sec. 3.3/3.4 and Fig. 4 (mask -> pack -> counts/offsets): retained gradient rows and
    their matching saved activations are packed in pair order.  Row i of the output belongs to the
    forward row r = sel_row[i] with pair p = row_pair[r] and token t = p // k:
        Gc[i]   = RNE_dtype(fl32(alpha_p * g_t))     (delta_u of Appendix 7.1, Eq. (5))
        Phic[i] = phi[r]                             (exact copy)
        sel_pair[i] = p
    Returns (Gc, Phic, sel_pair) in the storage type (bf16 as uint16 bits).
    """
    sel_row = np.asarray(sel_row, np.int64)
    p = np.asarray(row_pair, np.int64)[sel_row]
    t = p // k
    a32 = np.asarray(topk_w, np.float32)[p][:, None]
    Gc = np.empty((sel_row.size, g.shape[1]), np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, sel_row.size, chunk):        # row blocks only bound the temporaries
        rows = slice(s, s + chunk)
        if dtype == "f32":
            Gc[rows] = a32[rows] * np.asarray(g, np.float32)[t[rows]]       # one fp32 product
        else:
            g32 = (np.asarray(g, np.uint16)[t[rows]].astype(np.uint32) << 16).view(np.float32)
            Gc[rows] = f32_to_bf16_rne(a32[rows] * g32)
    Phic = np.asarray(phi)[sel_row].copy()
    return Gc, Phic, p


# ------------------------------------------------------------------------------------------------
# a6 / a7: grouped FC2 gradients over the retained rows
# ------------------------------------------------------------------------------------------------


def grouped_dw(Gc, Phic, cmp_off, dtype: str) -> np.ndarray:
    """dW_e = sum over retained rows i of expert e of delta_i phi_i^T  (shape [E_loc, h, d]).

    [LRMoE] Sec. 3.2, Eq. (1) and Appendix 7.1, Eq. (8)-(9): the protected (FC2) weight gradient
    is the sum of the retained pairs' rank-one contributions; an expert with no retained row gets
    an all-zero gradient.
    """
    D = widen(Gc, dtype)
    P = widen(Phic, dtype)
    E_loc = len(cmp_off) - 1
    dW = np.zeros((E_loc, D.shape[1], P.shape[1]), np.float64)
    for e in range(E_loc):
        s, t = int(cmp_off[e]), int(cmp_off[e + 1])
        if t > s:
            dW[e] = D[s:t].T @ P[s:t]
    return dW


def grouped_dx(Gc, W, cmp_off, dtype: str) -> np.ndarray:
    """dphi_i = W_e^T delta_i for every retained row i of expert e (shape [K, d]).

    [LRMoE] Appendix 7.1, Eq. (4)-(7): W_e in R^{d_out x d_in} maps phi_u to the expert output
    y_u = alpha_u W_e phi_u, so the cotangent of phi_u is W_e^T (alpha_u g_t) = W_e^T delta_u;
    Sec. 3.3: the retained count is the row dimension of the input-gradient product.
    """
    D = widen(Gc, dtype)
    E_loc = len(cmp_off) - 1
    out = np.zeros((D.shape[0], W.shape[2]), np.float64)
    for e in range(E_loc):
        s, t = int(cmp_off[e]), int(cmp_off[e + 1])
        if t > s:
            out[s:t] = D[s:t] @ widen(W[e], dtype)       # row i: sum_j delta_ij W_e[j, :]
    return out


def dw_rows(Gc, Phic, cmp_off, e: int, rows_h, dtype: str) -> np.ndarray:
    """Rows ``rows_h`` (FC2 output indices) of dW_e, as grouped_dw computes them, in float64."""
    s, t = int(cmp_off[e]), int(cmp_off[e + 1])
    rows_h = np.asarray(rows_h, np.int64)
    if t == s:
        return np.zeros((rows_h.size, Phic.shape[1]), np.float64)
    return widen(Gc[s:t][:, rows_h], dtype).T @ widen(Phic[s:t], dtype)


def dx_rows(Gc, W, cmp_off, rows_i, dtype: str) -> np.ndarray:
    """Rows ``rows_i`` (compacted row indices) of dphi, as grouped_dx computes them, in float64."""
    rows_i = np.asarray(rows_i, np.int64)
    off = np.asarray(cmp_off, np.int64)
    e_of = np.searchsorted(off, rows_i, side="right") - 1
    out = np.zeros((rows_i.size, W.shape[2]), np.float64)
    for j, (i, e) in enumerate(zip(rows_i, e_of)):
        out[j] = widen(Gc[i], dtype) @ widen(W[e], dtype)
    return out


# ------------------------------------------------------------------------------------------------
# rest of the expert backward: activation, FC1 gradients, return to the tokens
# ------------------------------------------------------------------------------------------------


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 values directly to bfloat16 (nearest, ties to even); returns uint16 bits.

    bfloat16 keeps 8 significant bits with float32's exponent range.  With v = m * 2^e and
    1/2 <= |m| < 1, the spacing of bf16 values around v is 2^(e-8), and never finer than the
    smallest subnormal 2^-133; v is rounded at that spacing (scaling by powers of two is exact,
    np.rint rounds halves to even).  Values that round beyond the largest finite bf16 become
    infinities.  Finite inputs only.
    """
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)                   # exact, or +-inf past the finite range
    return (np.ascontiguousarray(f).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values rounded once, to nearest even, to the storage type."""
    if dtype == "f32":
        return np.asarray(v, np.float64).astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_rne(v)
    raise ValueError(dtype)


def swiglu_backward64(dphi, a, c):
    """Cotangents of the gate and up inputs of phi = SiLU(a) * c, in float64.

    SiLU(a) = a * s with s = 1 / (1 + exp(-a)) the logistic function, whose derivative is
    s * (1 - s); so d phi / d a = c * s * (1 + a * (1 - s)) and d phi / d c = SiLU(a), and the
    cotangents are dA = dphi * c * SiLU'(a), dC = dphi * SiLU(a) (elementwise).
    """
    dphi = np.asarray(dphi, np.float64)
    a = np.asarray(a, np.float64)
    c = np.asarray(c, np.float64)
    s = 1.0 / (1.0 + np.exp(-a))
    silu = a * s
    dsilu = s * (1.0 + a * (1.0 - s))
    return (dphi * c) * dsilu, dphi * silu


def swiglu_backward(dphi, ac, sel_row, dtype: str, chunk: int = 8192) -> np.ndarray:
    """The activation's backward over the retained rows: dH[i] = [dA_i | dC_i], rounded to the
    storage type ([LRMoE] Sec. 3.1: the activation function uses the same retained identities as
    FC2; its saved context is the FC1 output of the forward row r = sel_row[i]: gate a in columns
    [0, d), up c in [d, 2d)).  dphi[i] is the FC2 input gradient of retained row i (any float
    type, taken at its exact value).
    """
    sel_row = np.asarray(sel_row, np.int64)
    K = sel_row.size
    d = np.asarray(ac).shape[1] // 2
    out = np.empty((K, 2 * d), np.float32 if dtype == "f32" else np.uint16)
    for s0 in range(0, K, chunk):                  # row blocks only bound the temporaries
        rows = slice(s0, s0 + chunk)
        ctx = widen(np.asarray(ac)[sel_row[rows]], dtype)
        dA, dC = swiglu_backward64(np.asarray(dphi[rows], np.float64), ctx[:, :d], ctx[:, d:])
        out[rows, :d] = round_to(dA, dtype)
        out[rows, d:] = round_to(dC, dtype)
    return out


def gather_tokens(x, sel_pair, k: int) -> np.ndarray:
    """FC1's input rows of the retained pairs: Xc[i] = x[t] with t = sel_pair[i] // k (exact copy;
    [LRMoE] Sec. 3.1: retained rows and their matching saved states are gathered in one pair
    order)."""
    return np.asarray(x)[np.asarray(sel_pair, np.int64) // k].copy()


def fc1_grouped_dw(dH, Xc, cmp_off, dtype: str) -> np.ndarray:
    """dW1_e = sum over retained rows i of expert e of dH_i x_i^T, shape [E_loc, 2d, h]: the FC1
    weight gradient over the retained rows only ([LRMoE] Sec. 3.4: repacking shrinks the row
    dimension of the FC1 weight-gradient GEMM too).  Same definition as the FC2 weight gradient
    with (dH, Xc) in place of (delta, phi)."""
    return grouped_dw(dH, Xc, cmp_off, dtype)


def fc1_grouped_dx(dH, W1, cmp_off, dtype: str) -> np.ndarray:
    """dX_i = W1_e^T dH_i for every retained row i of expert e, shape [K, h]: the FC1 input
    gradient ([LRMoE] Sec. 3.4, FC1 data gradient), W1_e in R^{2d x h} mapping x to [a; c]."""
    return grouped_dx(dH, W1, cmp_off, dtype)


def scatter_with_zeros(dXc, sel_pair, T: int, k: int) -> np.ndarray:
    """Input gradient of every token: the retained rows' contributions returned to their token
    and summed, tokens without a retained pair left at zero ([LRMoE] Sec. 3.1: a kept row's
    input gradient goes back to the token and slot it came from, in an output that starts as all
    zeros, so dropped slots contribute nothing; Algorithm 1, scatter-with-zeros).

    Float64 sum per token over its slots j = 0..k-1 in order, starting from zero; shape [T, h].
    """
    dXc = np.asarray(dXc)
    sel_pair = np.asarray(sel_pair, np.int64)
    row_of = np.full(T * k, -1, np.int64)
    row_of[sel_pair] = np.arange(sel_pair.size)
    out = np.zeros((T, dXc.shape[1]), np.float64)
    tok = np.arange(T, dtype=np.int64)
    for j in range(k):
        i = row_of[tok * k + j]
        m = i >= 0
        out[m] += np.asarray(dXc[i[m]], np.float64)
    return out


def run_layer(o: dict, dphi, ac, x, W1, *, T: int, k: int, dtype: str) -> dict:
    """The rest of the expert backward from FC2's input gradient `dphi` (compacted order), on the
    retained rows of the path result `o` (sel_row, sel_pair, cmp_off)."""
    dH = swiglu_backward(dphi, ac, o["sel_row"], dtype)
    Xc = gather_tokens(x, o["sel_pair"], k)
    dW1 = fc1_grouped_dw(dH, Xc, o["cmp_off"], dtype)
    dXc = fc1_grouped_dx(dH, W1, o["cmp_off"], dtype)
    dx = scatter_with_zeros(dXc, o["sel_pair"], T, k)
    return dict(dH=dH, Xc=Xc, dW1=dW1, dXc=dXc, dx=dx)


# ------------------------------------------------------------------------------------------------
# whole path
# ------------------------------------------------------------------------------------------------


def run(topk_idx, topk_w, g, phi, W, *, T, k, E, e_lo, E_loc, dtype, policy,
        gemms: bool = True, criterion: str = "lrm", keys=None) -> dict:
    """Run every step of the path on the CPU and return all intermediate results."""
    n = routed_counts(topk_idx, E)
    row_pair, fwd_off = forward_layout(topk_idx, e_lo, E_loc)
    quota, cmp_off = plan_quotas(n[e_lo:e_lo + E_loc], policy)
    R = scores(criterion, topk_w, g, phi, row_pair, k, dtype, keys)
    score32 = R.astype(np.float32)
    sel_row = select_top_quota(score32, fwd_off, quota, row_pair)
    Gc, Phic, sel_pair = compact(sel_row, row_pair, topk_w, g, phi, k, dtype)
    out = dict(counts=n, row_pair=row_pair, fwd_off=fwd_off, quota=quota, cmp_off=cmp_off,
               score64=R, score32=score32, sel_row=sel_row, Gc=Gc, Phic=Phic, sel_pair=sel_pair)
    if gemms:
        out["dW"] = grouped_dw(Gc, Phic, cmp_off, dtype)
        out["dphi"] = grouped_dx(Gc, W, cmp_off, dtype)
    return out
