/*
 * lrm.h -- C ABI of the LRMoE backward hot path on one MI355X (gfx950).
 *
 * The library implements, for one GPU's share of an expert-parallel MoE layer, the backward-time
 * steps of "LRMoE: Demand-Side Load Re-Calibration for Efficient MoE Training on
 * Memory-Constrained Nodes" (Hu et al., arXiv 2610.37720):
 *   lrm_plan_quotas  routed counts n_e, forward layout, quotas q_e, compacted offsets
 *   lrm_admit_quotas forward-time admission: the largest candidate retention rate whose retained
 *                    total fits this GPU's budgets fixes the quotas (Algorithm 1's admission loop)
 *                    (Algorithm 1's count of each expert's pairs; Sec. 3.1 and 3.3 quotas 0 <= K_e <= N_e; the capacity
 *                    form of "Expert Parallel Math Deep", "Capacity and the exact drop-rate
 *                    formula")
 *   lrm_score        Load Recalibration Metric R_u = alpha_u^2 ||g_t||^2 ||phi_u||^2
 *                    (Sec. 3.2, Prop. 3.1, Eq. (3); Algorithm 1's score)
 *   lrm_score_norms / lrm_score_combine  the same in two halves: the norms need neither the
 *                    routing nor the layout, so they can run beside lrm_plan_quotas
 *   lrm_score_criterion  the same or one of the ablation criteria of Table 2
 *   lrm_select       per-expert TopK(q_e) (Algorithm 1's per-expert TopK; Sec. 3.3; Appendix 7.2 Prop. 7.1)
 *   lrm_compact      physical compaction into contiguous expert-major segments
 *                    (Sec. 3.3, Sec. 3.4, Fig. 4; Appendix 7.1 Eq. (5))
 *   lrm_grouped_dw   variable-size grouped FC2 weight gradient dW_e = sum_u delta_u phi_u^T
 *                    (Sec. 3.2 Eq. (1); Appendix 7.1 Eq. (8)-(9); Algorithm 1's grouped weight-gradient GEMM)
 *   lrm_grouped_dx   variable-size grouped FC2 input gradient dphi_u = W_e^T delta_u
 *                    (Appendix 7.1 Eq. (4)-(7); Sec. 3.3: the retained count is the row dimension
 *                    of the input-gradient product)
 *   lrm_grouped_dw_dx  both of the above in one launch
 *
 * and the rest of the expert backward over the same retained rows (Sec. 3.1: FC2, the activation
 * function, FC1 and the backward dispatch use the same retained identities; Sec. 3.4: repacking
 * shrinks all four expert-backward GEMMs; Algorithm 1's ScatterWithZeros):
 *   lrm_swiglu_backward   cotangent of the saved FC1 output [a | c] through phi = SiLU(a) * c
 *   lrm_gather_tokens     FC1's input row x_t of every retained pair
 *   lrm_grouped_fc1_dw    grouped FC1 weight gradient dW1_e = sum_u dH_u x_u^T
 *   lrm_grouped_fc1_dx    grouped FC1 input gradient dX_u = W1_e^T dH_u
 *   lrm_grouped_fc1_dw_dx both in one launch
 *   lrm_scatter_tokens    input-gradient rows returned to their tokens, zeros elsewhere
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pairs.  Token t routes to k experts; pair p = t*k + j, slot j in descending-logit order.
 *    topk_idx[p] is the expert of pair p, topk_w[p] its routing weight alpha (float32).
 *  - Local experts are [e_lo, e_lo + E_loc).  L = number of local pairs, K = sum of quotas.
 *  - Forward layout: the L local pairs ordered by (expert, pair index); "row" r indexes it.
 *    row_pair[r] = p, rows of expert e_lo+i are [fwd_off[i], fwd_off[i+1]).  phi is given in this
 *    layout: phi[r] is the saved SwiGLU activation of pair row_pair[r].
 *  - Compacted layout: retained rows of local expert i are [cmp_off[i], cmp_off[i+1]), in
 *    ascending forward-row (= pair) order.
 *  - Element type (problem.dtype): LRM_F32 or LRM_BF16 for g, phi, W, Gc, Phic.  Scores, dW and
 *    dphi are float32; indices and offsets int32.
 *  - Layouts are row-major and dense.  Row widths: g, Gc have h elements; phi, Phic, dphi have
 *    d elements; W is [E_loc][h][d] (W_e maps d_in = d to d_out = h); dW is [E_loc][h][d].
 *  - Every pointer except problem/policy (host structs, read during the call only) is device
 *    memory owned by the caller.  The library never allocates, frees or retains anything.
 *    Inputs are never written.  Outputs are fully (re)written up to their device-side lengths;
 *    entries past L or K are left untouched.
 *  - Every call enqueues work on `stream` and returns without waiting: no host synchronisation,
 *    no allocation, so a sequence of calls can be captured in a HIP graph.  Results are bitwise
 *    deterministic for identical inputs.
 *  - Rest of the expert backward: ac is the saved FC1 output per forward row, [L_cap][2d], gate
 *    pre-activation a in columns [0, d) and up projection c in [d, 2d) (phi = SiLU(a) * c); x is
 *    the layer input [T][h]; W1 is [E_loc][2d][h] (W1_e maps x (h) to [a; c] (2d)); dH, Xc are
 *    compacted [K_cap][2d] and [K_cap][h] in the element type; dW1 [E_loc][2d][h], dX [K_cap][h]
 *    and dx [T][h] are float32.
 *  - ws is caller-provided device scratch of at least lrm_workspace_bytes(problem) bytes,
 *    16-byte aligned.  Its first word is a sticky device error word (LRM_DEVERR_* bits) that
 *    lrm_plan_quotas clears and every call may set; read it with lrm_read_device_error.
 *  - Host-side validation returns LRM_ERR_INVALID_ARGUMENT (null pointer, non-positive sizes,
 *    k > E, e_lo + E_loc > E, rho_den <= 0, an unknown quota kind or criterion, caps too small
 *    for the problem) or
 *    LRM_ERR_UNSUPPORTED (pointer not 16-byte aligned, h or d not a multiple of 8 or above
 *    2^23, unknown dtype, E > 4096 or E_loc > 1024).  Launch failures return LRM_ERR_HIP.  Nothing is enqueued when a
 *    call returns an error.
 *  - Device-detected violations set error bits instead of faulting; results are then unspecified
 *    but every access stays inside the buffers described here.
 */
#ifndef LRM_H_
#define LRM_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LRM_OK = 0,
  LRM_ERR_INVALID_ARGUMENT = 1,
  LRM_ERR_UNSUPPORTED = 2,
  LRM_ERR_WORKSPACE_TOO_SMALL = 3,
  LRM_ERR_HIP = 4
} lrm_status;

typedef enum { LRM_F32 = 0, LRM_BF16 = 1 } lrm_dtype;

/* Device error word bits. */
#define LRM_DEVERR_EXPERT_ID 1  /* a topk_idx entry outside [0, E); the pair was ignored        */
#define LRM_DEVERR_L_CAP 2      /* L > L_cap; forward segments were truncated at L_cap           */
#define LRM_DEVERR_K_CAP 4      /* K > K_cap (or an offset past K_cap); segments truncated       */
#define LRM_DEVERR_QUOTA 8      /* quota[i] outside [0, n_i]; clamped into range                  */
#define LRM_DEVERR_NONFINITE 16 /* a score that is NaN, infinite or negative                      */
#define LRM_DEVERR_INDEX 32     /* sel_row / row_pair entry out of range; the row was skipped     */

typedef struct {
  int32_t T;      /* tokens                                                                   */
  int32_t k;      /* experts per token (top-k)                                                */
  int32_t E;      /* global experts                                                           */
  int32_t e_lo;   /* first local expert                                                       */
  int32_t E_loc;  /* number of local experts                                                  */
  int32_t h;      /* FC2 output width (hidden size): columns of g, Gc; rows of W_e, dW_e      */
  int32_t d;      /* FC2 input width (expert FFN size): columns of phi, Phic, dphi, W_e, dW_e */
  int32_t dtype;  /* lrm_dtype of g, phi, W, Gc, Phic                                          */
  int32_t L_cap;  /* rows of row_pair, phi, score; >= 1                                        */
  int32_t K_cap;  /* rows of sel_row, sel_pair, Gc, Phic, dphi; >= 1                           */
} lrm_problem;

/*
 * Quota policy.  The pages fix the constraints 0 <= q_i <= n_i and leave the split of the
 * retained total across experts open (LRMoE Sec. 3.2, Sec. 3.3); `kind` picks one of three
 * readings.  With n_i the routed count of local expert e_lo + i and L = sum of n_i:
 *   full != 0 :  q_i = n_i  for every kind                 (full retention, rho = 1)
 *   LRM_QUOTA_CAP (0, the default of a zeroed struct): the capacity form C = CF * mean load of
 *                "Expert Parallel Math Deep" ("Capacity and the exact drop-rate formula"):
 *                q_i = min(n_i, floor(rho_num * L / (rho_den * E_loc)), cap_abs if cap_abs >= 0)
 *   LRM_QUOTA_PROPORTIONAL (1): a retained total B = min(L, floor(rho_num * L / rho_den)) split
 *                in proportion to the loads, shares B * n_i / L rounded by largest remainder
 *                (equal remainders: lower i first); sum q_i = B.  This is the split of LRMoE
 *                Fig. 4, where loads [4,2,3] keep [3,1,2].  cap_abs must be negative.
 *   LRM_QUOTA_WATERFILL (2): the same B water-filled under m_i = min(n_i, cap_abs if >= 0):
 *                q_i = min(m_i, level) at the highest integer level whose total is <= B, then
 *                one more row to each of the lowest-indexed experts with m_i > level until the
 *                total is B; q_i = m_i when sum m_i <= B.
 * Everything is computed exactly in integers on the device.
 */
#define LRM_QUOTA_CAP 0
#define LRM_QUOTA_PROPORTIONAL 1
#define LRM_QUOTA_WATERFILL 2

typedef struct {
  int32_t full;
  int32_t rho_num;
  int32_t rho_den;
  int32_t cap_abs;
  int32_t kind;   /* LRM_QUOTA_* */
} lrm_quota_policy;

/*
 * Forward-time admission on one GPU (LRMoE Algorithm 1's admission loop; Sec. 3.3: candidate retained
 * counts are tested in decreasing order starting with full retention, against the memory budget
 * and the communication window; the first feasible one fixes the quotas; if none is feasible,
 * admission fails).  Candidate c is the quota policy {full[c], rho_num[c], rho_den[c], cap_abs,
 * kind} of lrm_quota_policy; its retained total K_c = sum of its quotas is feasible when
 *   K_c <= K_cap,   mem_base + K_c * mem_per_row <= mem_budget,
 *   and (comm_budget < 0 or K_c * comm_per_row <= comm_budget)
 * where mem_base counts the bytes needed whatever the retention (the complete forward workload
 * and its saved state: feasibility covers those, not only the reduced backward), mem_per_row the
 * bytes of one retained row's compacted buffers and gradients, comm_per_row the bytes one
 * retained row sends in the backward dispatch, and comm_budget = B_eff * T_ovlp the bytes that fit
 * the overlap window.  Replica placement, planned jointly on the pages, needs several GPUs and is
 * not part of this call.
 */
#define LRM_MAX_CANDIDATES 16

typedef struct {
  int32_t n_cand;                          /* 1 .. LRM_MAX_CANDIDATES, tested in this order      */
  int32_t kind;                            /* LRM_QUOTA_* of every candidate                      */
  int32_t cap_abs;                         /* absolute per-expert cap (< 0: none)                 */
  int32_t full[LRM_MAX_CANDIDATES];        /* candidate c keeps every routed row                  */
  int32_t rho_num[LRM_MAX_CANDIDATES];     /* else its retention fraction rho_num / rho_den       */
  int32_t rho_den[LRM_MAX_CANDIDATES];
  int64_t mem_budget;                      /* bytes                                               */
  int64_t mem_base;                        /* bytes, >= 0                                         */
  int64_t mem_per_row;                     /* bytes, 0 .. 2^32                                    */
  int64_t comm_budget;                     /* bytes; < 0: no communication limit                  */
  int64_t comm_per_row;                    /* bytes, 0 .. 2^32                                    */
} lrm_admission;

/* Bytes of device scratch every call needs for this problem, the FC1 calls included (0 if the
 * problem is invalid). */
size_t lrm_workspace_bytes(const lrm_problem* problem);

/*
 * Counts, forward layout, quotas and compacted offsets (LRMoE Algorithm 1's count of each expert's pairs; Sec. 3.3).
 *  in : topk_idx  int32 [T*k]
 *  out: counts    int32 [E]          routed pairs of every global expert (sum = T*k)
 *       fwd_off   int32 [E_loc + 1]  exclusive prefix of the local counts; fwd_off[E_loc] = L
 *       row_pair  int32 [L_cap]      pair index of each forward row (first L written)
 *       quota     int32 [E_loc]      q_i under `policy`
 *       cmp_off   int32 [E_loc + 1]  exclusive prefix of the quotas; cmp_off[E_loc] = K
 * Clears the device error word first.  Out-of-range expert ids are skipped and flagged.
 */
lrm_status lrm_plan_quotas(const lrm_problem* problem, const lrm_quota_policy* policy,
                           const int32_t* topk_idx, int32_t* counts, int32_t* fwd_off,
                           int32_t* row_pair, int32_t* quota, int32_t* cmp_off, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * Admission (see lrm_admission): from the local counts in fwd_off (as lrm_plan_quotas writes it),
 * writes the quotas and compacted offsets of the first feasible candidate and its index to
 * *admitted (device int32); if none is feasible, every quota is zero, cmp_off is all zeros and
 * *admitted = -1 -- the later calls then keep no row.  Overwrites what lrm_plan_quotas wrote to
 * quota and cmp_off; computed on the device in one launch, so the outcome needs no host
 * round trip.
 *  in : fwd_off int32 [E_loc+1]
 *  out: quota int32 [E_loc]; cmp_off int32 [E_loc+1]; admitted int32 [1]
 * Invalid candidates (rho_den <= 0 or rho_num < 0 without full, a cap with the proportional
 * kind, n_cand outside [1, LRM_MAX_CANDIDATES], negative or oversized byte figures) return
 * LRM_ERR_INVALID_ARGUMENT.
 */
lrm_status lrm_admit_quotas(const lrm_problem* problem, const lrm_admission* admission,
                            const int32_t* fwd_off, int32_t* quota, int32_t* cmp_off,
                            int32_t* admitted, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * LRM score of every local forward row (LRMoE Sec. 3.2, Prop. 3.1, Eq. (3)):
 *   score[r] = fl32(alpha_p^2 * ||g_t||^2 * ||phi_r||^2),  p = row_pair[r], t = p / k,
 * with both squared norms accumulated in float64 (every square of a bf16 or fp32 value is exact
 * in float64) by a fixed-order reduction that does not depend on the row's position, then one
 * rounding to float32.
 *  in : topk_w float32 [T*k]; g [T][h]; phi [L_cap][d]; row_pair int32 [L_cap];
 *       fwd_off int32 [E_loc+1] (only fwd_off[E_loc] = L is read)
 *  out: score float32 [L_cap] (first L written)
 * Non-finite or negative results set LRM_DEVERR_NONFINITE.
 */
lrm_status lrm_score(const lrm_problem* problem, const float* topk_w, const void* g,
                     const void* phi, const int32_t* row_pair, const int32_t* fwd_off,
                     float* score, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * lrm_score in two halves (LRMoE Sec. 3.2, Eq. (3): R_u factors into alpha_u^2, a norm of the
 * token's upstream gradient and a norm of the pair's saved activation; neither norm depends on
 * the routing counts, the quotas or the layout).
 *
 * lrm_score_norms writes ||g_t||^2 of every token t < T and ||phi_r||^2 of every row r < L_cap
 * (float64, the same fixed-order sums as lrm_score) into the workspace's norm region.  It reads
 * only g and all L_cap rows of phi (so phi must hold L_cap rows) -- rows at or past L may hold
 * anything; their norms are never used -- and
 * writes nothing but that region, which no other call writes, so it may run on another stream
 * at the same time as lrm_plan_quotas (or lrm_admit_quotas) on the same workspace; the caller
 * orders it (an event) before lrm_score_combine.  It sets no device error bits.
 *  in : g [T][h]; phi [L_cap][d]
 *
 * lrm_score_combine then writes score[r] = fl32(alpha_p^2 * ||g_t||^2 * ||phi_r||^2) for every
 * r < L (p = row_pair[r], t = p / k), from the norms the last lrm_score_norms on this workspace
 * left.  Scores are bitwise equal to lrm_score's on the same inputs.
 *  in : topk_w float32 [T*k]; row_pair int32 [L_cap]; fwd_off int32 [E_loc+1] (only fwd_off[E_loc])
 *  out: score float32 [L_cap] (first L written)
 * Row pairs outside [0, T*k) set LRM_DEVERR_INDEX (score 0); non-finite or negative results set
 * LRM_DEVERR_NONFINITE.
 */
lrm_status lrm_score_norms(const lrm_problem* problem, const void* g, const void* phi, void* ws,
                           size_t ws_bytes, hipStream_t stream);
lrm_status lrm_score_combine(const lrm_problem* problem, const float* topk_w,
                             const int32_t* row_pair, const int32_t* fwd_off, float* score,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Selection criteria (LRMoE Table 2 and Sec. 4.7 ablation).  The LRM criterion is lrm_score; the
 * others are the gradient-only rules and random drop the ablation compares it with:
 *   LRM_CRIT_LRM      (0)  score[r] = fl32(alpha_p^2 ||g_t||^2 ||phi_r||^2)   (as lrm_score)
 *   LRM_CRIT_GRAD_SQ  (1)  score[r] = fl32(||g_t||_2^2)        ("L-2 norm for grad")
 *   LRM_CRIT_GRAD_ABS (2)  score[r] = fl32(sum_i |g_t,i|)      ("absolute value for grad")
 *   LRM_CRIT_RANDOM   (3)  score[r] = keys[p]                  ("random drop")
 * with p = row_pair[r], t = p / k.  The gradient-only rules use the upstream gradient g_t alone,
 * without the routing weight (a gradient-only rule cannot tell apart pairs whose routing weights
 * or saved activations differ, Sec. 4.7).  Sums are accumulated in float64 in a fixed order and
 * rounded once.  Random drop ranks by caller-drawn keys, one float32 per pair; independent
 * uniform keys make each expert's kept set a uniformly random quota-sized subset, and the tie
 * rule of lrm_select decides equal keys.
 */
#define LRM_CRIT_LRM 0
#define LRM_CRIT_GRAD_SQ 1
#define LRM_CRIT_GRAD_ABS 2
#define LRM_CRIT_RANDOM 3

/*
 * Score of every local forward row under `criterion` (LRM_CRIT_*).
 *  in : topk_w float32 [T*k] (LRM only); g [T][h] (all but RANDOM); phi [L_cap][d] (LRM only);
 *       keys float32 [T*k] (RANDOM only); row_pair int32 [L_cap]; fwd_off int32 [E_loc+1]
 *       (only fwd_off[E_loc] = L is read).  Inputs a criterion does not read may be NULL.
 *  out: score float32 [L_cap] (first L written)
 * An unknown criterion or a NULL input the criterion reads returns LRM_ERR_INVALID_ARGUMENT.
 * Non-finite or negative results (a NaN or negative key included) set LRM_DEVERR_NONFINITE.
 */
lrm_status lrm_score_criterion(const lrm_problem* problem, int32_t criterion, const float* topk_w,
                               const void* g, const void* phi, const float* keys,
                               const int32_t* row_pair, const int32_t* fwd_off, float* score,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Per-expert top-q selection (LRMoE Algorithm 1's per-expert TopK; Appendix 7.2 Prop. 7.1).  In each
 * forward segment i keep the quota[i] rows that come first in the order (score descending, pair
 * index ascending; within a segment pair order equals row order) and write their forward-row ids,
 * ascending, to sel_row[cmp_off[i] ...].  Scores are compared as float32 (equal bit patterns tie).
 *  in : score float32 [L_cap]; fwd_off, quota, cmp_off as written by lrm_plan_quotas (any values
 *       with cmp_off[i+1] - cmp_off[i] == quota[i] are accepted)
 *  out: sel_row int32 [K_cap] (first K written)
 * A quota outside [0, n_i] is clamped (LRM_DEVERR_QUOTA); a NaN/negative score sets
 * LRM_DEVERR_NONFINITE.
 */
lrm_status lrm_select(const lrm_problem* problem, const float* score, const int32_t* fwd_off,
                      const int32_t* quota, const int32_t* cmp_off, int32_t* sel_row, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/*
 * Physical compaction (LRMoE Sec. 3.3/3.4, Fig. 4; Appendix 7.1 Eq. (5)).  For i < K:
 *   r = sel_row[i], p = row_pair[r], t = p / k
 *   Gc[i]       = RNE_dtype(fl32(topk_w[p] * g[t]))   (one float32 product per element, then
 *                                                      round-to-nearest-even to the element type)
 *   Phic[i]     = phi[r]                              (bit copy)
 *   sel_pair[i] = p
 *  in : sel_row int32 [K_cap], strictly ascending over [0, K) (as lrm_select writes it);
 *       row_pair int32 [L_cap], distinct pair ids on the selected rows (as lrm_plan_quotas
 *       writes it); cmp_off int32 [E_loc+1] (only cmp_off[E_loc] = K is read); topk_w; g; phi
 *  out: Gc [K_cap][h]; Phic [K_cap][d]; sel_pair int32 [K_cap]
 * Each g[t] row is read once per call however many of its pairs are kept; the workspace holds a
 * pair -> compacted-row map (T*k int32) that needs no clearing between calls.  A selected row out
 * of [0, L_cap) or out of order, a pair id out of [0, T*k), or two selected rows with one pair id
 * set LRM_DEVERR_INDEX; the rows concerned get sel_pair = -1 or undefined data.
 */
lrm_status lrm_compact(const lrm_problem* problem, const int32_t* sel_row, const int32_t* row_pair,
                       const int32_t* cmp_off, const float* topk_w, const void* g,
                       const void* phi, void* Gc, void* Phic, int32_t* sel_pair, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Grouped FC2 weight gradient over the retained rows only (LRMoE Sec. 3.2 Eq. (1); Appendix 7.1
 * Eq. (8)-(9); Sec. 3.4: no padding rows):  for every local expert i,
 *   dW[i] = sum_{c in [cmp_off[i], cmp_off[i+1])} Gc[c]^T (outer) Phic[c]      ([h][d], float32)
 * bf16 inputs use bf16 matrix-core products with float32 accumulation; fp32 inputs use fp32
 * matrix-core products.  An expert with no retained row gets exact zeros.  Summation order is
 * fixed, so results are bitwise reproducible.
 */
lrm_status lrm_grouped_dw(const lrm_problem* problem, const void* Gc, const void* Phic,
                          const int32_t* cmp_off, float* dW, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Grouped FC2 input gradient over the retained rows only (LRMoE Appendix 7.1 Eq. (4)-(7)):
 *   dphi[c] = W_e^T Gc[c]   for c in [cmp_off[i], cmp_off[i+1]),   i.e. dphi[c][j] =
 *   sum_o Gc[c][o] * W[i][o][j]  ([K_cap][d] float32; first K rows written).
 * The row tiles are scheduled on the device from cmp_off; no host synchronisation.
 */
lrm_status lrm_grouped_dx(const lrm_problem* problem, const void* Gc, const void* W,
                          const int32_t* cmp_off, float* dphi, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Both grouped FC2 gradients in one call: dW exactly as lrm_grouped_dw and dphi exactly as
 * lrm_grouped_dx (same arguments, same results bit for bit), computed by one persistent kernel
 * for bf16 inputs: workgroups whose share of the weight-gradient tiles ends early take
 * input-gradient tiles, so neither product leaves the device partly idle while the other still
 * has work (LRMoE Sec. 3.4: all expert-backward GEMMs run over the retained rows only).  When the
 * weight-gradient stores dominate (few retained rows per expert), or when the input-gradient
 * tiles fit in one round of the device and starting them first is estimated to end sooner (a few
 * experts holding most retained rows), the input-gradient tiles start first and both kinds are
 * taken from shared counters.  fp32 inputs run the two products one after the other.  Requires
 * Gc, Phic, W, dW, dphi 16-byte aligned.
 */
lrm_status lrm_grouped_dw_dx(const lrm_problem* problem, const void* Gc, const void* Phic,
                             const void* W, const int32_t* cmp_off, float* dW, float* dphi,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * lrm_grouped_dw_dx without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Computes dW and
 * dphi as lrm_grouped_dw_dx does, from the same inputs, but never splits an expert's rows across
 * workgroup groups, so where lrm_grouped_dw_dx would split (strongly skewed expert sizes) dW may
 * differ from it in rounding; elsewhere the results are equal bit for bit.
 *  - The GEMM schedule lives in a static device array of 1 MiB that each GPU holds until the
 *    process ends.  Problems whose schedule does not fit return LRM_ERR_WORKSPACE_TOO_SMALL
 *    without enqueuing anything: at E_loc = 16 that is K_cap above 33,001,216 rows (bf16) or
 *    8,250,304 rows (fp32); more local experts lower the bound (about 1.6e7 bf16 rows at
 *    E_loc = 1024).
 *  - The call itself allocates nothing; its first call on a device looks up the array's device
 *    address (make that first call outside graph capture).
 *  - All calls on one GPU share the array: calls that overlap on one GPU (different streams
 *    without ordering) race and give undefined results.  Calls ordered on one stream are safe.
 * Arguments, layouts and alignment requirements as lrm_grouped_dw_dx.
 */
lrm_status lrm_grouped_dw_dx_noalloc(const lrm_problem* problem, const void* Gc, const void* Phic,
                                     const void* W, const int32_t* cmp_off, float* dW,
                                     float* dphi, hipStream_t stream);

/*
 * Backward of the SwiGLU activation over the retained rows (LRMoE Sec. 3.1: the activation
 * function uses the same retained identities as FC2).  For i < K, with r = sel_row[i], a =
 * ac[r][0:d], c = ac[r][d:2d] and g = dphi[i] (float32, as lrm_grouped_dx writes it):
 *   s = 1 / (1 + exp(-a)),  SiLU(a) = a s,  SiLU'(a) = s (1 + a (1 - s))
 *   dH[i][0:d]  = RNE_dtype((g c) SiLU'(a))        (cotangent of the gate a)
 *   dH[i][d:2d] = RNE_dtype(g SiLU(a))             (cotangent of the up projection c)
 * evaluated elementwise in float64 in exactly this operation order (no fused multiply-add) and
 * rounded once, to nearest even, to the element type.
 *  in : sel_row int32 [K_cap] (as lrm_select writes it); cmp_off (only cmp_off[E_loc] = K read);
 *       dphi float32 [K_cap][d]; ac [L_cap][2d]
 *  out: dH [K_cap][2d] (first K rows written)
 * A selected row outside [0, L_cap) sets LRM_DEVERR_INDEX and gets zeros.  dphi, ac and dH must
 * be 16-byte aligned.
 */
lrm_status lrm_swiglu_backward(const lrm_problem* problem, const int32_t* sel_row,
                               const int32_t* cmp_off, const float* dphi, const void* ac,
                               void* dH, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * FC1's input rows of the retained pairs (LRMoE Sec. 3.1: retained rows and their matching saved
 * states are gathered in one pair order):  Xc[i] = x[sel_pair[i] / k] (bit copy) for i < K.
 *  in : sel_pair int32 [K_cap] (as lrm_compact writes it); cmp_off (cmp_off[E_loc] = K read);
 *       x [T][h]
 *  out: Xc [K_cap][h] (first K rows written)
 * Each x[t] is read once however many of its pairs are kept.  The workspace's pair -> row map is
 * rebuilt from sel_pair by this call.  A pair id outside [0, T*k), or two rows naming one pair,
 * sets LRM_DEVERR_INDEX; the rows concerned are left unwritten.
 */
lrm_status lrm_gather_tokens(const lrm_problem* problem, const int32_t* sel_pair,
                             const int32_t* cmp_off, const void* x, void* Xc, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * Grouped FC1 weight gradient over the retained rows only (LRMoE Sec. 3.4: the FC1
 * weight-gradient GEMM runs over the retained rows):  for every local expert i,
 *   dW1[i] = sum_{c in [cmp_off[i], cmp_off[i+1])} dH[c]^T (outer) Xc[c]     ([2d][h], float32)
 * Same kernels and guarantees as lrm_grouped_dw (zeros for an expert with no retained row,
 * bitwise reproducible) with the widths exchanged.  All pointers 16-byte aligned.
 */
lrm_status lrm_grouped_fc1_dw(const lrm_problem* problem, const void* dH, const void* Xc,
                              const int32_t* cmp_off, float* dW1, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Grouped FC1 input gradient over the retained rows only (LRMoE Sec. 3.4):
 *   dX[c][j] = sum_o dH[c][o] * W1[i][o][j]   for c in [cmp_off[i], cmp_off[i+1])
 * i.e. dX[c] = W1_i^T dH[c] ([K_cap][h] float32, first K rows written).  Same kernels as
 * lrm_grouped_dx with the widths exchanged.  All pointers 16-byte aligned.
 */
lrm_status lrm_grouped_fc1_dx(const lrm_problem* problem, const void* dH, const void* W1,
                              const int32_t* cmp_off, float* dX, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Both FC1 gradients in one call: results bit for bit those of the two calls above (one
 * persistent kernel for bf16, as lrm_grouped_dw_dx). */
lrm_status lrm_grouped_fc1_dw_dx(const lrm_problem* problem, const void* dH, const void* Xc,
                                 const void* W1, const int32_t* cmp_off, float* dW1, float* dX,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Input gradient of every token (LRMoE Sec. 3.1: a kept row's input gradient goes back to the
 * token and slot it came from, in an output that starts as all zeros; Algorithm 1,
 * scatter-with-zeros):
 *   dx[t] = fl32( sum over slots j = 0..k-1 in order, pair p = t*k + j retained at row i, of
 *                 dX[i] ),  the sum taken in float64 from zero; dx[t] = 0 if no pair of t is kept
 *  in : sel_pair int32 [K_cap]; cmp_off (cmp_off[E_loc] = K read); dX float32 [K_cap][h]
 *  out: dx float32 [T][h] (every row written)
 * The workspace's pair -> row map is rebuilt from sel_pair by this call.  A pair id outside
 * [0, T*k), or two rows naming one pair, sets LRM_DEVERR_INDEX.  dX and dx 16-byte aligned.
 */
lrm_status lrm_scatter_tokens(const lrm_problem* problem, const int32_t* sel_pair,
                              const int32_t* cmp_off, const float* dX, float* dx, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * Copies the device error word to *code (host).  Synchronises `stream` (tests and diagnostics
 * only, never inside a captured sequence).  If clear != 0 the word is reset to zero afterwards.
 */
lrm_status lrm_read_device_error(void* ws, int32_t* code, int32_t clear, hipStream_t stream);

/* Static description of a status code. */
const char* lrm_status_string(lrm_status status);

#ifdef __cplusplus
}
#endif

#endif /* LRM_H_ */
