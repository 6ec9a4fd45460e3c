// Host side of the C ABI declared in include/lrm.h: argument validation, workspace layout and
// kernel launches.  No allocation, no synchronisation (except lrm_read_device_error).
#include <stddef.h>
#include <stdint.h>

#include "lrm_internal.hpp"

using lrm::WsLayout;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static_assert(sizeof(lrm_admission) == 248 && offsetof(lrm_admission, mem_budget) == 208,
              "lrm_admission layout is part of the ABI");

lrm_status check_problem(const lrm_problem* p) {
  if (!p) return LRM_ERR_INVALID_ARGUMENT;
  if (p->T <= 0 || p->k <= 0 || p->E <= 0 || p->E_loc <= 0 || p->h <= 0 || p->d <= 0)
    return LRM_ERR_INVALID_ARGUMENT;
  if (p->k > p->E || p->e_lo < 0 || (int64_t)p->e_lo + p->E_loc > p->E)
    return LRM_ERR_INVALID_ARGUMENT;
  if (p->L_cap <= 0 || p->K_cap <= 0) return LRM_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->T * p->k > INT32_MAX) return LRM_ERR_UNSUPPORTED;
  if (p->dtype != LRM_F32 && p->dtype != LRM_BF16) return LRM_ERR_UNSUPPORTED;
  if (p->h % 8 != 0 || p->d % 8 != 0) return LRM_ERR_UNSUPPORTED;
  if (p->h > (1 << 23) || p->d > (1 << 23)) return LRM_ERR_UNSUPPORTED;
  if (p->E > 4096 || p->E_loc > 1024) return LRM_ERR_UNSUPPORTED;
  return LRM_OK;
}

lrm_status check_ws(const lrm_problem* p, const void* ws, size_t ws_bytes, WsLayout* wl) {
  if (!ws) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(ws)) return LRM_ERR_UNSUPPORTED;
  *wl = lrm::ws_layout(*p);
  if (ws_bytes < wl->total) return LRM_ERR_WORKSPACE_TOO_SMALL;
  return LRM_OK;
}

lrm_status from_hip(hipError_t e) { return e == hipSuccess ? LRM_OK : LRM_ERR_HIP; }

// FC1's gradients are the grouped products of the FC2 calls with the widths exchanged: rows of
// width 2d (the activation's cotangent dH) against rows of width h (the token inputs x), and FC1
// weights [E_loc][2d][h].  The workspace layout of this problem differs from the original's only
// in the size of its last region (the split experts' partial slots).
lrm_problem fc1_problem(const lrm_problem& p) {
  lrm_problem q = p;
  q.h = 2 * p.d;
  q.d = p.h;
  return q;
}

}  // namespace

#define LRM_TRY(expr)                  \
  do {                                 \
    const lrm_status _s = (expr);      \
    if (_s != LRM_OK) return _s;       \
  } while (0)

extern "C" {

size_t lrm_workspace_bytes(const lrm_problem* problem) {
  if (check_problem(problem) != LRM_OK) return 0;
  const size_t a = lrm::ws_layout(*problem).total, b = lrm::ws_layout(fc1_problem(*problem)).total;
  return a > b ? a : b;
}

lrm_status lrm_plan_quotas(const lrm_problem* problem, const lrm_quota_policy* policy,
                           const int32_t* topk_idx, int32_t* counts, int32_t* fwd_off,
                           int32_t* row_pair, int32_t* quota, int32_t* cmp_off, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!policy || !topk_idx || !counts || !fwd_off || !row_pair || !quota || !cmp_off)
    return LRM_ERR_INVALID_ARGUMENT;
  if (!policy->full && (policy->rho_den <= 0 || policy->rho_num < 0))
    return LRM_ERR_INVALID_ARGUMENT;
  if (policy->kind < LRM_QUOTA_CAP || policy->kind > LRM_QUOTA_WATERFILL) return LRM_ERR_INVALID_ARGUMENT;
  if (policy->kind == LRM_QUOTA_PROPORTIONAL && policy->cap_abs >= 0) return LRM_ERR_INVALID_ARGUMENT;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_plan(*problem, *policy, topk_idx, counts, fwd_off, row_pair, quota,
                                   cmp_off, (char*)ws, wl, stream));
}

lrm_status lrm_admit_quotas(const lrm_problem* problem, const lrm_admission* admission,
                            const int32_t* fwd_off, int32_t* quota, int32_t* cmp_off,
                            int32_t* admitted, void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  const lrm_admission* a = admission;
  if (!a || !fwd_off || !quota || !cmp_off || !admitted) return LRM_ERR_INVALID_ARGUMENT;
  if (a->n_cand < 1 || a->n_cand > LRM_MAX_CANDIDATES) return LRM_ERR_INVALID_ARGUMENT;
  if (a->kind < LRM_QUOTA_CAP || a->kind > LRM_QUOTA_WATERFILL) return LRM_ERR_INVALID_ARGUMENT;
  if (a->kind == LRM_QUOTA_PROPORTIONAL && a->cap_abs >= 0) return LRM_ERR_INVALID_ARGUMENT;
  for (int c = 0; c < a->n_cand; ++c)
    if (!a->full[c] && (a->rho_den[c] <= 0 || a->rho_num[c] < 0)) return LRM_ERR_INVALID_ARGUMENT;
  const int64_t lim = (int64_t)1 << 32;
  if (a->mem_base < 0 || a->mem_per_row < 0 || a->mem_per_row > lim || a->comm_per_row < 0 ||
      a->comm_per_row > lim || a->mem_base > ((int64_t)1 << 62))
    return LRM_ERR_INVALID_ARGUMENT;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_admit(*problem, *a, fwd_off, quota, cmp_off, admitted, stream));
}

lrm_status lrm_score(const lrm_problem* problem, const float* topk_w, const void* g,
                     const void* phi, const int32_t* row_pair, const int32_t* fwd_off,
                     float* score, void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!topk_w || !g || !phi || !row_pair || !fwd_off || !score) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(g) || !aligned16(phi)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_score(*problem, topk_w, g, phi, row_pair, fwd_off, score, (char*)ws,
                                    wl, stream));
}

lrm_status lrm_score_norms(const lrm_problem* problem, const void* g, const void* phi, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!g || !phi) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(g) || !aligned16(phi)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_score_norms(*problem, g, phi, (char*)ws, wl, stream));
}

lrm_status lrm_score_combine(const lrm_problem* problem, const float* topk_w,
                             const int32_t* row_pair, const int32_t* fwd_off, float* score,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!topk_w || !row_pair || !fwd_off || !score) return LRM_ERR_INVALID_ARGUMENT;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_score_combine(*problem, topk_w, row_pair, fwd_off, score, (char*)ws,
                                            wl, stream));
}

lrm_status lrm_score_criterion(const lrm_problem* problem, int32_t criterion, const float* topk_w,
                               const void* g, const void* phi, const float* keys,
                               const int32_t* row_pair, const int32_t* fwd_off, float* score,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  if (criterion == LRM_CRIT_LRM)
    return lrm_score(problem, topk_w, g, phi, row_pair, fwd_off, score, ws, ws_bytes, stream);
  LRM_TRY(check_problem(problem));
  if (criterion != LRM_CRIT_GRAD_SQ && criterion != LRM_CRIT_GRAD_ABS && criterion != LRM_CRIT_RANDOM)
    return LRM_ERR_INVALID_ARGUMENT;
  if (!row_pair || !fwd_off || !score) return LRM_ERR_INVALID_ARGUMENT;
  if (criterion == LRM_CRIT_RANDOM ? !keys : !g) return LRM_ERR_INVALID_ARGUMENT;
  if (criterion != LRM_CRIT_RANDOM && !aligned16(g)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_score_criterion(*problem, criterion, g, keys, row_pair, fwd_off,
                                              score, (char*)ws, wl, stream));
}

lrm_status lrm_select(const lrm_problem* problem, const float* score, const int32_t* fwd_off,
                      const int32_t* quota, const int32_t* cmp_off, int32_t* sel_row, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!score || !fwd_off || !quota || !cmp_off || !sel_row) return LRM_ERR_INVALID_ARGUMENT;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_select(*problem, score, fwd_off, quota, cmp_off, sel_row, (char*)ws,
                                     wl, stream));
}

lrm_status lrm_compact(const lrm_problem* problem, const int32_t* sel_row, const int32_t* row_pair,
                       const int32_t* cmp_off, const float* topk_w, const void* g,
                       const void* phi, void* Gc, void* Phic, int32_t* sel_pair, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!sel_row || !row_pair || !cmp_off || !topk_w || !g || !phi || !Gc || !Phic || !sel_pair)
    return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(g) || !aligned16(phi) || !aligned16(Gc) || !aligned16(Phic))
    return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_compact(*problem, sel_row, row_pair, cmp_off, topk_w, g, phi, Gc,
                                      Phic, sel_pair, (char*)ws, wl, stream));
}

lrm_status lrm_grouped_dw(const lrm_problem* problem, const void* Gc, const void* Phic,
                          const int32_t* cmp_off, float* dW, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!Gc || !Phic || !cmp_off || !dW) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(Gc) || !aligned16(Phic) || !aligned16(dW)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_dw(*problem, Gc, Phic, cmp_off, dW, (char*)ws, wl, stream));
}

lrm_status lrm_grouped_dx(const lrm_problem* problem, const void* Gc, const void* W,
                          const int32_t* cmp_off, float* dphi, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!Gc || !W || !cmp_off || !dphi) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(Gc) || !aligned16(W) || !aligned16(dphi)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_dx(*problem, Gc, W, cmp_off, dphi, (char*)ws, wl, stream));
}

lrm_status lrm_grouped_dw_dx(const lrm_problem* problem, const void* Gc, const void* Phic,
                             const void* W, const int32_t* cmp_off, float* dW, float* dphi,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!Gc || !Phic || !W || !cmp_off || !dW || !dphi) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(Gc) || !aligned16(Phic) || !aligned16(W) || !aligned16(dW) || !aligned16(dphi))
    return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_gemms(*problem, Gc, Phic, W, cmp_off, dW, dphi, (char*)ws, wl,
                                    stream, 2));
}

lrm_status lrm_grouped_dw_dx_noalloc(const lrm_problem* problem, const void* Gc,
                                     const void* Phic, const void* W, const int32_t* cmp_off,
                                     float* dW, float* dphi, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!Gc || !Phic || !W || !cmp_off || !dW || !dphi) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(Gc) || !aligned16(Phic) || !aligned16(W) || !aligned16(dW) || !aligned16(dphi))
    return LRM_ERR_UNSUPPORTED;
  if (lrm::noalloc_layout(*problem).total > lrm::kNoallocScratchBytes)
    return LRM_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(lrm::launch_gemms_noalloc(*problem, Gc, Phic, W, cmp_off, dW, dphi, stream));
}

lrm_status lrm_swiglu_backward(const lrm_problem* problem, const int32_t* sel_row,
                                const int32_t* cmp_off, const float* dphi, const void* ac,
                                void* dH, void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!sel_row || !cmp_off || !dphi || !ac || !dH) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(dphi) || !aligned16(ac) || !aligned16(dH)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_swiglu_bwd(*problem, sel_row, cmp_off, dphi, ac, dH, (char*)ws, wl,
                                         stream));
}

lrm_status lrm_gather_tokens(const lrm_problem* problem, const int32_t* sel_pair,
                             const int32_t* cmp_off, const void* x, void* Xc, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!sel_pair || !cmp_off || !x || !Xc) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(Xc)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_gather_tokens(*problem, sel_pair, cmp_off, x, Xc, (char*)ws, wl,
                                            stream));
}

lrm_status lrm_grouped_fc1_dw(const lrm_problem* problem, const void* dH, const void* Xc,
                              const int32_t* cmp_off, float* dW1, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!dH || !Xc || !cmp_off || !dW1) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(dH) || !aligned16(Xc) || !aligned16(dW1)) return LRM_ERR_UNSUPPORTED;
  const lrm_problem q = fc1_problem(*problem);
  WsLayout wl;
  LRM_TRY(check_ws(&q, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_dw(q, dH, Xc, cmp_off, dW1, (char*)ws, wl, stream));
}

lrm_status lrm_grouped_fc1_dx(const lrm_problem* problem, const void* dH, const void* W1,
                              const int32_t* cmp_off, float* dX, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!dH || !W1 || !cmp_off || !dX) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(dH) || !aligned16(W1) || !aligned16(dX)) return LRM_ERR_UNSUPPORTED;
  const lrm_problem q = fc1_problem(*problem);
  WsLayout wl;
  LRM_TRY(check_ws(&q, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_dx(q, dH, W1, cmp_off, dX, (char*)ws, wl, stream));
}

lrm_status lrm_grouped_fc1_dw_dx(const lrm_problem* problem, const void* dH, const void* Xc,
                                 const void* W1, const int32_t* cmp_off, float* dW1, float* dX,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!dH || !Xc || !W1 || !cmp_off || !dW1 || !dX) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(dH) || !aligned16(Xc) || !aligned16(W1) || !aligned16(dW1) || !aligned16(dX))
    return LRM_ERR_UNSUPPORTED;
  const lrm_problem q = fc1_problem(*problem);
  WsLayout wl;
  LRM_TRY(check_ws(&q, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_gemms(q, dH, Xc, W1, cmp_off, dW1, dX, (char*)ws, wl, stream, 1));
}

lrm_status lrm_scatter_tokens(const lrm_problem* problem, const int32_t* sel_pair,
                              const int32_t* cmp_off, const float* dX, float* dx, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  LRM_TRY(check_problem(problem));
  if (!sel_pair || !cmp_off || !dX || !dx) return LRM_ERR_INVALID_ARGUMENT;
  if (!aligned16(dX) || !aligned16(dx)) return LRM_ERR_UNSUPPORTED;
  WsLayout wl;
  LRM_TRY(check_ws(problem, ws, ws_bytes, &wl));
  return from_hip(lrm::launch_scatter_tokens(*problem, sel_pair, cmp_off, dX, dx, (char*)ws, wl,
                                             stream));
}

lrm_status lrm_read_device_error(void* ws, int32_t* code, int32_t clear, hipStream_t stream) {
  if (!ws || !code) return LRM_ERR_INVALID_ARGUMENT;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return LRM_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return LRM_ERR_HIP;
  *code = v;
  if (clear) {
    const int32_t z = 0;
    if (hipMemcpyAsync(ws, &z, sizeof(z), hipMemcpyHostToDevice, stream) != hipSuccess)
      return LRM_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return LRM_ERR_HIP;
  }
  return LRM_OK;
}

const char* lrm_status_string(lrm_status status) {
  switch (status) {
    case LRM_OK: return "ok";
    case LRM_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LRM_ERR_UNSUPPORTED: return "unsupported problem or alignment";
    case LRM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LRM_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

}  // extern "C"
