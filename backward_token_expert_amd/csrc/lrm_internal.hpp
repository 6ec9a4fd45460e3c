// Internal declarations shared by the host glue and the kernel translation units of liblrm.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lrm.h"

namespace lrm {

// Pairs handled by one wavefront in the counting passes of lrm_plan_quotas.
constexpr int kPlanChunk = 1024;
// Smallest row tile of the grouped input-gradient GEMMs (sizes the workspace tile table).
constexpr int kDxTileM = 64;
// Upper bound on the accelerator dies (XCDs) the GEMM schedules spread work over.
constexpr int kMaxXcd = 8;
// dW schedule: at most kMaxGroupsPerXcd groups of workgroups per die share a job list; experts far
// larger than a group's share are split along K into pieces whose partial sums (kMaxDwSlots at
// most, h x d float32 each) are added by a fix-up kernel.
constexpr int kMaxGroupsPerXcd = 4;
constexpr int kMaxDwSlots = 16;
// Header (ints) of the dW schedule: groups, groups per die, split experts, then 3 ints per split
// expert (expert, first slot, extra pieces), then the job count of every group.
constexpr int kDwHeader = 4 + 3 * kMaxDwSlots + kMaxXcd * kMaxGroupsPerXcd;
__host__ __device__ inline int64_t dw_jobs_per_group(int E_loc) { return (int64_t)E_loc + kMaxDwSlots; }

// Word of the workspace header where the fused GEMM launch keeps its kMaxXcd unit counters.
constexpr int kQueueWord = 8;
static_assert((kQueueWord + kMaxXcd + 1) * 4 <= 256, "the unit counters fit the 256-byte header");

// Layout of the caller-provided workspace (byte offsets, all 256-byte aligned).
struct WsLayout {
  size_t err;     // int32 error word; words kQueueWord.. hold the fused GEMM's unit counters
  size_t hist;     // int32 [nchunks][E_loc] per-chunk counts of the local experts
  size_t hist_all; // int32 [ceil(nchunks/4)][E+1] per 4 chunks, counts of every expert; column E
                   //                      counts expert ids outside [0, E)
  size_t gnorm;   // double [T]           ||g_t||^2
  size_t pnorm;   // double [L_cap]       ||phi_r||^2 of the split score (lrm_score_norms)
  size_t tiles;   // int32 [1 + 2*max_tiles] dx tile table: count, then (expert, row0) pairs
  size_t order;   // int32 [kDwHeader + groups * jobs * 4] dW schedule: header, per-group job lists
  size_t dwslots; // float [kMaxDwSlots][h][d] partial dW of split experts
  size_t inv;     // int32 [T*k]          compaction: pair id -> compacted row (validated on use)
  size_t total;
  int64_t nchunks;
  int64_t max_tiles;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline WsLayout ws_layout(const lrm_problem& p) {
  WsLayout w{};
  const int64_t P = (int64_t)p.T * p.k;
  w.nchunks = (P + kPlanChunk - 1) / kPlanChunk;
  w.max_tiles = ((int64_t)p.K_cap + kDxTileM - 1) / kDxTileM + p.E_loc;
  size_t off = 0;
  w.err = off;
  off += 256;
  w.hist = off;
  off = align_up(off + (size_t)w.nchunks * p.E_loc * 4, 256);
  w.hist_all = off;
  off = align_up(off + (size_t)((w.nchunks + 3) / 4) * (p.E + 1) * 4, 256);
  w.gnorm = off;
  off = align_up(off + (size_t)p.T * 8, 256);
  w.pnorm = off;
  off = align_up(off + (size_t)p.L_cap * 8, 256);
  w.tiles = off;
  off = align_up(off + (size_t)(1 + 2 * w.max_tiles) * 4, 256);
  w.order = off;
  off = align_up(off + (size_t)(kDwHeader + (int64_t)kMaxXcd * kMaxGroupsPerXcd *
                                             dw_jobs_per_group(p.E_loc) * 4) * 4, 256);
  w.inv = off;
  off = align_up(off + (size_t)P * 4, 256);
  w.dwslots = off;
  off = align_up(off + (size_t)kMaxDwSlots * p.h * p.d * 4, 256);
  w.total = off;
  return w;
}

// Allocation-free FC2 GEMMs: the schedule lives in a static device array of this many bytes (one
// per GPU), laid out as below; devices with ids up to kMaxDevices - 1 are supported.
constexpr size_t kNoallocScratchBytes = size_t(1) << 20;
constexpr int kMaxDevices = 64;
struct NoallocLayout {
  size_t queue;   // int32 [kMaxXcd + 1] unit counters of the one-launch kernel (dphi per die, dW)
  size_t sched;   // int32 dW schedule (header, per-group job lists)
  size_t tiles;   // int32 [1 + 2*max_tiles] dphi tile table
  size_t total;
  int64_t max_tiles;
};
NoallocLayout noalloc_layout(const lrm_problem& p);
hipError_t launch_gemms_noalloc(const lrm_problem& p, const void* Gc, const void* Phic,
                                const void* W, const int32_t* cmp_off, float* dW, float* dphi,
                                hipStream_t s);

// Kernel launchers (one per translation unit).  Each returns the hipError_t of its launches.
hipError_t launch_plan(const lrm_problem& p, const lrm_quota_policy& pol, const int32_t* topk_idx,
                       int32_t* counts, int32_t* fwd_off, int32_t* row_pair, int32_t* quota,
                       int32_t* cmp_off, char* ws, const WsLayout& wl, hipStream_t s);
hipError_t launch_score(const lrm_problem& p, const float* topk_w, const void* g, const void* phi,
                        const int32_t* row_pair, const int32_t* fwd_off, float* score, char* ws,
                        const WsLayout& wl, hipStream_t s);
hipError_t launch_score_norms(const lrm_problem& p, const void* g, const void* phi, char* ws,
                              const WsLayout& wl, hipStream_t s);
hipError_t launch_score_combine(const lrm_problem& p, const float* topk_w, const int32_t* row_pair,
                                const int32_t* fwd_off, float* score, char* ws, const WsLayout& wl,
                                hipStream_t s);
hipError_t launch_score_criterion(const lrm_problem& p, int criterion, const void* g,
                                  const float* keys, const int32_t* row_pair,
                                  const int32_t* fwd_off, float* score, char* ws,
                                  const WsLayout& wl, hipStream_t s);
hipError_t launch_select(const lrm_problem& p, const float* score, const int32_t* fwd_off,
                         const int32_t* quota, const int32_t* cmp_off, int32_t* sel_row, char* ws,
                         const WsLayout& wl, hipStream_t s);
// layer: 2 for FC2's gradients, 1 for FC1's (same kernels, told apart in profiles)
hipError_t launch_gemms(const lrm_problem& p, const void* Gc, const void* Phic, const void* W,
                        const int32_t* cmp_off, float* dW, float* dphi, char* ws,
                        const WsLayout& wl, hipStream_t s, int layer);
hipError_t launch_admit(const lrm_problem& p, const lrm_admission& adm, const int32_t* fwd_off,
                        int32_t* quota, int32_t* cmp_off, int32_t* admitted, hipStream_t s);
hipError_t launch_swiglu_bwd(const lrm_problem& p, const int32_t* sel_row, const int32_t* cmp_off,
                             const float* dphi, const void* ac, void* dH, char* ws,
                             const WsLayout& wl, hipStream_t s);
hipError_t launch_gather_tokens(const lrm_problem& p, const int32_t* sel_pair,
                                const int32_t* cmp_off, const void* x, void* Xc, char* ws,
                                const WsLayout& wl, hipStream_t s);
hipError_t launch_scatter_tokens(const lrm_problem& p, const int32_t* sel_pair,
                                 const int32_t* cmp_off, const float* dX, float* dx, char* ws,
                                 const WsLayout& wl, hipStream_t s);
hipError_t launch_compact(const lrm_problem& p, const int32_t* sel_row, const int32_t* row_pair,
                          const int32_t* cmp_off, const float* topk_w, const void* g,
                          const void* phi, void* Gc, void* Phic, int32_t* sel_pair, char* ws,
                          const WsLayout& wl, hipStream_t s);
hipError_t launch_dw(const lrm_problem& p, const void* Gc, const void* Phic, const int32_t* cmp_off,
                     float* dW, char* ws, const WsLayout& wl, hipStream_t s);
hipError_t launch_dx(const lrm_problem& p, const void* Gc, const void* W, const int32_t* cmp_off,
                     float* dphi, char* ws, const WsLayout& wl, hipStream_t s);

}  // namespace lrm
