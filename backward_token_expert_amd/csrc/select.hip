// lrm_select: per-expert TopK(q_e) with a deterministic tie-break.
//
// LRMoE (arXiv 2610.37720) Algorithm 1 step 14 and Sec. 3.3: within each logical expert keep the
// q_e highest-scoring pairs (per-expert, not layer-wide).  Appendix 7.2, Prop. 7.1: keeping the
// largest scores is optimal and ties at the boundary leave several optimal sets; the kept set is
// made unique by ranking on (score descending, pair index ascending).
//
// One workgroup (16 wavefronts) per local expert:
//   1. stage the segment's float32 score bit patterns in LDS (non-negative floats order like
//      their unsigned bit patterns);
//   2. MSB-first radix select, passes of 12, 10 and 10 bits, finds the q-th largest key T and
//      how many keys equal to T must be kept;
//   3. one ordered pass keeps key > T, and the first `need` keys == T in row order, writing the
//      kept row ids ascending through a wavefront-ballot prefix sum and a cross-wave LDS scan.
// Segments longer than the LDS stage are read from global memory in every pass instead.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsKeys = 32768;   // 128 KiB of keys: a whole 32768-token segment fits on chip
constexpr int kMaxBins = 4096;    // first radix digit: 12 bits

__global__ __launch_bounds__(kThreads) void select_topq(const uint32_t* __restrict__ score,
                                                       const int32_t* __restrict__ fwd_off,
                                                       const int32_t* __restrict__ quota,
                                                       const int32_t* __restrict__ cmp_off,
                                                       int L_cap, int K_cap,
                                                       int32_t* __restrict__ sel_row,
                                                       int32_t* __restrict__ err) {
  __shared__ uint32_t keys[kLdsKeys];
  __shared__ int hist[kMaxBins];
  __shared__ int wsum[kWaves + 1];
  __shared__ int pick[2];
  __shared__ int weq[kWaves], wkeep[kWaves];

  const int e = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  int r0 = fwd_off[e], r1 = fwd_off[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > L_cap ? L_cap : r0);
  r1 = r1 < r0 ? r0 : (r1 > L_cap ? L_cap : r1);
  const int n = r1 - r0;
  int q = quota[e];
  const int o0 = cmp_off[e];
  if (q < 0 || q > n) {
    if (tid == 0) set_error(err, LRM_DEVERR_QUOTA);
    q = q < 0 ? 0 : n;
  }
  if (o0 < 0 || o0 > K_cap) {
    if (tid == 0) set_error(err, LRM_DEVERR_K_CAP);
    return;
  }
  if (o0 + q > K_cap) {
    if (tid == 0) set_error(err, LRM_DEVERR_K_CAP);
    q = K_cap - o0;
  }
  if (q == 0) return;
  if (q == n) {  // full retention: every row, already ascending
    for (int i = tid; i < n; i += kThreads) sel_row[o0 + i] = r0 + i;
    return;
  }

  const bool staged = n <= kLdsKeys;
  const uint32_t* src = score + r0;
  bool bad = false;
  // Eight independent loads in flight per thread before any is used.
  for (int base = 0; base < n; base += 8 * kThreads) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kThreads + tid;
      v[j] = i < n ? src[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kThreads + tid;
      bad |= v[j] > 0x7F800000u;  // NaN or negative
      if (staged && i < n) keys[i] = v[j];
    }
  }
  if (bad) set_error(err, LRM_DEVERR_NONFINITE);
  __syncthreads();

  // Radix select of the q-th largest key: 3 passes of 12, 10 and 10 bits, MSB first.  Scores of
  // one expert share their top bits (sign and most of the exponent), so the first digit also takes
  // 4 mantissa bits: candidates then spread over many bins and the shared-histogram atomics rarely
  // collide within a wavefront.
  uint32_t prefix = 0, mask = 0;
  int rank = q;  // rank (1-based, from the top) still to locate among the candidates
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 0 ? 4096 : 1024;
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t v = staged ? keys[i] : src[i];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & dmask], 1);
    }
    __syncthreads();
    // Thread t owns bins nbins-1-t*per .. nbins-per-t*per (descending); an exclusive scan over
    // threads counts the candidates in all higher bins.
    const int per = nbins / kThreads;
    int c = 0;
    for (int j = 0; j < per; ++j) c += hist[nbins - 1 - tid * per - j];
    const int inc = wave_inclusive_scan(c);
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int before = 0;
    for (int x = 0; x < w; ++x) before += wsum[x];
    int cum = before + inc - c;
    for (int j = 0; j < per; ++j) {
      const int b = nbins - 1 - tid * per - j, hb = hist[b];
      if (cum < rank && rank <= cum + hb) {
        pick[0] = b;
        pick[1] = cum;
      }
      cum += hb;
    }
    __syncthreads();
    const int dgt = pick[0];
    rank -= pick[1];
    prefix |= (uint32_t)dgt << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int need = rank;  // keys equal to thr that are kept, first in row order

  // Ordered output pass.
  const uint64_t lt = lanemask_lt();
  int run_eq = 0, run_keep = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const bool valid = i < n;
    const uint32_t v = valid ? (staged ? keys[i] : src[i]) : 0u;
    const bool is_eq = valid && v == thr;
    const bool is_gt = valid && v > thr;
    const uint64_t beq = ballot(is_eq);
    if (lane == 0) weq[w] = __builtin_popcountll(beq);
    __syncthreads();
    int eq_before = run_eq + __builtin_popcountll(beq & lt);
    int eq_total = 0;
    for (int x = 0; x < kWaves; ++x) {
      const int c = weq[x];
      if (x < w) eq_before += c;
      eq_total += c;
    }
    const bool keep = is_gt || (is_eq && eq_before < need);
    const uint64_t bk = ballot(keep);
    if (lane == 0) wkeep[w] = __builtin_popcountll(bk);
    __syncthreads();
    int pos = run_keep + __builtin_popcountll(bk & lt);
    int keep_total = 0;
    for (int x = 0; x < kWaves; ++x) {
      const int c = wkeep[x];
      if (x < w) pos += c;
      keep_total += c;
    }
    if (keep && pos < q) sel_row[o0 + pos] = r0 + i;
    run_eq += eq_total;
    run_keep += keep_total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_select(const lrm_problem& p, const float* score, const int32_t* fwd_off,
                         const int32_t* quota, const int32_t* cmp_off, int32_t* sel_row, char* ws,
                         const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  hipLaunchKernelGGL(select_topq, dim3(p.E_loc), dim3(kThreads), 0, s, (const uint32_t*)score,
                     fwd_off, quota, cmp_off, p.L_cap, p.K_cap, sel_row, err);
  return hipGetLastError();
}

}  // namespace lrm
