// lrm_select: per-expert TopK(q_e) with a deterministic tie-break.
//
// LRMoE (arXiv 2610.37720) Algorithm 1's per-expert TopK and Sec. 3.3: within each logical expert keep the
// q_e highest-scoring pairs (per-expert, not layer-wide).  Appendix 7.2, Prop. 7.1: keeping the
// largest scores is optimal and ties at the boundary leave several optimal sets; the kept set is
// made unique by ranking on (score descending, pair index ascending).
//
// One workgroup (16 wavefronts) per local expert:
//   1. stage the segment's float32 score bit patterns in LDS (non-negative floats order like
//      their unsigned bit patterns);
//   2. MSB-first radix select over bits 30..0 in digits of 12, 10 and 9 bits finds the q-th
//      largest key T and how many keys equal to T must be kept; after the first digit the keys
//      still in play are gathered into a short list that the later digits scan;
//   3. each thread owns a row of 32 consecutive keys: it counts those above T and equal to T, one
//      scan of the packed counts places its kept rows (key > T, or key == T among the first
//      `need` tied rows of the segment), it writes them in row order into the LDS stage, and the
//      workgroup copies the q rows out with coalesced stores.
// The stage is swizzled (stage_pos) so that both the strided passes and a thread's own row read
// without bank conflicts.  Segments longer than the LDS stage are read from global memory in
// every pass instead; their output pass gives each wavefront a contiguous run of rows, counts
// first and then writes from the keys themselves with ballot prefix sums.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsKeys = 32768;   // 128 KiB of keys: a whole 32768-token segment fits on chip
constexpr int kMaxBins = 4096;    // first radix digit: 12 bits
constexpr int kCandBase = 1024;   // candidate list: histogram words past the later digits' bins
constexpr int kMaxCand = kMaxBins - kCandBase;
constexpr int kBatch = 8;         // keys a thread loads before using them (strided passes)
constexpr int kStageBatch = 32;   // keys a thread loads before staging them (one pass for 32768)
constexpr int kOutBatch = 4;      // 64-key groups a wavefront loads ahead in the output pass

// Position of key i in the stage: rows of 32 keys, the column XOR-ed with the row (mod 32).  A
// wavefront reading 64 consecutive keys touches two rows, each a permutation of one half of the
// 64 banks; a thread reading its own row of 32 keys shares a bank with one other lane at most.
__device__ __forceinline__ int stage_pos(int i) {
  return (i & ~31) | ((i & 31) ^ ((i >> 5) & 31));
}

struct SelectSmem {
  uint32_t keys[kLdsKeys];
  int hist[kMaxBins];  // radix bins; words from kCandBase on also hold the candidate list
  int wsum[kWaves + 1];
  int pick[3];
  int weq[kWaves], wkeep[kWaves];
  int ncand;
};

// Everything after the early exits; kStaged: the segment's keys are held in LDS.
template <bool kStaged>
__device__ __forceinline__ void select_segment(SelectSmem& sm, const uint32_t* __restrict__ src,
                                               int n, int q, int r0, int o0,
                                               int32_t* __restrict__ sel_row,
                                               int32_t* __restrict__ err) {
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  uint32_t* sm_cand = (uint32_t*)(sm.hist + kCandBase);
  // A NaN or negative score is flagged and ranked as +0, so every key has its sign bit clear.
  auto sanitize = [](uint32_t v) -> uint32_t { return v > 0x7F800000u ? 0u : v; };
  auto key_at = [&](int i) -> uint32_t {
    return kStaged ? sm.keys[stage_pos(i)] : sanitize(src[i]);
  };

  for (int i = tid; i < kMaxBins; i += kThreads) sm.hist[i] = 0;
  if (tid == 0) sm.ncand = 0;
  __syncthreads();

  // Stage the keys in LDS and count the first radix digit (bits 30..19) on the way, kStageBatch
  // independent loads in flight per thread.
  bool bad = false;
  for (int base = 0; base < n; base += kStageBatch * kThreads) {
    uint32_t v[kStageBatch];
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
      const int i = base + j * kThreads + tid;
      v[j] = i < n ? src[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
      const int i = base + j * kThreads + tid;
      if (i < n) {
        bad |= v[j] > 0x7F800000u;
        const uint32_t k = sanitize(v[j]);
        if (kStaged) sm.keys[stage_pos(i)] = k;
        atomicAdd(&sm.hist[k >> 19], 1);
      }
    }
  }
  if (bad) set_error(err, LRM_DEVERR_NONFINITE);
  __syncthreads();

  // Radix select of the q-th largest key over bits 30..0, MSB first, in digits of 12, 10 and 9
  // bits.  The first digit spans the whole exponent and 4 mantissa bits, so one expert's scores
  // spread over many bins; the keys matching it (the candidates) are then gathered into a short
  // list when it fits, and the last two digits are counted over that list only.
  uint32_t prefix = 0, mask = 0;
  int rank = q;  // rank (1-based, from the top) still to locate among the candidates
  bool use_cand = false;
  int nc = 0;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 19 : (pass == 1 ? 9 : 0);
    const int nbins = pass == 0 ? 4096 : (pass == 1 ? 1024 : 512);
    const uint32_t dmask = (uint32_t)nbins - 1;
    if (pass > 0) {
      for (int i = tid; i < nbins; i += kThreads) sm.hist[i] = 0;
      __syncthreads();
      const int cnt = use_cand ? nc : n;
      for (int base = 0; base < cnt; base += kBatch * kThreads) {
        uint32_t v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = base + j * kThreads + tid;
          v[j] = i < cnt ? (use_cand ? sm_cand[i] : key_at(i)) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = base + j * kThreads + tid;
          if (i < cnt && (v[j] & mask) == prefix) atomicAdd(&sm.hist[(v[j] >> shift) & dmask], 1);
        }
      }
      __syncthreads();
    }
    // Thread t owns bins nbins-1-t*per .. nbins-per-t*per (descending); an exclusive scan over
    // threads counts the candidates in all higher bins.
    const int per = (nbins + kThreads - 1) / kThreads;
    int c = 0;
    for (int j = 0; j < per; ++j) {
      const int b = nbins - 1 - tid * per - j;
      c += b >= 0 ? sm.hist[b] : 0;
    }
    const int inc = wave_inclusive_scan(c);
    if (lane == kWave - 1) sm.wsum[w] = inc;
    __syncthreads();
    int before = 0;
    for (int x = 0; x < w; ++x) before += sm.wsum[x];
    int cum = before + inc - c;
    for (int j = 0; j < per; ++j) {
      const int b = nbins - 1 - tid * per - j;
      const int hb = b >= 0 ? sm.hist[b] : 0;
      if (b >= 0 && cum < rank && rank <= cum + hb) {
        sm.pick[0] = b;
        sm.pick[1] = cum;
        sm.pick[2] = hb;
      }
      cum += hb;
    }
    __syncthreads();
    const int dgt = sm.pick[0];
    rank -= sm.pick[1];
    const int in_bin = sm.pick[2];
    prefix |= (uint32_t)dgt << shift;
    mask |= dmask << shift;
    if (pass == 0 && in_bin <= kMaxCand) {
      // Gather the candidates of the chosen first digit (any order: only values matter here),
      // one slot reservation per wavefront and batch.  The list aliases the top of the
      // histogram, which the later digits do not use.
      for (int base = 0; base < n; base += kBatch * kThreads) {
        uint32_t v[kBatch];
        uint64_t bm[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = base + j * kThreads + tid;
          v[j] = i < n ? key_at(i) : 0u;
        }
        int tot = 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = base + j * kThreads + tid;
          bm[j] = ballot(i < n && (v[j] & mask) == prefix);
          tot += __builtin_popcountll(bm[j]);
        }
        int slot = 0;
        if (lane == 0 && tot) slot = atomicAdd(&sm.ncand, tot);
        slot = __shfl(slot, 0, kWave);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if ((bm[j] >> lane) & 1) sm_cand[slot + __builtin_popcountll(bm[j] & lt)] = v[j];
          slot += __builtin_popcountll(bm[j]);
        }
      }
      use_cand = true;
    }
    __syncthreads();
    if (pass == 0) nc = sm.ncand;
  }
  const uint32_t thr = prefix;
  const int need = rank;  // keys equal to thr that are kept, first in row order

  if constexpr (kStaged) {
    // Ordered output, thread-contiguous: thread t owns keys 32t .. 32t+31 (one row of the
    // stage).  One scan of the packed counts (keys above thr in the high half, ties in the low
    // half: fewer than q keys lie above thr, so the sum stays below 2^31) gives each thread the
    // kept keys and the ties before it; it then writes its own kept rows in row order.
    const int i0 = tid * 32;
    uint32_t kv[32];
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int i = i0 + c;
      kv[c] = i < n ? sm.keys[stage_pos(i)] : 0u;
      n_gt += (i < n && kv[c] > thr) ? 1 : 0;
      n_eq += (i < n && kv[c] == thr) ? 1 : 0;
    }
    int both = 0;
    const int before = block_exclusive_scan_1024((n_gt << 16) | n_eq, sm.wsum, &both);
    const int eq_before = before & 0xFFFF;
    int pos = (before >> 16) + (eq_before < need ? eq_before : need);
    int ties = eq_before;
    // the scan's barriers follow every read of the stage, which now holds the output
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int i = i0 + c;
      const bool valid = i < n;
      const bool is_eq = valid && kv[c] == thr;
      const bool keep = (valid && kv[c] > thr) || (is_eq && ties < need);
      ties += is_eq ? 1 : 0;
      if (keep) {
        if (pos < q) sm.keys[pos] = (uint32_t)(r0 + i);
        ++pos;
      }
    }
    __syncthreads();
    for (int j = tid; j < q; j += kThreads) sel_row[o0 + j] = (int32_t)sm.keys[j];
    return;
  }

  // Ordered output of a segment read from global memory: wavefront w owns the contiguous rows
  // [w*chunk, (w+1)*chunk).  It counts its kept and tied keys; after one barrier every wave knows
  // how many rows the waves before it keep and how many tied keys they hold, and writes its kept
  // rows in row order with ballot prefix sums (no further barriers).
  const int chunk = ((n + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const int c0 = w * chunk < n ? w * chunk : n;
  const int c1 = c0 + chunk < n ? c0 + chunk : n;
  int n_eq = 0, n_gt = 0;
  for (int base = c0; base < c1; base += kOutBatch * kWave) {
    uint32_t v[kOutBatch];
#pragma unroll
    for (int u = 0; u < kOutBatch; ++u) {
      const int i = base + u * kWave + lane;
      v[u] = i < c1 ? key_at(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kOutBatch; ++u) {
      const bool valid = base + u * kWave + lane < c1;
      n_eq += valid && v[u] == thr;
      n_gt += valid && v[u] > thr;
    }
  }
  n_eq = wave_sum_int(n_eq);
  n_gt = wave_sum_int(n_gt);
  if (lane == 0) {
    sm.weq[w] = n_eq;
    sm.wkeep[w] = n_gt;
  }
  __syncthreads();
  int eq_before = 0, pos = 0;
  for (int x = 0; x < w; ++x) {
    const int e_x = sm.weq[x];
    int tied = need - eq_before;
    tied = tied < 0 ? 0 : (tied > e_x ? e_x : tied);
    pos += sm.wkeep[x] + tied;
    eq_before += e_x;
  }
  for (int base = c0; base < c1; base += kOutBatch * kWave) {
    uint32_t v[kOutBatch];
#pragma unroll
    for (int u = 0; u < kOutBatch; ++u) {
      const int i = base + u * kWave + lane;
      v[u] = i < c1 ? key_at(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kOutBatch; ++u) {
      const int i = base + u * kWave + lane;
      const bool valid = i < c1;
      const bool is_eq = valid && v[u] == thr;
      const uint64_t beq = ballot(is_eq);
      const bool keep =
          (valid && v[u] > thr) || (is_eq && eq_before + __builtin_popcountll(beq & lt) < need);
      const uint64_t bk = ballot(keep);
      const int at = pos + __builtin_popcountll(bk & lt);
      if (keep && at < q) sel_row[o0 + at] = r0 + i;
      pos += __builtin_popcountll(bk);
      eq_before += __builtin_popcountll(beq);
    }
  }
}

__global__ __launch_bounds__(kThreads) void select_topq(const uint32_t* __restrict__ score,
                                                       const int32_t* __restrict__ fwd_off,
                                                       const int32_t* __restrict__ quota,
                                                       const int32_t* __restrict__ cmp_off,
                                                       int L_cap, int K_cap,
                                                       int32_t* __restrict__ sel_row,
                                                       int32_t* __restrict__ err) {
  __shared__ SelectSmem sm;

  const int e = blockIdx.x;
  const int tid = threadIdx.x;
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

  if (n <= kLdsKeys)
    select_segment<true>(sm, score + r0, n, q, r0, o0, sel_row, err);
  else
    select_segment<false>(sm, score + r0, n, q, r0, o0, sel_row, err);
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
