// lrm_plan_quotas: routed counts, stable forward layout, quotas and compacted offsets.
//
// LRMoE (arXiv 2610.37720) Algorithm 1's count of each expert's pairs (N_e <- |P_e|), Sec. 3.1/3.3 (quotas fixed before
// backward, 0 <= K_e <= N_e; rows kept in a consistent pair order grouped by expert), Fig. 4
// (counts and prefix offsets define the segments).  The quota cap follows the capacity rule
// C = CF * mean load of "Expert Parallel Math Deep" ("Capacity and the exact drop-rate formula").
//
// Two launches, all sizes device-resident (no host round trip, as the TopoEP paper argues for
// planning in its host-plan latency model):
//   plan_hist    one wavefront per chunk of kPlanChunk pairs: the chunk's counts of the local
//                experts, and per workgroup of 4 chunks the counts of every expert plus a column
//                counting expert ids outside [0, E)
//   plan_place   1024-thread workgroups.  Each placing workgroup owns 16 consecutive chunks (one
//                per wavefront): it sums the local experts' columns of the histogram table itself
//                -- the totals, and the pairs in the chunks before its own -- so no workgroup
//                waits for another, derives fwd_off, and scatters its chunks' local pairs (stable
//                counting sort).  One more workgroup sums every column (counts, ids outside
//                [0, E)) and writes fwd_off, the quotas, cmp_off and the device error word
//                (overwritten, which clears what earlier calls left).
// The planning is latency-bound (about 1 MB of indices): every pass keeps 16 loads per lane in
// flight, so a pass costs one memory round trip.  The scatter ranks equal experts inside a
// wavefront with ballots (a 64-lane "match"), so the layout is stable (pair index ascending
// within each expert) without any sort.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kPlanBlock = 256;                 // 4 wavefronts, one chunk each
constexpr int kChunksPerBlock = kPlanBlock / kWave;
static_assert(kChunksPerBlock == 4, "ws_layout sizes hist_all for 4 chunks per row");
constexpr int kMaxE = 4096;

constexpr int kHistBatch = 16;  // index loads a lane issues before using them (a whole chunk)
static_assert(kPlanChunk == kHistBatch * kWave, "one load batch per chunk");

// hist_loc [nchunks][E_loc]: per chunk, its pairs of each local expert.
// hist_all [nblocks][E+1]: per workgroup of kChunksPerBlock chunks, its pairs of each expert.
__global__ __launch_bounds__(kPlanBlock) void plan_hist(const int32_t* __restrict__ idx, int64_t P,
                                                        int E, int e_lo, int E_loc, int64_t nchunks,
                                                        int32_t* __restrict__ hist_loc,
                                                        int32_t* __restrict__ hist_all) {
  __shared__ int32_t h[kChunksPerBlock][kMaxE + 1];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int cols = E + 1;  // column E counts expert ids outside [0, E)
  for (int i = threadIdx.x; i < kChunksPerBlock * cols; i += kPlanBlock) h[i / cols][i % cols] = 0;
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kChunksPerBlock + w;
  if (c < nchunks) {
    const int64_t p0 = c * kPlanChunk;
    for (int r = 0; r < kPlanChunk; r += kHistBatch * kWave) {
      int e[kHistBatch];
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const int64_t p = p0 + r + u * kWave + lane;
        e[u] = p < P ? idx[p] : -2;
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        if (e[u] == -2) continue;
        atomicAdd(&h[w][(e[u] >= 0 && e[u] < E) ? e[u] : E], 1);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kChunksPerBlock * E_loc; i += kPlanBlock) {
    const int64_t cc = (int64_t)blockIdx.x * kChunksPerBlock + i / E_loc;
    if (cc < nchunks) hist_loc[cc * E_loc + i % E_loc] = h[i / E_loc][e_lo + i % E_loc];
  }
  for (int i = threadIdx.x; i < cols; i += kPlanBlock) {
    int t = 0;
#pragma unroll
    for (int x = 0; x < kChunksPerBlock; ++x) t += h[x][i];  // rows of absent chunks stay zero
    hist_all[(int64_t)blockIdx.x * cols + i] = t;
  }
}

// Largest value over the 1024 threads of a workgroup.
__device__ __forceinline__ int block_max_1024(int v, int* sh /* >= 17 ints */) {
  const int w = threadIdx.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const int u = __shfl_xor(v, o, kWave);
    v = u > v ? u : v;
  }
  if (lane_id() == 0) sh[w] = v;
  __syncthreads();
  int m = sh[0];
  for (int i = 1; i < 16; ++i) m = sh[i] > m ? sh[i] : m;
  __syncthreads();
  return m;
}

// Proportional split of B rows over the E_loc experts (thread i holds expert i's load n, the
// loads sum to L): floor(B * n / L) each, then one more row to the B - sum(floors) experts with
// the largest remainders (B * n) mod L, the lower expert first on equal remainders.  Remainders
// of different experts share the denominator L, so comparing them as integers is exact.
__device__ __forceinline__ int proportional_quota(int n, int L, int B, int E_loc, int* rem,
                                                  int* sh) {
  const int tid = threadIdx.x;
  int fl = 0, r = 0;
  if (tid < E_loc && L > 0) {
    const int64_t prod = (int64_t)B * n;
    fl = (int)(prod / L);
    r = (int)(prod % L);
  }
  int sum_fl = 0;
  block_exclusive_scan_1024(fl, sh, &sum_fl);
  if (tid < E_loc) rem[tid] = r;
  __syncthreads();
  const int left = B - sum_fl;
  int rank = 0;  // experts ahead of this one in the (remainder desc, index asc) order
  if (tid < E_loc && left > 0)
    for (int f = 0; f < E_loc; ++f) {
      const int rf = rem[f];
      rank += (rf > r) | ((rf == r) & (f < tid));
    }
  __syncthreads();
  return fl + (tid < E_loc && rank < left ? 1 : 0);
}

// Water-fill of B rows under m = min(n, cap): every expert keeps min(m, level) at the highest
// integer level whose total is <= B, then the lowest-indexed experts with m > level get one row
// more until the total is B; q = m when the m sum to at most B.  The level is found exactly: the
// total T(x) = sum_f min(m_f, x) is piecewise linear with breakpoints at the m_f, so the last
// breakpoint v with T(v) <= B (v = 0 if none) and the slope c = #{f : m_f > v} give
// level = v + (B - T(v)) / c, which stays below the next breakpoint because T there exceeds B.
__device__ __forceinline__ int waterfill_quota(int n, int cap, int B, int E_loc, int* mv, int* sh) {
  const int tid = threadIdx.x;
  const int m = tid < E_loc ? (cap >= 0 && n > cap ? cap : n) : 0;
  int S = 0;
  block_exclusive_scan_1024(m, sh, &S);
  if (S <= B) return m;
  if (tid < E_loc) mv[tid] = m;
  __syncthreads();
  int64_t at_m = 0;  // T(m) at this expert's breakpoint
  if (tid < E_loc)
    for (int f = 0; f < E_loc; ++f) {
      const int x = mv[f];
      at_m += x < m ? x : m;
    }
  const int v = block_max_1024(tid < E_loc && at_m <= B ? m : 0, sh);
  int Tv = 0, c = 0;
  block_exclusive_scan_1024(m < v ? m : v, sh, &Tv);
  block_exclusive_scan_1024(m > v ? 1 : 0, sh, &c);
  const int level = v + (B - Tv) / c;  // c >= 1: T(max m) = S > B
  int q = m < level ? m : level;
  int total = 0;
  block_exclusive_scan_1024(q, sh, &total);
  const int above = m > level ? 1 : 0;
  int n_above = 0;
  const int before = block_exclusive_scan_1024(above, sh, &n_above);
  if (above && before < B - total) ++q;
  return q;
}


// Quota of thread tid's expert (tid < E_loc; 0 for the other threads) under `pol`, the expert
// holding seg of the Lc local rows.  Every thread of the workgroup must call it (the proportional
// and water-fill splits hold barriers); `pol` is the same for all of them.
__device__ __forceinline__ int policy_quota(const lrm_quota_policy& pol, int seg, int Lc,
                                            int E_loc, int* rem, int* sh) {
  const int tid = threadIdx.x;
  if (pol.full) return tid < E_loc ? seg : 0;
  if (pol.kind == LRM_QUOTA_CAP) {
    if (tid >= E_loc) return 0;
    const int64_t c = ((int64_t)pol.rho_num * Lc) / ((int64_t)pol.rho_den * E_loc);
    int64_t qq = seg < c ? seg : c;
    if (pol.cap_abs >= 0 && qq > pol.cap_abs) qq = pol.cap_abs;
    return (int)qq;
  }
  const int64_t bb = ((int64_t)pol.rho_num * Lc) / pol.rho_den;
  const int B = (int)(bb < Lc ? bb : Lc);
  return pol.kind == LRM_QUOTA_PROPORTIONAL ? proportional_quota(seg, Lc, B, E_loc, rem, sh)
                                            : waterfill_quota(seg, pol.cap_abs, B, E_loc, rem, sh);
}

constexpr int kPlaceWaves = 16;  // chunks per placing workgroup, one per wavefront
constexpr int kPlaceThreads = kPlaceWaves * kWave;
constexpr int kMaxLoc = 1024;
constexpr int kSumBatch = 16;    // table loads a thread keeps in flight

struct PlaceSmem {
  union {
    int base[kPlaceWaves][kMaxLoc];  // placing workgroups: next row of each local expert per wave
    int cnt[kMaxE + 1];              // the quota workgroup: every column's total
  };
  int tot[kMaxLoc];  // local totals, then the clamped segment ends
  int bef[kMaxLoc];  // local pairs in the chunks before this workgroup's first
  int rem[1024];
  int sh[32];
};

__global__ __launch_bounds__(kPlaceThreads) void plan_place(
    const int32_t* __restrict__ idx, int64_t P, int E, int e_lo, int E_loc, int nbits,
    int64_t nchunks, const int32_t* __restrict__ hist_loc, const int32_t* __restrict__ hist_all,
    int L_cap, int K_cap, lrm_quota_policy pol,
    int32_t* __restrict__ counts, int32_t* __restrict__ fwd_off, int32_t* __restrict__ row_pair,
    int32_t* __restrict__ quota, int32_t* __restrict__ cmp_off, int32_t* __restrict__ err) {
  __shared__ PlaceSmem sm;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int cols = E + 1;
  const bool quota_wg = blockIdx.x == gridDim.x - 1;
  const int64_t c_first = (int64_t)blockIdx.x * kPlaceWaves;
  for (int i = tid; i < E_loc; i += kPlaceThreads) {
    sm.tot[i] = 0;
    sm.bef[i] = 0;
  }
  if (quota_wg)
    for (int i = tid; i < cols; i += kPlaceThreads) sm.cnt[i] = 0;
  __syncthreads();

  // A placing wave's own chunk of expert ids, loaded first so the memory round trip overlaps the
  // table sums below.
  const int64_t c = c_first + w;
  const int64_t p0 = c * kPlanChunk;
  int ev[kHistBatch];
#pragma unroll
  for (int u = 0; u < kHistBatch; ++u) {
    const int64_t p = p0 + u * kWave + lane;
    ev[u] = !quota_wg && c < nchunks && p < P ? idx[p] : -1;
  }

  int nbad = 0;
  if (quota_wg) {
    // Every column's total over the per-workgroup rows: thread (rg, cc) sums rows rg, rg + R, ...
    // of columns cc, cc + C0, ... (consecutive threads read consecutive columns of a row).
    const int64_t nrows = (nchunks + kChunksPerBlock - 1) / kChunksPerBlock;
    const int C0 = cols < kPlaceThreads ? cols : kPlaceThreads, R = kPlaceThreads / C0;
    const int rg = tid / C0, cc = tid % C0;
    if (rg < R)
      for (int col = cc; col < cols; col += C0) {
        int sum = 0;
        for (int64_t r0 = rg; r0 < nrows; r0 += (int64_t)R * kSumBatch) {
          int v[kSumBatch];
#pragma unroll
          for (int u = 0; u < kSumBatch; ++u) {
            const int64_t r = r0 + (int64_t)u * R;
            v[u] = r < nrows ? hist_all[r * cols + col] : 0;
          }
#pragma unroll
          for (int u = 0; u < kSumBatch; ++u) sum += v[u];
        }
        if (sum != 0) atomicAdd(&sm.cnt[col], sum);
      }
    __syncthreads();
    for (int e = tid; e < E; e += kPlaceThreads) counts[e] = sm.cnt[e];
    for (int i = tid; i < E_loc; i += kPlaceThreads) sm.tot[i] = sm.cnt[e_lo + i];
    nbad = sm.cnt[E];
  } else {
    // The local columns: J threads per local expert walk the chunks j, j + J, ...; chunks before
    // this workgroup's first add to bef, its own 16 are kept one by one for the wave offsets.
    const int J = kPlaceThreads / E_loc;
    const int el = tid % E_loc, j = tid / E_loc;
    if (j < J) {
      int t_sum = 0, b_sum = 0;
      for (int64_t c0 = j; c0 < nchunks; c0 += (int64_t)J * kSumBatch) {
        int v[kSumBatch];
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) {
          const int64_t ch = c0 + (int64_t)u * J;
          v[u] = ch < nchunks ? hist_loc[ch * E_loc + el] : 0;
        }
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) {
          const int64_t ch = c0 + (int64_t)u * J;
          if (ch >= nchunks) continue;
          t_sum += v[u];
          if (ch < c_first)
            b_sum += v[u];
          else if (ch < c_first + kPlaceWaves)
            sm.base[ch - c_first][el] = v[u];
        }
      }
      atomicAdd(&sm.tot[el], t_sum);
      atomicAdd(&sm.bef[el], b_sum);
    }
  }
  __syncthreads();

  // Forward offsets, clamped to L_cap (every workgroup derives the same values).
  const int n = tid < E_loc ? sm.tot[tid] : 0;
  int L = 0;
  const int pre = block_exclusive_scan_1024(n, sm.sh, &L);
  const int f0 = pre < L_cap ? pre : L_cap;
  const int f1 = pre + n < L_cap ? pre + n : L_cap;
  const int Lc = L < L_cap ? L : L_cap;

  if (quota_wg) {
    if (tid < E_loc) fwd_off[tid] = f0;
    if (tid == 0) fwd_off[E_loc] = Lc;
    const int q = policy_quota(pol, f1 - f0, Lc, E_loc, sm.rem, sm.sh);
    int K = 0;
    const int cpre = block_exclusive_scan_1024(q, sm.sh, &K);
    const int o0 = cpre < K_cap ? cpre : K_cap;
    const int o1 = cpre + q < K_cap ? cpre + q : K_cap;
    if (tid < E_loc) {
      cmp_off[tid] = o0;
      quota[tid] = o1 - o0;
    }
    if (tid == 0) {
      cmp_off[E_loc] = K < K_cap ? K : K_cap;
      // The first call of a sequence: its error word replaces whatever earlier calls left.
      *err = (nbad ? LRM_DEVERR_EXPERT_ID : 0) | (L > L_cap ? LRM_DEVERR_L_CAP : 0) |
             (K > K_cap ? LRM_DEVERR_K_CAP : 0);
    }
    return;
  }

  // Each wave's first row per local expert: the segment start, the pairs of earlier chunks, then
  // the counts of this workgroup's earlier chunks (waves past the last chunk get unused values).
  if (tid < E_loc) {
    int run = f0 + sm.bef[tid];
    for (int x = 0; x < kPlaceWaves; ++x) {
      const int v = sm.base[x][tid];
      sm.base[x][tid] = run;
      run += v;
    }
    sm.tot[tid] = f1;
  }
  __syncthreads();
  if (c >= nchunks) return;  // no barrier follows
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int u = 0; u < kHistBatch; ++u) {
    const int64_t p = p0 + u * kWave + lane;
    const int e = ev[u];
    const bool local = e >= e_lo && e < e_lo + E_loc;
    const int el = local ? e - e_lo : 0;
    uint64_t peers = ballot(local);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (el >> b) & 1;
      const uint64_t m = ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int leader = local ? __builtin_ctzll(peers) : lane;
    int old = 0;
    if (local && leader == lane) {
      old = sm.base[w][el];
      sm.base[w][el] = old + __builtin_popcountll(peers);
    }
    old = __shfl(old, leader, kWave);
    if (local) {
      const int row = old + __builtin_popcountll(peers & lt);
      if (row < sm.tot[el]) row_pair[row] = (int32_t)p;
    }
  }
}

// Forward-time admission (one workgroup): the candidates are tested in order; each one's quotas
// come from policy_quota on the local counts fwd_off[i+1] - fwd_off[i], and the first whose total
// K fits (K <= K_cap, mem_base + K * mem_per_row <= mem_budget, and K * comm_per_row <=
// comm_budget unless that is negative) fixes quota, cmp_off and *admitted = its index.  If none
// fits, every quota is zero and *admitted = -1.
__global__ __launch_bounds__(1024) void admit_scan(const int32_t* __restrict__ fwd_off, int E_loc,
                                                   int K_cap, lrm_admission adm,
                                                   int32_t* __restrict__ quota,
                                                   int32_t* __restrict__ cmp_off,
                                                   int32_t* __restrict__ admitted) {
  __shared__ int rem[1024];
  __shared__ int sh[32];
  const int tid = threadIdx.x;
  int seg = 0;
  if (tid < E_loc) {
    seg = fwd_off[tid + 1] - fwd_off[tid];
    seg = seg < 0 ? 0 : seg;
  }
  int Lc = 0;
  (void)block_exclusive_scan_1024(seg, sh, &Lc);
  int chosen = -1, q = 0;
  for (int c = 0; c < adm.n_cand && chosen < 0; ++c) {
    const lrm_quota_policy pol{adm.full[c], adm.rho_num[c], adm.rho_den[c], adm.cap_abs, adm.kind};
    q = policy_quota(pol, seg, Lc, E_loc, rem, sh);
    int K = 0;
    (void)block_exclusive_scan_1024(q, sh, &K);
    const bool fits = K <= K_cap && adm.mem_base + (int64_t)K * adm.mem_per_row <= adm.mem_budget &&
                      (adm.comm_budget < 0 || (int64_t)K * adm.comm_per_row <= adm.comm_budget);
    if (fits) chosen = c;            // K is the same in every thread, so is the decision
  }
  if (chosen < 0) q = 0;
  int K = 0;
  const int cpre = block_exclusive_scan_1024(q, sh, &K);
  if (tid < E_loc) {
    cmp_off[tid] = cpre;
    quota[tid] = q;
  }
  if (tid == 0) {
    cmp_off[E_loc] = K;
    *admitted = chosen;
  }
}

}  // namespace

hipError_t launch_admit(const lrm_problem& p, const lrm_admission& adm, const int32_t* fwd_off,
                        int32_t* quota, int32_t* cmp_off, int32_t* admitted, hipStream_t s) {
  hipLaunchKernelGGL(admit_scan, dim3(1), dim3(1024), 0, s, fwd_off, p.E_loc, p.K_cap, adm, quota,
                     cmp_off, admitted);
  return hipGetLastError();
}

hipError_t launch_plan(const lrm_problem& p, const lrm_quota_policy& pol, const int32_t* topk_idx,
                       int32_t* counts, int32_t* fwd_off, int32_t* row_pair, int32_t* quota,
                       int32_t* cmp_off, char* ws, const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  int32_t* hist_loc = (int32_t*)(ws + wl.hist);
  int32_t* hist_all = (int32_t*)(ws + wl.hist_all);
  const int64_t P = (int64_t)p.T * p.k;
  const unsigned nblk = (unsigned)((wl.nchunks + kChunksPerBlock - 1) / kChunksPerBlock);
  int nbits = 0;
  while ((1 << nbits) < p.E_loc) ++nbits;
  const unsigned nplace = (unsigned)((wl.nchunks + kPlaceWaves - 1) / kPlaceWaves);
  hipLaunchKernelGGL(plan_hist, dim3(nblk), dim3(kPlanBlock), 0, s, topk_idx, P, p.E, p.e_lo,
                     p.E_loc, wl.nchunks, hist_loc, hist_all);
  hipLaunchKernelGGL(plan_place, dim3(nplace + 1), dim3(kPlaceThreads), 0, s, topk_idx, P, p.E,
                     p.e_lo, p.E_loc, nbits, wl.nchunks, hist_loc, hist_all, p.L_cap, p.K_cap, pol,
                     counts,
                     fwd_off, row_pair, quota, cmp_off, err);
  return hipGetLastError();
}

}  // namespace lrm
