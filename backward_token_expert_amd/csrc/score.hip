// lrm_score: Load Recalibration Metric of every local forward row.
//
// LRMoE (arXiv 2610.37720) Sec. 3.2, Prop. 3.1, Eq. (3) and Algorithm 1's score:
//   R_u = alpha_u^2 * ||g_t||_2^2 * ||phi_u||_2^2,
// the squared Frobenius norm of the pair's FC2 weight-gradient contribution (alpha_u g_t) phi_u^T,
// evaluated without materialising it (rank-one identity, Appendix 7.1 Eq. (11)-(12)).
//
// Two streaming launches, HBM-bound (about 2 flops per loaded element):
//   token_norm    ||g_t||^2 for all T tokens (one wavefront per row, 16-byte loads)
//   row_score     ||phi_r||^2 per forward row (16 lanes per row, 4 rows per wavefront), then the
//                 product with alpha^2 and ||g_t||^2
// The split form (launch_score_norms, then launch_score_combine) takes the squared norms of g and
// of every phi row up to L_cap before the layout exists -- neither norm depends on the routing --
// so a caller can run it on a second stream while the counts and quotas are planned; the product
// (row_combine) then only gathers alpha and the two norms per row.  Both forms evaluate the same
// float64 expressions in the same order, so their scores are bitwise equal.
// Squares of bf16/fp32 values are exact in float64, and the sums are accumulated in float64 with
// a fixed lane assignment and a fixed butterfly, so two rows with equal contents give bitwise
// equal scores wherever they sit; the final product is rounded once to float32.
//
// The ablation criteria of Table 2 (launch_score_criterion) reuse the token pass with squares or
// absolute values, then copy each row's token norm, or the caller's key for random drop, into
// the row's score (row_gather).
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// One 16-byte chunk added to a float64 accumulator: squares (kAbs = false) or absolute values,
// the chunk's elements in memory order.
template <bool kBF16, bool kAbs>
__device__ __forceinline__ double add_chunk(double acc, uint4 a) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (kBF16) {
      const double x0 = bf16_lo(wa[i]), x1 = bf16_hi(wa[i]);
      acc += kAbs ? fabs(x0) : x0 * x0;
      acc += kAbs ? fabs(x1) : x1 * x1;
    } else {
      const double x = __uint_as_float(wa[i]);
      acc += kAbs ? fabs(x) : x * x;
    }
  }
  return acc;
}

// This lane's share (chunks lane, lane + 64, ...) of the sum over one row of `chunks` 16-byte
// chunks, in float64.
template <bool kBF16, bool kAbs>
__device__ __forceinline__ double lane_sum(const uint4* __restrict__ row, int chunks) {
  double acc = 0.0;
  int c = lane_id();
  // Two chunks in flight per lane per step.
  for (; c + kWave < chunks; c += 2 * kWave) {
    const uint4 a = load_nt(row + c);
    const uint4 b = load_nt(row + c + kWave);
    acc = add_chunk<kBF16, kAbs>(acc, a);
    acc = add_chunk<kBF16, kAbs>(acc, b);
  }
  if (c < chunks) acc = add_chunk<kBF16, kAbs>(acc, load_nt(row + c));
  return acc;
}

// Per-token norm of g: ||g_t||_2^2 (kAbs = false) or ||g_t||_1, one wavefront per row.
template <bool kBF16, bool kAbs>
__global__ __launch_bounds__(kBlock) void token_norm(const uint4* __restrict__ g, int T,
                                                     int chunks, double* __restrict__ gnorm) {
  const int lane = lane_id();
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
    const double s = wave_sum(lane_sum<kBF16, kAbs>(g + t * chunks, chunks));
    if (lane == 0) gnorm[t] = s;
  }
}

// ||phi_r||^2 and the score of 4 forward rows per wavefront: 16 lanes per row, each lane summing
// every 16th chunk of its row, then a 16-lane butterfly (the same shape for every row).
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerWave = kWave / kLanesPerRow;

// kNorms: only ||phi_r||^2 (float64) to pnorm[r], for every row below L_cap, without reading the
// layout (fwd_off, row_pair, score and err are unused).  Eight waves per SIMD (at most 64 VGPRs,
// no spills) keep more rows' loads in flight than the compiler's own choice of five.
template <bool kBF16, bool kNorms>
__global__ __launch_bounds__(kBlock, 8) void row_score(const uint4* __restrict__ phi, int chunks,
                                                    const int32_t* __restrict__ fwd_off, int E_loc,
                                                    int L_cap, const int32_t* __restrict__ row_pair,
                                                    const float* __restrict__ topk_w, int k,
                                                    int64_t P, const double* __restrict__ gnorm,
                                                    float* __restrict__ score,
                                                    double* __restrict__ pnorm,
                                                    int32_t* __restrict__ err) {
  const int lane = lane_id(), sub = lane % kLanesPerRow;
  int L = L_cap;
  if (!kNorms) {
    L = fwd_off[E_loc];
    L = L < 0 ? 0 : (L > L_cap ? L_cap : L);
  }
  const int64_t groups = ((int64_t)L + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  int bad = 0;
  for (int64_t gi = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; gi < groups;
       gi += nw) {
    const int64_t r = gi * kRowsPerWave + lane / kLanesPerRow;
    const bool live = r < L;
    const int p = live && !kNorms ? row_pair[r] : 0;
    // The row's routing weight and token norm are fetched while its phi chunks stream in.
    const bool pair_ok = live && !kNorms && p >= 0 && p < P;
    const float alpha = pair_ok ? topk_w[p] : 0.0f;
    const double gn = pair_ok ? gnorm[p / k] : 0.0;
    const uint4* row = phi + (live ? r : 0) * chunks;
    double acc = 0.0;
    int c = sub;
    // four chunks in flight per lane per step
    for (; c + 3 * kLanesPerRow < chunks; c += 4 * kLanesPerRow) {
      const uint4 a0 = load_nt(row + c), a1 = load_nt(row + c + kLanesPerRow);
      const uint4 a2 = load_nt(row + c + 2 * kLanesPerRow), a3 = load_nt(row + c + 3 * kLanesPerRow);
      acc = add_chunk<kBF16, false>(acc, a0);
      acc = add_chunk<kBF16, false>(acc, a1);
      acc = add_chunk<kBF16, false>(acc, a2);
      acc = add_chunk<kBF16, false>(acc, a3);
    }
    for (; c < chunks; c += kLanesPerRow) acc = add_chunk<kBF16, false>(acc, load_nt(row + c));
#pragma unroll
    for (int o = kLanesPerRow / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (kNorms) {
      if (live && sub == 0) pnorm[r] = acc;
    } else if (live && sub == 0) {
      float out = 0.0f;
      if (!pair_ok) {
        bad |= LRM_DEVERR_INDEX;
      } else {
        const double a = (double)alpha;
        out = (float)(((a * a) * gn) * acc);
        // Scores are products of squares: anything but a finite value >= +0 is an input error.
        if (!(out >= 0.0f && out <= 3.402823466e38f)) bad |= LRM_DEVERR_NONFINITE;
      }
      score[r] = out;
    }
  }
  if (bad) set_error(err, bad);
}

// Product of the split form: score[r] = fl32(alpha_p^2 * ||g_t||^2 * ||phi_r||^2) from the norms
// in gnorm and pnorm, one row per thread, with the same checks and the same float64 expression as
// row_score.
__global__ __launch_bounds__(kBlock) void row_combine(const int32_t* __restrict__ fwd_off, int E_loc,
                                                      int L_cap, const int32_t* __restrict__ row_pair,
                                                      const float* __restrict__ topk_w, int k,
                                                      int64_t P, const double* __restrict__ gnorm,
                                                      const double* __restrict__ pnorm,
                                                      float* __restrict__ score,
                                                      int32_t* __restrict__ err) {
  int L = fwd_off[E_loc];
  L = L < 0 ? 0 : (L > L_cap ? L_cap : L);
  int bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x; r < L; r += stride) {
    const int p = row_pair[r];
    float out = 0.0f;
    if (p < 0 || p >= P) {
      bad |= LRM_DEVERR_INDEX;
    } else {
      const double a = (double)topk_w[p];
      out = (float)(((a * a) * gnorm[p / k]) * pnorm[r]);
      if (!(out >= 0.0f && out <= 3.402823466e38f)) bad |= LRM_DEVERR_NONFINITE;
    }
    score[r] = out;
  }
  if (bad) set_error(err, bad);
}

// Score of the ablation criteria: the pair's token norm (kKeys = false) or its caller-drawn key,
// one row per thread.  -0 is taken as +0 (the selection ranks by the bit pattern).
template <bool kKeys>
__global__ __launch_bounds__(kBlock) void row_gather(const int32_t* __restrict__ fwd_off, int E_loc,
                                                     int L_cap, const int32_t* __restrict__ row_pair,
                                                     int k, int64_t P,
                                                     const double* __restrict__ gnorm,
                                                     const float* __restrict__ keys,
                                                     float* __restrict__ score,
                                                     int32_t* __restrict__ err) {
  int L = fwd_off[E_loc];
  L = L < 0 ? 0 : (L > L_cap ? L_cap : L);
  int bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x; r < L; r += stride) {
    const int p = row_pair[r];
    float out = 0.0f;
    if (p < 0 || p >= P) {
      bad |= LRM_DEVERR_INDEX;
    } else {
      out = kKeys ? keys[p] + 0.0f : (float)gnorm[p / k];
      if (!(out >= 0.0f && out <= 3.402823466e38f)) bad |= LRM_DEVERR_NONFINITE;
    }
    score[r] = out;
  }
  if (bad) set_error(err, bad);
}

}  // namespace

hipError_t launch_score_criterion(const lrm_problem& p, int criterion, const void* g,
                                  const float* keys, const int32_t* row_pair,
                                  const int32_t* fwd_off, float* score, char* ws,
                                  const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  double* gnorm = (double*)(ws + wl.gnorm);
  const int esz = p.dtype == LRM_BF16 ? 2 : 4;
  const int gch = p.h * esz / 16;
  const int64_t tb = ((int64_t)p.T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t lb = ((int64_t)p.L_cap + kBlock - 1) / kBlock;
  const unsigned gblk = (unsigned)(tb < 4096 ? tb : 4096);
  const unsigned lblk = (unsigned)(lb < 2048 ? lb : 2048);
  const int64_t P = (int64_t)p.T * p.k;
  if (criterion == LRM_CRIT_RANDOM) {
    hipLaunchKernelGGL(row_gather<true>, dim3(lblk), dim3(kBlock), 0, s, fwd_off, p.E_loc, p.L_cap,
                       row_pair, p.k, P, gnorm, keys, score, err);
    return hipGetLastError();
  }
  const bool abs = criterion == LRM_CRIT_GRAD_ABS;
  const uint4* g4 = (const uint4*)g;
  if (p.dtype == LRM_BF16) {
    if (abs)
      hipLaunchKernelGGL((token_norm<true, true>), dim3(gblk), dim3(kBlock), 0, s, g4, p.T, gch, gnorm);
    else
      hipLaunchKernelGGL((token_norm<true, false>), dim3(gblk), dim3(kBlock), 0, s, g4, p.T, gch, gnorm);
  } else {
    if (abs)
      hipLaunchKernelGGL((token_norm<false, true>), dim3(gblk), dim3(kBlock), 0, s, g4, p.T, gch, gnorm);
    else
      hipLaunchKernelGGL((token_norm<false, false>), dim3(gblk), dim3(kBlock), 0, s, g4, p.T, gch, gnorm);
  }
  hipLaunchKernelGGL(row_gather<false>, dim3(lblk), dim3(kBlock), 0, s, fwd_off, p.E_loc, p.L_cap,
                     row_pair, p.k, P, gnorm, keys, score, err);
  return hipGetLastError();
}

hipError_t launch_score(const lrm_problem& p, const float* topk_w, const void* g, const void* phi,
                        const int32_t* row_pair, const int32_t* fwd_off, float* score, char* ws,
                        const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  double* gnorm = (double*)(ws + wl.gnorm);
  const int esz = p.dtype == LRM_BF16 ? 2 : 4;
  const int gch = p.h * esz / 16, pch = p.d * esz / 16;
  // Persistent grids: enough wavefronts to keep every CU's memory pipeline full.
  const int64_t tb = ((int64_t)p.T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t lb = ((int64_t)p.L_cap + 4 * kWavesPerBlock - 1) / (4 * kWavesPerBlock);
  const unsigned gblk = (unsigned)(tb < 4096 ? tb : 4096);
  const unsigned lblk = (unsigned)(lb < 4096 ? lb : 4096);
  const int64_t P = (int64_t)p.T * p.k;
  if (p.dtype == LRM_BF16) {
    hipLaunchKernelGGL((token_norm<true, false>), dim3(gblk), dim3(kBlock), 0, s, (const uint4*)g, p.T,
                       gch, gnorm);
    hipLaunchKernelGGL((row_score<true, false>), dim3(lblk), dim3(kBlock), 0, s, (const uint4*)phi,
                       pch, fwd_off, p.E_loc, p.L_cap, row_pair, topk_w, p.k, P, gnorm, score,
                       nullptr, err);
  } else {
    hipLaunchKernelGGL((token_norm<false, false>), dim3(gblk), dim3(kBlock), 0, s, (const uint4*)g, p.T,
                       gch, gnorm);
    hipLaunchKernelGGL((row_score<false, false>), dim3(lblk), dim3(kBlock), 0, s, (const uint4*)phi,
                       pch, fwd_off, p.E_loc, p.L_cap, row_pair, topk_w, p.k, P, gnorm, score,
                       nullptr, err);
  }
  return hipGetLastError();
}

hipError_t launch_score_norms(const lrm_problem& p, const void* g, const void* phi, char* ws,
                              const WsLayout& wl, hipStream_t s) {
  double* gnorm = (double*)(ws + wl.gnorm);
  double* pnorm = (double*)(ws + wl.pnorm);
  const int esz = p.dtype == LRM_BF16 ? 2 : 4;
  const int gch = p.h * esz / 16, pch = p.d * esz / 16;
  const int64_t tb = ((int64_t)p.T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t lb = ((int64_t)p.L_cap + 4 * kWavesPerBlock - 1) / (4 * kWavesPerBlock);
  const unsigned gblk = (unsigned)(tb < 4096 ? tb : 4096);
  const unsigned lblk = (unsigned)(lb < 4096 ? lb : 4096);
  if (p.dtype == LRM_BF16) {
    hipLaunchKernelGGL((token_norm<true, false>), dim3(gblk), dim3(kBlock), 0, s, (const uint4*)g, p.T,
                       gch, gnorm);
    hipLaunchKernelGGL((row_score<true, true>), dim3(lblk), dim3(kBlock), 0, s, (const uint4*)phi,
                       pch, nullptr, p.E_loc, p.L_cap, nullptr, nullptr, p.k, (int64_t)0, nullptr,
                       nullptr, pnorm, nullptr);
  } else {
    hipLaunchKernelGGL((token_norm<false, false>), dim3(gblk), dim3(kBlock), 0, s, (const uint4*)g, p.T,
                       gch, gnorm);
    hipLaunchKernelGGL((row_score<false, true>), dim3(lblk), dim3(kBlock), 0, s, (const uint4*)phi,
                       pch, nullptr, p.E_loc, p.L_cap, nullptr, nullptr, p.k, (int64_t)0, nullptr,
                       nullptr, pnorm, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_score_combine(const lrm_problem& p, const float* topk_w, const int32_t* row_pair,
                                const int32_t* fwd_off, float* score, char* ws, const WsLayout& wl,
                                hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  const double* gnorm = (const double*)(ws + wl.gnorm);
  const double* pnorm = (const double*)(ws + wl.pnorm);
  const int64_t lb = ((int64_t)p.L_cap + kBlock - 1) / kBlock;
  const unsigned lblk = (unsigned)(lb < 2048 ? lb : 2048);
  hipLaunchKernelGGL(row_combine, dim3(lblk), dim3(kBlock), 0, s, fwd_off, p.E_loc, p.L_cap,
                     row_pair, topk_w, p.k, (int64_t)p.T * p.k, gnorm, pnorm, score, err);
  return hipGetLastError();
}

}  // namespace lrm
