// The rest of the expert backward over the retained rows: the SwiGLU activation's backward, the
// gather of FC1's input rows, and the return of FC1's input-gradient rows to their tokens.
//
// LRMoE (arXiv 2610.37720) Sec. 3.1: FC2, the activation function, FC1 and the backward dispatch
// work on one set of retained pair identities, and a kept row's input gradient goes back to the
// token and slot it came from, in an output that starts as all zeros (Algorithm 1,
// scatter-with-zeros); Sec. 3.4: repacking shrinks the row dimension of all four expert-backward
// GEMMs.  The FC1 GEMMs themselves are the grouped kernels of gemm.hip with the
// roles of the widths exchanged (their launchers are in api.hip).
//
//   swiglu_bwd      dH[i] = [dphi*c*SiLU'(a) | dphi*SiLU(a)] from the saved FC1 output [a | c] of
//                   forward row sel_row[i]; float64 arithmetic in a fixed operation order with no
//                   contraction, one rounding to the storage type
//   pair_rows       pair -> compacted-row map of the retained rows (workspace, never cleared)
//   gather_tokens   Xc[i] = x[t] for every retained row i of token t, reading each x[t] once
//   scatter_tokens  dx[t] = sum of dX[i] over the token's retained slots in slot order, in float64,
//                   rounded once to float32; zeros for a token without a retained row
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ int clamp_k(const int32_t* cmp_off, int E_loc, int K_cap) {
  const int K = cmp_off[E_loc];
  return K < 0 ? 0 : (K > K_cap ? K_cap : K);
}

// float64 -> bf16 bits, round to nearest even.  A bf16 value keeps 8 significant bits over
// float32's exponent range.  Inside the normal range (2^-126 <= |v| < 2^128) the 45 low mantissa
// bits of the float64 pattern are rounded away (a carry may step the exponent, up to 2^128, which
// converts to infinity); *ok reports whether v was inside that range.
__device__ __forceinline__ uint32_t f64_to_bf16_normal(double v, bool* ok) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  const int ex = (int)((u >> 52) & 0x7FF);
  *ok = ex >= 1023 - 126 && ex <= 1023 + 127;
  const uint64_t low = (1ull << 45) - 1;
  u += (low >> 1) + ((u >> 45) & 1);
  u &= ~low;
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}

// The same rounding for any float64: v is rounded at the spacing 2^(e-8) of its binade
// (v = m 2^e, 1/2 <= |m| < 1), never below the smallest bf16 subnormal 2^-133.
__device__ __forceinline__ uint32_t f64_to_bf16_any(double v) {
  int e;
  (void)frexp(v, &e);
  const int q = e - 8 > -133 ? e - 8 : -133;
  return __float_as_uint((float)ldexp(rint(ldexp(v, -q)), q)) >> 16;
}

// dA, dC of phi = SiLU(a) * c for the upstream dphi, in float64, in this operation order:
//   s = 1 / (1 + exp(-a)); silu = a * s; dsilu = s * (1 + a * (1 - s));
//   dA = (dphi * c) * dsilu; dC = dphi * silu.
__device__ __forceinline__ void swiglu_grad(double g, double a, double c, double& dA, double& dC) {
#pragma clang fp contract(off)
  const double s = 1.0 / (1.0 + exp(-a));
  const double silu = a * s;
  const double dsilu = s * (1.0 + a * (1.0 - s));
  dA = (g * c) * dsilu;
  dC = g * silu;
}

// One thread per chunk of 8 (bf16) or 4 (f32) columns of a retained row; chunks of a row are
// consecutive threads.  A selected row outside [0, L_cap) sets LRM_DEVERR_INDEX and gets zeros.
// Bounded to seven waves per SIMD (at most 72 VGPRs, no spills; the compiler alone takes 88 and
// five waves).
template <bool kBF16>
__global__ __launch_bounds__(kBlock, 7) void swiglu_bwd(const int32_t* __restrict__ sel_row,
                                                     const int32_t* __restrict__ cmp_off,
                                                     int E_loc, int K_cap, int L_cap, int d,
                                                     const float* __restrict__ dphi,
                                                     const void* __restrict__ ac,
                                                     void* __restrict__ dH,
                                                     int32_t* __restrict__ err) {
  constexpr int CW = kBF16 ? 8 : 4;  // columns per chunk
  const int K = clamp_k(cmp_off, E_loc, K_cap);
  const int nch = d / CW;
  // chunk f = i * nch + jc; the grid-stride step advances (i, jc) by (stride / nch, stride % nch)
  const int64_t f0 = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  const int64_t di = stride / nch;
  const int dj = (int)(stride - di * nch);
  int64_t i = f0 / nch;
  int jc = (int)(f0 - i * nch);
  int bad = 0;
  for (; i < K; i += di, jc += dj) {
    if (jc >= nch) {
      jc -= nch;
      ++i;
      if (i >= K) break;
    }
    const int j = jc * CW;
    const int r = sel_row[i];
    const bool ok = r >= 0 && r < L_cap;
    if (!ok) bad = LRM_DEVERR_INDEX;
    const float4* gp = (const float4*)(dphi + i * d + j);
    float gv[8];
    const float4 g0 = gp[0];
    gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
    if constexpr (kBF16) {
      const float4 g1 = gp[1];
      gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
    }
    if constexpr (kBF16) {
      const uint16_t* row = (const uint16_t*)ac + (int64_t)(ok ? r : 0) * 2 * d;
      const uint4 av = ok ? *(const uint4*)(row + j) : make_uint4(0, 0, 0, 0);
      const uint4 cv = ok ? *(const uint4*)(row + d + j) : make_uint4(0, 0, 0, 0);
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, cw[4] = {cv.x, cv.y, cv.z, cv.w};
      double dA[8], dC[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        swiglu_grad(gv[2 * q], bf16_lo(aw[q]), bf16_lo(cw[q]), dA[2 * q], dC[2 * q]);
        swiglu_grad(gv[2 * q + 1], bf16_hi(aw[q]), bf16_hi(cw[q]), dA[2 * q + 1], dC[2 * q + 1]);
      }
      // round in the normal range; only a chunk holding a value outside it (zero, tiny, huge)
      // takes the general rounding, so the common case skips it
      uint32_t oa[4], oc[4];
      bool all_ok = true;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bool k0, k1, k2, k3;
        oa[q] = f64_to_bf16_normal(dA[2 * q], &k0) | (f64_to_bf16_normal(dA[2 * q + 1], &k1) << 16);
        oc[q] = f64_to_bf16_normal(dC[2 * q], &k2) | (f64_to_bf16_normal(dC[2 * q + 1], &k3) << 16);
        all_ok = all_ok && k0 && k1 && k2 && k3;
      }
      if (!all_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          oa[q] = f64_to_bf16_any(dA[2 * q]) | (f64_to_bf16_any(dA[2 * q + 1]) << 16);
          oc[q] = f64_to_bf16_any(dC[2 * q]) | (f64_to_bf16_any(dC[2 * q + 1]) << 16);
        }
      }
      uint16_t* out = (uint16_t*)dH + i * 2 * d;
      if (!ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) oa[q] = oc[q] = 0;
      }
      *(uint4*)(out + j) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
      *(uint4*)(out + d + j) = make_uint4(oc[0], oc[1], oc[2], oc[3]);
    } else {
      const float* row = (const float*)ac + (int64_t)(ok ? r : 0) * 2 * d;
      const float4 av = ok ? *(const float4*)(row + j) : make_float4(0, 0, 0, 0);
      const float4 cv = ok ? *(const float4*)(row + d + j) : make_float4(0, 0, 0, 0);
      const float aa[4] = {av.x, av.y, av.z, av.w}, cc[4] = {cv.x, cv.y, cv.z, cv.w};
      float oa[4], oc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double dA, dC;
        swiglu_grad(gv[q], aa[q], cc[q], dA, dC);
        oa[q] = ok ? (float)dA : 0.0f;
        oc[q] = ok ? (float)dC : 0.0f;
      }
      float* out = (float*)dH + i * 2 * d;
      *(float4*)(out + j) = make_float4(oa[0], oa[1], oa[2], oa[3]);
      *(float4*)(out + d + j) = make_float4(oc[0], oc[1], oc[2], oc[3]);
    }
  }
  if (bad) set_error(err, bad);
}

// inv[sel_pair[i]] = i for every retained row; a pair id outside [0, P) sets LRM_DEVERR_INDEX.
__global__ __launch_bounds__(kBlock) void pair_rows(const int32_t* __restrict__ sel_pair,
                                                    const int32_t* __restrict__ cmp_off, int E_loc,
                                                    int K_cap, int64_t P, int32_t* __restrict__ inv,
                                                    int32_t* __restrict__ err) {
  const int K = clamp_k(cmp_off, E_loc, K_cap);
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < K;
       i += (int64_t)gridDim.x * kBlock) {
    const int p = sel_pair[i];
    if (p >= 0 && p < P)
      inv[p] = (int32_t)i;
    else
      bad = LRM_DEVERR_INDEX;
  }
  if (bad) set_error(err, bad);
}

// The compacted row of pair p = t*k + j, or -1: a map entry counts only if it points inside
// [0, K) at a row whose sel_pair names p, so stale entries of earlier calls are ignored.
__device__ __forceinline__ int kept_row(const int32_t* __restrict__ inv,
                                        const int32_t* __restrict__ sel_pair, int K, int64_t p) {
  const int v = inv[p];
  return (v >= 0 && v < K && sel_pair[v] == p) ? v : -1;
}

// Every retained row must own its map entry; two rows naming one pair leave one of them unwritten.
__device__ __forceinline__ void check_owners(const int32_t* __restrict__ inv,
                                             const int32_t* __restrict__ sel_pair, int K, int64_t P,
                                             int32_t* __restrict__ err) {
  int bad = 0;
  const int64_t nthreads = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < K; i += nthreads) {
    const int p = sel_pair[i];
    if (p >= 0 && p < P && inv[p] != i) bad = LRM_DEVERR_INDEX;
  }
  if (bad) set_error(err, bad);
}

// One wavefront per token: find its retained rows, load x[t] once (XC 16-byte chunks per lane kept
// in registers; XC = 0 re-reads x[t] for each row of wider rows) and copy it to each of them.
template <int XC>
__global__ __launch_bounds__(kBlock) void gather_tokens(const int32_t* __restrict__ inv,
                                                        const int32_t* __restrict__ sel_pair,
                                                        const int32_t* __restrict__ cmp_off,
                                                        int E_loc, int K_cap, int T, int k,
                                                        const uint4* __restrict__ x, int xch,
                                                        uint4* __restrict__ Xc,
                                                        int32_t* __restrict__ err) {
  const int lane = lane_id();
  const int K = clamp_k(cmp_off, E_loc, K_cap);
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
    uint4 v[XC > 0 ? XC : 1];
    bool loaded = false;
    const uint4* xs = x + t * xch;
    for (int j0 = 0; j0 < k; j0 += kWave) {
      const int j = j0 + lane;
      const int i = j < k ? kept_row(inv, sel_pair, K, t * k + j) : -1;
      uint64_t m = ballot(i >= 0);
      if (m == 0) continue;
      if (XC > 0 && !loaded) {
#pragma unroll
        for (int c = 0; c < (XC > 0 ? XC : 1); ++c) {
          const int ch = lane + c * kWave;
          v[c] = ch < xch ? xs[ch] : make_uint4(0, 0, 0, 0);
        }
        loaded = true;
      }
      while (m) {
        const int jj = __builtin_ctzll(m);
        m &= m - 1;
        uint4* dst = Xc + (int64_t)__shfl(i, jj, kWave) * xch;
        if (XC > 0) {
#pragma unroll
          for (int c = 0; c < (XC > 0 ? XC : 1); ++c) {
            const int ch = lane + c * kWave;
            if (ch < xch) dst[ch] = v[c];
          }
        } else {
          for (int ch = lane; ch < xch; ch += kWave) dst[ch] = xs[ch];
        }
      }
    }
  }
  check_owners(inv, sel_pair, K, (int64_t)T * k, err);
}

// One wavefront per token: dx[t] = sum over its retained slots, in slot order, of the float32 rows
// dX[i], accumulated in float64 from zero and rounded once; kCB float4 column chunks per lane per
// pass.  Tokens without a retained row get zeros.  dX rows are read and dx rows written with
// non-temporal hints (each is touched once).
constexpr int kCB = 4;

__global__ __launch_bounds__(kBlock) void scatter_tokens(const int32_t* __restrict__ inv,
                                                         const int32_t* __restrict__ sel_pair,
                                                         const int32_t* __restrict__ cmp_off,
                                                         int E_loc, int K_cap, int T, int k,
                                                         const float4* __restrict__ dX, int hch,
                                                         float4* __restrict__ dx,
                                                         int32_t* __restrict__ err) {
  const int lane = lane_id();
  const int K = clamp_k(cmp_off, E_loc, K_cap);
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
    float4* dst = dx + t * hch;
    for (int c0 = 0; c0 < hch; c0 += kCB * kWave) {
      double acc[kCB][4];
#pragma unroll
      for (int c = 0; c < kCB; ++c) acc[c][0] = acc[c][1] = acc[c][2] = acc[c][3] = 0.0;
      for (int j0 = 0; j0 < k; j0 += kWave) {
        const int j = j0 + lane;
        const int i = j < k ? kept_row(inv, sel_pair, K, t * k + j) : -1;
        uint64_t m = ballot(i >= 0);
        while (m) {                                   // slots in ascending order
          const int jj = __builtin_ctzll(m);
          m &= m - 1;
          const float4* src = dX + (int64_t)__shfl(i, jj, kWave) * hch;
          float4 v[kCB];
#pragma unroll
          for (int c = 0; c < kCB; ++c) {
            const int ch = c0 + lane + c * kWave;
            v[c] = ch < hch ? load_nt(src + ch) : make_float4(0, 0, 0, 0);
          }
#pragma unroll
          for (int c = 0; c < kCB; ++c) {
            acc[c][0] += (double)v[c].x;
            acc[c][1] += (double)v[c].y;
            acc[c][2] += (double)v[c].z;
            acc[c][3] += (double)v[c].w;
          }
        }
      }
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        const int ch = c0 + lane + c * kWave;
        if (ch < hch)
          store_nt(dst + ch, make_float4((float)acc[c][0], (float)acc[c][1], (float)acc[c][2],
                                         (float)acc[c][3]));
      }
    }
  }
  check_owners(inv, sel_pair, K, (int64_t)T * k, err);
}

unsigned blocks_for(int64_t units_per_block_total, unsigned cap) {
  return (unsigned)(units_per_block_total < 1 ? 1 : (units_per_block_total < cap ? units_per_block_total : cap));
}

void launch_pair_rows(const lrm_problem& p, const int32_t* sel_pair, const int32_t* cmp_off,
                      int32_t* inv, int32_t* err, hipStream_t s) {
  const unsigned nb = blocks_for(((int64_t)p.K_cap + kBlock - 1) / kBlock, 2048);
  hipLaunchKernelGGL(pair_rows, dim3(nb), dim3(kBlock), 0, s, sel_pair, cmp_off, p.E_loc, p.K_cap,
                     (int64_t)p.T * p.k, inv, err);
}

unsigned token_blocks(const lrm_problem& p) {
  return blocks_for(((int64_t)p.T + kWavesPerBlock - 1) / kWavesPerBlock, 16384);
}

}  // namespace

hipError_t launch_swiglu_bwd(const lrm_problem& p, const int32_t* sel_row, const int32_t* cmp_off,
                             const float* dphi, const void* ac, void* dH, char* ws,
                             const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  const int cw = p.dtype == LRM_BF16 ? 8 : 4;
  const unsigned nb = blocks_for(((int64_t)p.K_cap * (p.d / cw) + kBlock - 1) / kBlock, 8192);
  if (p.dtype == LRM_BF16)
    hipLaunchKernelGGL(swiglu_bwd<true>, dim3(nb), dim3(kBlock), 0, s, sel_row, cmp_off, p.E_loc,
                       p.K_cap, p.L_cap, p.d, dphi, ac, dH, err);
  else
    hipLaunchKernelGGL(swiglu_bwd<false>, dim3(nb), dim3(kBlock), 0, s, sel_row, cmp_off, p.E_loc,
                       p.K_cap, p.L_cap, p.d, dphi, ac, dH, err);
  return hipGetLastError();
}

hipError_t launch_gather_tokens(const lrm_problem& p, const int32_t* sel_pair,
                                const int32_t* cmp_off, const void* x, void* Xc, char* ws,
                                const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  int32_t* inv = (int32_t*)(ws + wl.inv);
  launch_pair_rows(p, sel_pair, cmp_off, inv, err, s);
  const int xch = p.h * (p.dtype == LRM_BF16 ? 2 : 4) / 16;
  const unsigned nb = token_blocks(p);
  if (xch <= 4 * kWave)
    hipLaunchKernelGGL(gather_tokens<4>, dim3(nb), dim3(kBlock), 0, s, inv, sel_pair, cmp_off,
                       p.E_loc, p.K_cap, p.T, p.k, (const uint4*)x, xch, (uint4*)Xc, err);
  else if (xch <= 8 * kWave)
    hipLaunchKernelGGL(gather_tokens<8>, dim3(nb), dim3(kBlock), 0, s, inv, sel_pair, cmp_off,
                       p.E_loc, p.K_cap, p.T, p.k, (const uint4*)x, xch, (uint4*)Xc, err);
  else
    hipLaunchKernelGGL(gather_tokens<0>, dim3(nb), dim3(kBlock), 0, s, inv, sel_pair, cmp_off,
                       p.E_loc, p.K_cap, p.T, p.k, (const uint4*)x, xch, (uint4*)Xc, err);
  return hipGetLastError();
}

hipError_t launch_scatter_tokens(const lrm_problem& p, const int32_t* sel_pair,
                                 const int32_t* cmp_off, const float* dX, float* dx, char* ws,
                                 const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  int32_t* inv = (int32_t*)(ws + wl.inv);
  launch_pair_rows(p, sel_pair, cmp_off, inv, err, s);
  hipLaunchKernelGGL(scatter_tokens, dim3(token_blocks(p)), dim3(kBlock), 0, s, inv, sel_pair,
                     cmp_off, p.E_loc, p.K_cap, p.T, p.k, (const float4*)dX, p.h / 4,
                     (float4*)dx, err);
  return hipGetLastError();
}

}  // namespace lrm
