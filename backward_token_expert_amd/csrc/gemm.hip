// lrm_grouped_dw / lrm_grouped_dx: variable-size grouped FC2 gradients over the retained rows.
//
// LRMoE (arXiv 2610.37720) Sec. 3.2 Eq. (1) and Appendix 7.1 Eq. (8)-(9): the FC2 weight gradient
// of expert e is the sum of the retained pairs' rank-one contributions delta_u phi_u^T;
// Appendix 7.1 Eq. (4)-(7): the FC2 input gradient of a retained pair is W_e^T delta_u.
// Sec. 3.3/3.4 and Fig. 4: the retained count of an expert is the reduction dimension of the
// weight-gradient product and the row dimension of the input-gradient product, with no padding
// rows; counts and offsets (cmp_off) describe the segments.
//
//   dW[e]   (h x d) = Gc[seg e]^T (h x K_e) * Phic[seg e] (K_e x d)   reduction over rows
//   dphi    (K_e x d) = Gc[seg e] (K_e x h) * W[e] (h x d)            reduction over h
//
// bf16: v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  A lane feeds 8 consecutive reduction
// elements of one row (A) or column (B), so every operand is staged in LDS as [mn][k] with k
// contiguous.  Operands stored in memory as [k][mn] (both dW operands, and W for dphi) are
// transposed in registers on the way in: each thread loads a 4 (k) x 8 (mn) block with four
// 16-byte loads and writes eight 8-byte LDS stores.  fp32: v_mfma_f32_32x32x2f32 with [k][mn]
// LDS tiles.
//
// Workgroup tile 128 x 128, four wavefronts of 64 x 64 (2 x 2 MFMA tiles), K step 32 (bf16) or
// 16 (fp32), LDS double-buffered with register prefetch of the next K step.  Expert sizes stay on
// the device: dW blocks read their segment bounds from cmp_off (a zero-length segment writes
// zeros); dphi row tiles come from a tile table that a one-workgroup kernel builds from cmp_off.
// No atomics: every output element is owned by one workgroup, so results are deterministic.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128;
static_assert(BM == kDxTileM, "dphi row tile must match the workspace tile table");

// ------------------------------------------------------------------------------------------------
// bf16 path
// ------------------------------------------------------------------------------------------------
constexpr int BKH = 32;           // K step (bf16 elements)
constexpr int PH = BKH + 8;       // LDS pitch in bf16 elements (80 bytes: conflict-free b128 reads)

// [k][mn] source, block (kb: 4 rows, mb: 8 columns) -> registers.
__device__ __forceinline__ void ld_kmn_bf16(const uint16_t* __restrict__ X, int64_t ld, int k0,
                                            int kend, int mn0, int mnend, int kb, int mb,
                                            uint4 v[4]) {
  const int col = mn0 + mb * 8;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = k0 + kb * 4 + r;
    if (row < kend && col < mnend)
      v[r] = *(const uint4*)(X + (int64_t)row * ld + col);
    else
      v[r] = make_uint4(0, 0, 0, 0);
  }
}

// Registers of ld_kmn_bf16 -> LDS [mn][k] (transposed): eight 8-byte stores.
__device__ __forceinline__ void st_kmn_bf16(uint16_t* __restrict__ s, int kb, int mb,
                                            const uint4 v[4]) {
  const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
  const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
  const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
  const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = i >> 1;
    uint2 o;
    if (i & 1) {
      o.x = (w0[q] >> 16) | (w1[q] & 0xFFFF0000u);
      o.y = (w2[q] >> 16) | (w3[q] & 0xFFFF0000u);
    } else {
      o.x = (w0[q] & 0xFFFFu) | (w1[q] << 16);
      o.y = (w2[q] & 0xFFFFu) | (w3[q] << 16);
    }
    *(uint2*)(s + (mb * 8 + i) * PH + kb * 4) = o;
  }
}

// [mn][k] source (k contiguous), thread t of 128 moves 4 chunks of 8 k-elements.
__device__ __forceinline__ void ld_mnk_bf16(const uint16_t* __restrict__ X, int64_t ld, int mn0,
                                            int mnend, int k0, int kend, int t, uint4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 2, kc = (c & 3) * 8;
    if (mn0 + row < mnend && k0 + kc < kend)
      v[j] = *(const uint4*)(X + (int64_t)(mn0 + row) * ld + k0 + kc);
    else
      v[j] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void st_mnk_bf16(uint16_t* __restrict__ s, int t, const uint4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 2, kc = (c & 3) * 8;
    *(uint4*)(s + row * PH + kc) = v[j];
  }
}

__device__ __forceinline__ void mma_step_bf16(const uint16_t* __restrict__ sa,
                                              const uint16_t* __restrict__ sb, int wm, int wn,
                                              int lane, f32x16 acc[2][2]) {
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < BKH; ks += 16) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8*)(sa + (wm * 64 + i * 32 + r) * PH + ks + kh);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(sb + (wn * 64 + j * 32 + r) * PH + ks + kh);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Writes the 128 x 128 tile: C[m][n] at out[(m - m0) ... ] with bounds (mend, nend).
__device__ __forceinline__ void store_tile(float* __restrict__ out, int64_t ldo, int m0, int mend,
                                           int n0, int nend, int wm, int wn, int lane,
                                           const f32x16 acc[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < mend && n < nend) out[(int64_t)m * ldo + n] = acc[i][j][r];
      }
    }
}

__global__ __launch_bounds__(kThreads) void dw_bf16(const uint16_t* __restrict__ Gc,
                                                   const uint16_t* __restrict__ Phic,
                                                   const int32_t* __restrict__ cmp_off, int K_cap,
                                                   int h, int d, float* __restrict__ dW) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * PH];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN * PH];
  const int e = blockIdx.z, m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  int s = cmp_off[e], t = cmp_off[e + 1];
  s = s < 0 ? 0 : (s > K_cap ? K_cap : s);
  t = t < s ? s : (t > K_cap ? K_cap : t);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const bool isA = tid < 128;
  const int blk = tid & 127, kb = blk & 7, mb = blk >> 3;
  const uint16_t* X = isA ? Gc : Phic;
  const int64_t ld = isA ? h : d;
  const int mn0 = isA ? m0 : n0, mnend = isA ? h : d;
  uint16_t* stage0 = isA ? sa[0] : sb[0];
  uint16_t* stage1 = isA ? sa[1] : sb[1];
  const int nk = (t - s + BKH - 1) / BKH;
  uint4 v[4];
  if (nk > 0) {
    ld_kmn_bf16(X, ld, s, t, mn0, mnend, kb, mb, v);
    st_kmn_bf16(stage0, kb, mb, v);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) ld_kmn_bf16(X, ld, s + (kt + 1) * BKH, t, mn0, mnend, kb, mb, v);
    mma_step_bf16(sa[cur], sb[cur], wm, wn, lane, acc);
    if (kt + 1 < nk) st_kmn_bf16(cur ? stage0 : stage1, kb, mb, v);
    __syncthreads();
  }
  store_tile(dW + (int64_t)e * h * d, d, m0, h, n0, d, wm, wn, lane, acc);
}

__global__ __launch_bounds__(kThreads) void dx_bf16(const uint16_t* __restrict__ Gc,
                                                   const uint16_t* __restrict__ W,
                                                   const int32_t* __restrict__ cmp_off,
                                                   const int32_t* __restrict__ tiles, int K_cap,
                                                   int h, int d, float* __restrict__ dphi) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * PH];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN * PH];
  const int tile = blockIdx.x;
  if (tile >= tiles[0]) return;
  const int e = tiles[1 + 2 * tile], m0 = tiles[2 + 2 * tile];
  int mend = cmp_off[e + 1];
  mend = mend > K_cap ? K_cap : mend;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const bool isA = tid < 128;
  const int blk = tid & 127, kb = blk & 7, mb = blk >> 3;
  const uint16_t* We = W + (int64_t)e * h * d;
  const int nk = (h + BKH - 1) / BKH;
  uint4 v[4];
  if (isA) {
    ld_mnk_bf16(Gc, h, m0, mend, 0, h, blk, v);
    st_mnk_bf16(sa[0], blk, v);
  } else {
    ld_kmn_bf16(We, d, 0, h, n0, d, kb, mb, v);
    st_kmn_bf16(sb[0], kb, mb, v);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int k1 = (kt + 1) * BKH;
    if (kt + 1 < nk) {
      if (isA) ld_mnk_bf16(Gc, h, m0, mend, k1, h, blk, v);
      else ld_kmn_bf16(We, d, k1, h, n0, d, kb, mb, v);
    }
    mma_step_bf16(sa[cur], sb[cur], wm, wn, lane, acc);
    if (kt + 1 < nk) {
      if (isA) st_mnk_bf16(sa[cur ^ 1], blk, v);
      else st_kmn_bf16(sb[cur ^ 1], kb, mb, v);
    }
    __syncthreads();
  }
  store_tile(dphi, d, m0, mend, n0, d, wm, wn, lane, acc);
}

// ------------------------------------------------------------------------------------------------
// fp32 path (v_mfma_f32_32x32x2f32); LDS tiles are [k][mn] with a padded pitch.
// ------------------------------------------------------------------------------------------------
constexpr int BKF = 16;
constexpr int PF = BM + 4;  // floats per LDS k-row

// [k][mn] source: 16 rows x 128 columns = 512 chunks of 4 floats; thread t of 128 moves 4.
__device__ __forceinline__ void ld_kmn_f32(const float* __restrict__ X, int64_t ld, int k0,
                                           int kend, int mn0, int mnend, int t, float4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 5, col = mn0 + (c & 31) * 4;
    if (k0 + row < kend && col < mnend)
      v[j] = *(const float4*)(X + (int64_t)(k0 + row) * ld + col);
    else
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ void st_kmn_f32(float* __restrict__ s, int t, const float4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 5, col = (c & 31) * 4;
    *(float4*)(s + row * PF + col) = v[j];
  }
}

// [mn][k] source: 128 rows x 16 k = 512 chunks of 4 k; stored transposed into [k][mn].
__device__ __forceinline__ void ld_mnk_f32(const float* __restrict__ X, int64_t ld, int mn0,
                                           int mnend, int k0, int kend, int t, float4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 2, kc = (c & 3) * 4;
    if (mn0 + row < mnend && k0 + kc < kend)
      v[j] = *(const float4*)(X + (int64_t)(mn0 + row) * ld + k0 + kc);
    else
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ void st_mnk_f32(float* __restrict__ s, int t, const float4 v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 128 * j, row = c >> 2, kc = (c & 3) * 4;
    s[(kc + 0) * PF + row] = v[j].x;
    s[(kc + 1) * PF + row] = v[j].y;
    s[(kc + 2) * PF + row] = v[j].z;
    s[(kc + 3) * PF + row] = v[j].w;
  }
}

__device__ __forceinline__ void mma_step_f32(const float* __restrict__ sa,
                                             const float* __restrict__ sb, int wm, int wn,
                                             int lane, f32x16 acc[2][2]) {
  const int r = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < BKF; ks += 2) {
    float a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = sa[(ks + kh) * PF + wm * 64 + i * 32 + r];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = sb[(ks + kh) * PF + wn * 64 + j * 32 + r];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads) void dw_f32(const float* __restrict__ Gc,
                                                  const float* __restrict__ Phic,
                                                  const int32_t* __restrict__ cmp_off, int K_cap,
                                                  int h, int d, float* __restrict__ dW) {
  __shared__ __attribute__((aligned(16))) float sa[2][BKF * PF];
  __shared__ __attribute__((aligned(16))) float sb[2][BKF * PF];
  const int e = blockIdx.z, m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  int s = cmp_off[e], t = cmp_off[e + 1];
  s = s < 0 ? 0 : (s > K_cap ? K_cap : s);
  t = t < s ? s : (t > K_cap ? K_cap : t);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const bool isA = tid < 128;
  const int blk = tid & 127;
  const float* X = isA ? Gc : Phic;
  const int64_t ld = isA ? h : d;
  const int mn0 = isA ? m0 : n0, mnend = isA ? h : d;
  const int nk = (t - s + BKF - 1) / BKF;
  float4 v[4];
  if (nk > 0) {
    ld_kmn_f32(X, ld, s, t, mn0, mnend, blk, v);
    st_kmn_f32(isA ? sa[0] : sb[0], blk, v);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) ld_kmn_f32(X, ld, s + (kt + 1) * BKF, t, mn0, mnend, blk, v);
    mma_step_f32(sa[cur], sb[cur], wm, wn, lane, acc);
    if (kt + 1 < nk) st_kmn_f32(isA ? sa[cur ^ 1] : sb[cur ^ 1], blk, v);
    __syncthreads();
  }
  store_tile(dW + (int64_t)e * h * d, d, m0, h, n0, d, wm, wn, lane, acc);
}

__global__ __launch_bounds__(kThreads) void dx_f32(const float* __restrict__ Gc,
                                                  const float* __restrict__ W,
                                                  const int32_t* __restrict__ cmp_off,
                                                  const int32_t* __restrict__ tiles, int K_cap,
                                                  int h, int d, float* __restrict__ dphi) {
  __shared__ __attribute__((aligned(16))) float sa[2][BKF * PF];
  __shared__ __attribute__((aligned(16))) float sb[2][BKF * PF];
  const int tile = blockIdx.x;
  if (tile >= tiles[0]) return;
  const int e = tiles[1 + 2 * tile], m0 = tiles[2 + 2 * tile];
  int mend = cmp_off[e + 1];
  mend = mend > K_cap ? K_cap : mend;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const bool isA = tid < 128;
  const int blk = tid & 127;
  const float* We = W + (int64_t)e * h * d;
  const int nk = (h + BKF - 1) / BKF;
  float4 v[4];
  if (isA) {
    ld_mnk_f32(Gc, h, m0, mend, 0, h, blk, v);
    st_mnk_f32(sa[0], blk, v);
  } else {
    ld_kmn_f32(We, d, 0, h, n0, d, blk, v);
    st_kmn_f32(sb[0], blk, v);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int k1 = (kt + 1) * BKF;
    if (kt + 1 < nk) {
      if (isA) ld_mnk_f32(Gc, h, m0, mend, k1, h, blk, v);
      else ld_kmn_f32(We, d, k1, h, n0, d, blk, v);
    }
    mma_step_f32(sa[cur], sb[cur], wm, wn, lane, acc);
    if (kt + 1 < nk) {
      if (isA) st_mnk_f32(sa[cur ^ 1], blk, v);
      else st_kmn_f32(sb[cur ^ 1], blk, v);
    }
    __syncthreads();
  }
  store_tile(dphi, d, m0, mend, n0, d, wm, wn, lane, acc);
}

// ------------------------------------------------------------------------------------------------
// dphi tile table: tiles[0] = number of row tiles, then (expert, first row) per tile, experts in
// order, BM rows per tile (the last tile of a segment is partial; empty segments have none).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void dx_schedule(const int32_t* __restrict__ cmp_off, int E_loc,
                                                    int K_cap, int64_t max_tiles,
                                                    int32_t* __restrict__ tiles) {
  __shared__ int sh[32];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  int base_tiles = 0;
  for (int e0 = 0; e0 < E_loc; e0 += 1024) {
    const int e = e0 + tid;
    int s = 0, t = 0, nt = 0;
    if (e < E_loc) {
      s = cmp_off[e];
      t = cmp_off[e + 1];
      s = s < 0 ? 0 : (s > K_cap ? K_cap : s);
      t = t < s ? s : (t > K_cap ? K_cap : t);
      nt = (t - s + BM - 1) / BM;
    }
    const int inc = wave_inclusive_scan(nt);
    if (lane == kWave - 1) sh[w] = inc;
    __syncthreads();
    int before = base_tiles, total = base_tiles;
    for (int x = 0; x < 16; ++x) {
      if (x < w) before += sh[x];
      total += sh[x];
    }
    before += inc - nt;
    for (int j = 0; j < nt; ++j) {
      const int64_t idx = before + j;
      if (idx < max_tiles) {
        tiles[1 + 2 * idx] = e;
        tiles[2 + 2 * idx] = s + j * BM;
      }
    }
    base_tiles = total;
    __syncthreads();
  }
  if (tid == 0) tiles[0] = (int)(base_tiles < max_tiles ? base_tiles : max_tiles);
}

}  // namespace

hipError_t launch_dw(const lrm_problem& p, const void* Gc, const void* Phic, const int32_t* cmp_off,
                     float* dW, char* ws, const WsLayout& wl, hipStream_t s) {
  (void)ws;
  (void)wl;
  const dim3 grid((p.d + BN - 1) / BN, (p.h + BM - 1) / BM, p.E_loc);
  if (p.dtype == LRM_BF16)
    hipLaunchKernelGGL(dw_bf16, grid, dim3(kThreads), 0, s, (const uint16_t*)Gc,
                       (const uint16_t*)Phic, cmp_off, p.K_cap, p.h, p.d, dW);
  else
    hipLaunchKernelGGL(dw_f32, grid, dim3(kThreads), 0, s, (const float*)Gc, (const float*)Phic,
                       cmp_off, p.K_cap, p.h, p.d, dW);
  return hipGetLastError();
}

hipError_t launch_dx(const lrm_problem& p, const void* Gc, const void* W, const int32_t* cmp_off,
                     float* dphi, char* ws, const WsLayout& wl, hipStream_t s) {
  int32_t* tiles = (int32_t*)(ws + wl.tiles);
  hipLaunchKernelGGL(dx_schedule, dim3(1), dim3(1024), 0, s, cmp_off, p.E_loc, p.K_cap,
                     wl.max_tiles, tiles);
  const dim3 grid((unsigned)wl.max_tiles, (p.d + BN - 1) / BN);
  if (p.dtype == LRM_BF16)
    hipLaunchKernelGGL(dx_bf16, grid, dim3(kThreads), 0, s, (const uint16_t*)Gc,
                       (const uint16_t*)W, cmp_off, tiles, p.K_cap, p.h, p.d, dphi);
  else
    hipLaunchKernelGGL(dx_f32, grid, dim3(kThreads), 0, s, (const float*)Gc, (const float*)W,
                       cmp_off, tiles, p.K_cap, p.h, p.d, dphi);
  return hipGetLastError();
}

}  // namespace lrm
