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
// bf16: v_mfma_f32_32x32x16_bf16 with fp32 accumulation; tiles of 256 rows x 128/256 columns,
// operands staged in LDS in their memory orientation and transposed on the LDS read (see the bf16
// section).  fp32: v_mfma_f32_32x32x2f32 on 128 x 128 tiles.  LDS is double-buffered with a
// register prefetch of the next K step.  Expert sizes stay on the device: dW workgroups read their
// segment bounds from cmp_off (a zero-length segment writes zeros) and take experts in order of
// decreasing retained rows from a one-workgroup ranking kernel; dphi row tiles come from a tile
// table that a one-workgroup kernel builds from cmp_off.  No atomics: every output element is
// owned by one workgroup, so results are deterministic.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// bf16 tile shapes (MFMA 32x32 tiles per wavefront in M and N; workgroup = 2 x 2 wavefronts).
#ifndef LRM_DW_MT
#define LRM_DW_MT 4
#endif
#ifndef LRM_DW_NT
#define LRM_DW_NT 4
#endif
#ifndef LRM_DW_BK
#define LRM_DW_BK 64
#endif
#ifndef LRM_DX_MT
#define LRM_DX_MT 4
#endif
#ifndef LRM_DX_NT
#define LRM_DX_NT 4
#endif
#ifndef LRM_DX_BK
#define LRM_DX_BK 64
#endif

// ------------------------------------------------------------------------------------------------
// bf16 path
//
// Workgroup = 4 wavefronts in a 2 x 2 arrangement; a wavefront owns MT x NT tiles of 32 x 32, so
// the workgroup tile is (64 MT) x (64 NT), K step 32.  Operands are staged in LDS in their memory
// orientation:
//   [k][mn] (mn contiguous): Gc and Phic for dW, W for dphi.  MFMA fragments are read with
//       ds_read_b64_tr_b16, which transposes 16-bit elements across each group of 16 lanes:
//       result lane i, element e = element (i % 4) of the 8 bytes that source lane 4e + i/4
//       addressed.  Source lane j therefore addresses row k0 + j/4, columns c0 + 4 (j % 4), and
//       result lane i receives column c0 + i at rows k0 .. k0+3; two such reads give the 8
//       consecutive reduction elements a 32x32x16 operand lane needs.
//   [mn][k] (k contiguous): Gc as the row operand of dphi; fragments are plain 16-byte reads.
// Pitches are padded (by 16 elements for [k][mn], 8 for [mn][k]) against LDS bank conflicts.
// ------------------------------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <int MT, int NT, int BK, bool AKMN, bool BKMN>
struct Tile {
  static constexpr int BM = 64 * MT, BN = 64 * NT;
  // LDS pitch (elements).  [k][mn]: +32 elements puts the four rows a 16-lane transpose read
  // touches 64 bytes apart in the 256-byte bank window, and the next 16 lanes 32 bytes further;
  // [mn][k]: +8 elements spreads 16 consecutive rows over distinct 16-byte bank groups.
  static constexpr int PA = AKMN ? BM + 32 : BK + 8;
  static constexpr int PB = BKMN ? BN + 32 : BK + 8;
  static constexpr int SA = AKMN ? BK * PA : BM * PA;  // elements per stage
  static constexpr int SB = BKMN ? BK * PB : BN * PB;
  static constexpr int CA = BM * BK / 8 / kThreads;     // 16-byte chunks per thread per stage
  static constexpr int CB = BN * BK / 8 / kThreads;
  static_assert(CA * 8 * kThreads == BM * BK && CB * 8 * kThreads == BN * BK, "tile / threads");
};

__device__ __forceinline__ s16x4 ds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// 32x32x16 operand fragment from a [k][mn] LDS tile: 32 mn starting at `base`, 16 k at `ks`.
template <int P>
__device__ __forceinline__ bf16x8 frag_kmn(const uint16_t* t, int ks, int base, int lane) {
  const int row = ks + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint16_t* p = t + row * P + col;
  const s16x4 lo = ds_tr16(p);
  const s16x4 hi = ds_tr16(p + 4 * P);
  return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Same fragment from a [mn][k] LDS tile.
template <int P>
__device__ __forceinline__ bf16x8 frag_mnk(const uint16_t* t, int ks, int base, int lane) {
  return *(const bf16x8*)(t + (base + (lane & 31)) * P + ks + 8 * (lane >> 5));
}

// Global -> registers for one stage.  [k][mn] source: rows k0.., columns mn0.. (BMN wide);
// consecutive threads take consecutive 16-byte chunks of a row.
template <int BMN, int C>
__device__ __forceinline__ void gload_kmn(const uint16_t* __restrict__ X, int64_t ld, int k0,
                                          int kend, int mn0, int mnend, int tid, uint4 (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = tid + kThreads * j, row = c / (BMN / 8), col = (c % (BMN / 8)) * 8;
    if (k0 + row < kend && mn0 + col < mnend)
      v[j] = *(const uint4*)(X + (int64_t)(k0 + row) * ld + mn0 + col);
    else
      v[j] = make_uint4(0, 0, 0, 0);
  }
}

template <int BMN, int C, int P>
__device__ __forceinline__ void sstore_kmn(uint16_t* __restrict__ t, int tid, const uint4 (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = tid + kThreads * j, row = c / (BMN / 8), col = (c % (BMN / 8)) * 8;
    *(uint4*)(t + row * P + col) = v[j];
  }
}

// [mn][k] source: rows mn0.. , reduction columns k0 .. k0+BK-1.
template <int BK, int C>
__device__ __forceinline__ void gload_mnk(const uint16_t* __restrict__ X, int64_t ld, int mn0,
                                          int mnend, int k0, int kend, int tid, uint4 (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = tid + kThreads * j, row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
    if (mn0 + row < mnend && k0 + kc < kend)
      v[j] = *(const uint4*)(X + (int64_t)(mn0 + row) * ld + k0 + kc);
    else
      v[j] = make_uint4(0, 0, 0, 0);
  }
}

template <int BK, int C, int P>
__device__ __forceinline__ void sstore_mnk(uint16_t* __restrict__ t, int tid, const uint4 (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = tid + kThreads * j, row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
    *(uint4*)(t + row * P + kc) = v[j];
  }
}

// One K step of MFMAs for this wavefront.
template <int MT, int NT, int BK, bool AKMN, bool BKMN>
__device__ __forceinline__ void mma_stage(const uint16_t* sa, const uint16_t* sb, int wm, int wn,
                                          int lane, f32x16 (&acc)[MT][NT]) {
  using C = Tile<MT, NT, BK, AKMN, BKMN>;
#pragma unroll
  for (int ks = 0; ks < BK; ks += 16) {
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int base = wm * 32 * MT + i * 32;
      a[i] = AKMN ? frag_kmn<C::PA>(sa, ks, base, lane) : frag_mnk<C::PA>(sa, ks, base, lane);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int base = wn * 32 * NT + j * 32;
      b[j] = BKMN ? frag_kmn<C::PB>(sb, ks, base, lane) : frag_mnk<C::PB>(sb, ks, base, lane);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C[m][n] for the wavefront's MT x NT tiles, rows < mend and columns < nend only.
template <int MT, int NT>
__device__ __forceinline__ void store_acc(float* __restrict__ out, int64_t ldo, int m0, int mend,
                                          int n0, int nend, int wm, int wn, int lane,
                                          const f32x16 (&acc)[MT][NT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wn * 32 * NT + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 * MT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < mend && n < nend) out[(int64_t)m * ldo + n] = acc[i][j][r];
      }
    }
}

// dW[e] tile: reduction over the retained rows of expert e.  Blocks walk the experts in the order
// of `order` (largest segment first), so the dispatcher hands out the longest tiles first.
template <int MT, int NT, int BK>
__global__ __launch_bounds__(kThreads) void dw_bf16(const uint16_t* __restrict__ Gc,
                                                   const uint16_t* __restrict__ Phic,
                                                   const int32_t* __restrict__ cmp_off,
                                                   const int32_t* __restrict__ order, int K_cap,
                                                   int h, int d, float* __restrict__ dW) {
  using C = Tile<MT, NT, BK, true, true>;
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][C::SA];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][C::SB];
  const int tn = (d + C::BN - 1) / C::BN, tm = (h + C::BM - 1) / C::BM;
  const int b = blockIdx.x, e = order[b / (tm * tn)], local = b % (tm * tn);
  const int m0 = (local / tn) * C::BM, n0 = (local % tn) * C::BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  int s = cmp_off[e], t = cmp_off[e + 1];
  s = s < 0 ? 0 : (s > K_cap ? K_cap : s);
  t = t < s ? s : (t > K_cap ? K_cap : t);
  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int nk = (t - s + BK - 1) / BK;
  uint4 va[C::CA], vb[C::CB];
  if (nk > 0) {
    gload_kmn<C::BM, C::CA>(Gc, h, s, t, m0, h, tid, va);
    gload_kmn<C::BN, C::CB>(Phic, d, s, t, n0, d, tid, vb);
    sstore_kmn<C::BM, C::CA, C::PA>(sa[0], tid, va);
    sstore_kmn<C::BN, C::CB, C::PB>(sb[0], tid, vb);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k1 = s + (kt + 1) * BK;
      gload_kmn<C::BM, C::CA>(Gc, h, k1, t, m0, h, tid, va);
      gload_kmn<C::BN, C::CB>(Phic, d, k1, t, n0, d, tid, vb);
    }
    mma_stage<MT, NT, BK, true, true>(sa[cur], sb[cur], wm, wn, lane, acc);
    if (more) {
      sstore_kmn<C::BM, C::CA, C::PA>(sa[cur ^ 1], tid, va);
      sstore_kmn<C::BN, C::CB, C::PB>(sb[cur ^ 1], tid, vb);
    }
    __syncthreads();
  }
  store_acc<MT, NT>(dW + (int64_t)e * h * d, d, m0, h, n0, d, wm, wn, lane, acc);
}

// dphi tile: rows [m0, m0 + BM) of one expert segment (from the tile table), reduction over h.
template <int MT, int NT, int BK>
__global__ __launch_bounds__(kThreads) void dx_bf16(const uint16_t* __restrict__ Gc,
                                                   const uint16_t* __restrict__ W,
                                                   const int32_t* __restrict__ cmp_off,
                                                   const int32_t* __restrict__ tiles, int K_cap,
                                                   int h, int d, float* __restrict__ dphi) {
  using C = Tile<MT, NT, BK, false, true>;
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][C::SA];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][C::SB];
  const int tile = blockIdx.x;
  if (tile >= tiles[0]) return;
  const int e = tiles[1 + 2 * tile], m0 = tiles[2 + 2 * tile];
  int mend = cmp_off[e + 1];
  mend = mend > K_cap ? K_cap : mend;
  const int n0 = blockIdx.y * C::BN;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;
  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const uint16_t* We = W + (int64_t)e * h * d;
  const int nk = (h + BK - 1) / BK;
  uint4 va[C::CA], vb[C::CB];
  gload_mnk<BK, C::CA>(Gc, h, m0, mend, 0, h, tid, va);
  gload_kmn<C::BN, C::CB>(We, d, 0, h, n0, d, tid, vb);
  sstore_mnk<BK, C::CA, C::PA>(sa[0], tid, va);
  sstore_kmn<C::BN, C::CB, C::PB>(sb[0], tid, vb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k1 = (kt + 1) * BK;
      gload_mnk<BK, C::CA>(Gc, h, m0, mend, k1, h, tid, va);
      gload_kmn<C::BN, C::CB>(We, d, k1, h, n0, d, tid, vb);
    }
    mma_stage<MT, NT, BK, false, true>(sa[cur], sb[cur], wm, wn, lane, acc);
    if (more) {
      sstore_mnk<BK, C::CA, C::PA>(sa[cur ^ 1], tid, va);
      sstore_kmn<C::BN, C::CB, C::PB>(sb[cur ^ 1], tid, vb);
    }
    __syncthreads();
  }
  store_acc<MT, NT>(dphi, d, m0, mend, n0, d, wm, wn, lane, acc);
}

// Experts ranked by retained rows, descending (ties by id): order[rank] = expert.
__global__ __launch_bounds__(1024) void dw_order(const int32_t* __restrict__ cmp_off, int E_loc,
                                                 int K_cap, int32_t* __restrict__ order) {
  __shared__ int ke[1024];
  const int tid = threadIdx.x;
  if (tid < E_loc) {
    int s = cmp_off[tid], t = cmp_off[tid + 1];
    s = s < 0 ? 0 : (s > K_cap ? K_cap : s);
    t = t < s ? s : (t > K_cap ? K_cap : t);
    ke[tid] = t - s;
  }
  __syncthreads();
  if (tid < E_loc) {
    const int mine = ke[tid];
    int rank = 0;
    for (int x = 0; x < E_loc; ++x) {
      const int o = ke[x];
      rank += (o > mine) || (o == mine && x < tid);
    }
    order[rank] = tid;
  }
}

// ------------------------------------------------------------------------------------------------
// fp32 path (v_mfma_f32_32x32x2f32); LDS tiles are [k][mn] with a padded pitch.
// ------------------------------------------------------------------------------------------------
constexpr int FBM = 128, FBN = 128;  // workgroup tile
constexpr int BKF = 16;
constexpr int PF = FBM + 4;  // floats per LDS k-row

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
  const int e = blockIdx.z, m0 = blockIdx.y * FBM, n0 = blockIdx.x * FBN;
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
  store_acc<2, 2>(dW + (int64_t)e * h * d, d, m0, h, n0, d, wm, wn, lane, acc);
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
  const int n0 = blockIdx.y * FBN;
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
  store_acc<2, 2>(dphi, d, m0, mend, n0, d, wm, wn, lane, acc);
}

// ------------------------------------------------------------------------------------------------
// dphi tile table: tiles[0] = number of row tiles, then (expert, first row) per tile, experts in
// order, `tm` rows per tile (the last tile of a segment is partial; empty segments have none).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void dx_schedule(const int32_t* __restrict__ cmp_off, int E_loc,
                                                    int K_cap, int tm, int64_t max_tiles,
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
      nt = (t - s + tm - 1) / tm;
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
        tiles[2 + 2 * idx] = s + j * tm;
      }
    }
    base_tiles = total;
    __syncthreads();
  }
  if (tid == 0) tiles[0] = (int)(base_tiles < max_tiles ? base_tiles : max_tiles);
}

template <int MT, int NT, int BK>
void launch_dw_bf16(const lrm_problem& p, const void* Gc, const void* Phic, const int32_t* cmp_off,
                    const int32_t* order, float* dW, hipStream_t s) {
  using C = Tile<MT, NT, BK, true, true>;
  const int tiles = ((p.h + C::BM - 1) / C::BM) * ((p.d + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((dw_bf16<MT, NT, BK>), dim3((unsigned)(tiles * p.E_loc)), dim3(kThreads), 0, s,
                     (const uint16_t*)Gc, (const uint16_t*)Phic, cmp_off, order, p.K_cap, p.h,
                     p.d, dW);
}

}  // namespace

hipError_t launch_dw(const lrm_problem& p, const void* Gc, const void* Phic, const int32_t* cmp_off,
                     float* dW, char* ws, const WsLayout& wl, hipStream_t s) {
  if (p.dtype == LRM_BF16) {
    int32_t* order = (int32_t*)(ws + wl.order);
    hipLaunchKernelGGL(dw_order, dim3(1), dim3(1024), 0, s, cmp_off, p.E_loc, p.K_cap, order);
    launch_dw_bf16<LRM_DW_MT, LRM_DW_NT, LRM_DW_BK>(p, Gc, Phic, cmp_off, order, dW, s);
  } else {
    const dim3 grid((p.d + FBN - 1) / FBN, (p.h + FBM - 1) / FBM, p.E_loc);
    hipLaunchKernelGGL(dw_f32, grid, dim3(kThreads), 0, s, (const float*)Gc, (const float*)Phic,
                       cmp_off, p.K_cap, p.h, p.d, dW);
  }
  return hipGetLastError();
}

hipError_t launch_dx(const lrm_problem& p, const void* Gc, const void* W, const int32_t* cmp_off,
                     float* dphi, char* ws, const WsLayout& wl, hipStream_t s) {
  int32_t* tiles = (int32_t*)(ws + wl.tiles);
  if (p.dtype == LRM_BF16) {
    constexpr int MT = LRM_DX_MT, NT = LRM_DX_NT, BK = LRM_DX_BK;
    using C = Tile<MT, NT, BK, false, true>;
    const int64_t max_tiles = ((int64_t)p.K_cap + C::BM - 1) / C::BM + p.E_loc;
    hipLaunchKernelGGL(dx_schedule, dim3(1), dim3(1024), 0, s, cmp_off, p.E_loc, p.K_cap, C::BM,
                       max_tiles, tiles);
    const dim3 grid((unsigned)max_tiles, (p.d + C::BN - 1) / C::BN);
    hipLaunchKernelGGL((dx_bf16<MT, NT, BK>), grid, dim3(kThreads), 0, s, (const uint16_t*)Gc,
                       (const uint16_t*)W, cmp_off, tiles, p.K_cap, p.h, p.d, dphi);
  } else {
    hipLaunchKernelGGL(dx_schedule, dim3(1), dim3(1024), 0, s, cmp_off, p.E_loc, p.K_cap, FBM,
                       wl.max_tiles, tiles);
    const dim3 grid((unsigned)wl.max_tiles, (p.d + FBN - 1) / FBN);
    hipLaunchKernelGGL(dx_f32, grid, dim3(kThreads), 0, s, (const float*)Gc, (const float*)W,
                       cmp_off, tiles, p.K_cap, p.h, p.d, dphi);
  }
  return hipGetLastError();
}

}  // namespace lrm
