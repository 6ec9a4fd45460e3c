// lrm_compact: physical compaction of the retained rows into contiguous expert-major segments.
//
// LRMoE (arXiv 2610.37720) Sec. 3.3 and 3.4, Fig. 4 (mask -> pack -> counts/offsets -> grouped
// GEMM): retained gradient rows and their matching saved activations are packed in pair order so
// that the grouped GEMMs run over the retained rows only, with no zero-masked padding.  The
// packed gradient is the weighted cotangent delta_u = alpha_u g_t of Appendix 7.1 Eq. (5), so the
// routing weight is applied here and never again.
//
// A persistent grid of wavefronts walks the K retained rows (K read on the device) in batches of 8;
// each row moves as 16-byte loads of g_t, one float32 product by alpha per element, hardware
// round-to-nearest-even to bf16 (v_cvt_pk_bf16_f32), 16-byte stores; phi is copied as bits.
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

template <bool kBF16>
__device__ __forceinline__ uint4 scale_chunk(uint4 v, float a) {
  uint4 o;
  if (kBF16) {
    o.x = pack_bf16x2(bf16_lo(v.x) * a, bf16_hi(v.x) * a);
    o.y = pack_bf16x2(bf16_lo(v.y) * a, bf16_hi(v.y) * a);
    o.z = pack_bf16x2(bf16_lo(v.z) * a, bf16_hi(v.z) * a);
    o.w = pack_bf16x2(bf16_lo(v.w) * a, bf16_hi(v.w) * a);
  } else {
    o.x = __float_as_uint(__uint_as_float(v.x) * a);
    o.y = __float_as_uint(__uint_as_float(v.y) * a);
    o.z = __float_as_uint(__uint_as_float(v.z) * a);
    o.w = __float_as_uint(__uint_as_float(v.w) * a);
  }
  return o;
}

// Moves one retained row (g part scaled and rounded, phi part copied): all of this lane's loads
// for the row are issued before its stores.
template <bool kBF16, int GC, int PC>
__device__ __forceinline__ void move_row(const uint4* __restrict__ gs, uint4* __restrict__ gd,
                                         const uint4* __restrict__ ps, uint4* __restrict__ pd,
                                         int gch, int pch, float a, int lane) {
  uint4 x[GC], y[PC];
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    const int c = lane + j * kWave;
    x[j] = c < gch ? gs[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < PC; ++j) {
    const int c = lane + j * kWave;
    y[j] = c < pch ? load_nt(ps + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    const int c = lane + j * kWave;
    if (c < gch) gd[c] = scale_chunk<kBF16>(x[j], a);
  }
#pragma unroll
  for (int j = 0; j < PC; ++j) {
    const int c = lane + j * kWave;
    if (c < pch) pd[c] = y[j];
  }
}

// Rows wider than the register-staged path (GC x 64 or PC x 64 chunks) fall back to a loop.
template <bool kBF16>
__device__ __forceinline__ void move_row_loop(const uint4* __restrict__ gs, uint4* __restrict__ gd,
                                              const uint4* __restrict__ ps, uint4* __restrict__ pd,
                                              int gch, int pch, float a, int lane) {
  for (int c = lane; c < gch; c += kWave) gd[c] = scale_chunk<kBF16>(gs[c], a);
  for (int c = lane; c < pch; c += kWave) pd[c] = load_nt(ps + c);
}

// A persistent grid of wavefronts walks the retained rows in batches of kBatch: lanes 0..kBatch-1
// resolve the batch's (forward row, pair, weight) chain once, then the wavefront moves the rows.
constexpr int kBatch = 8;

template <bool kBF16, int GC, int PC>
__global__ __launch_bounds__(kBlock) void compact_rows(
    const int32_t* __restrict__ sel_row, const int32_t* __restrict__ row_pair,
    const int32_t* __restrict__ cmp_off, int E_loc, int L_cap, int K_cap, int k, int64_t P,
    const float* __restrict__ topk_w, const uint4* __restrict__ g, const uint4* __restrict__ phi,
    int gch, int pch, uint4* __restrict__ Gc, uint4* __restrict__ Phic,
    int32_t* __restrict__ sel_pair, int32_t* __restrict__ err) {
  const int lane = lane_id();
  int K = cmp_off[E_loc];
  K = K < 0 ? 0 : (K > K_cap ? K_cap : K);
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  const bool staged = gch <= GC * kWave && pch <= PC * kWave;
  int bad = 0;
  for (int64_t b0 = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * kBatch; b0 < K;
       b0 += nw * kBatch) {
    int r = -1, p = -1;
    float a = 0.0f;
    if (lane < kBatch && b0 + lane < K) {
      r = sel_row[b0 + lane];
      if (r >= 0 && r < L_cap) {
        p = row_pair[r];
        if (p >= 0 && p < P) a = topk_w[p];
        else p = -1;
      } else {
        r = -1;
      }
      if (p < 0) bad = LRM_DEVERR_INDEX;
      else sel_pair[b0 + lane] = p;
    }
    const int nb = K - b0 < kBatch ? (int)(K - b0) : kBatch;
    for (int j = 0; j < nb; ++j) {
      const int rj = __shfl(r, j, kWave), pj = __shfl(p, j, kWave);
      const float aj = __shfl(a, j, kWave);
      if (pj < 0) continue;  // flagged above; the row is skipped
      const int64_t i = b0 + j;
      const uint4* gs = g + (int64_t)(pj / k) * gch;
      const uint4* ps = phi + (int64_t)rj * pch;
      if (staged)
        move_row<kBF16, GC, PC>(gs, Gc + i * gch, ps, Phic + i * pch, gch, pch, aj, lane);
      else
        move_row_loop<kBF16>(gs, Gc + i * gch, ps, Phic + i * pch, gch, pch, aj, lane);
    }
  }
  if (bad) set_error(err, bad);
}

}  // namespace

hipError_t launch_compact(const lrm_problem& p, const int32_t* sel_row, const int32_t* row_pair,
                          const int32_t* cmp_off, const float* topk_w, const void* g,
                          const void* phi, void* Gc, void* Phic, int32_t* sel_pair, char* ws,
                          const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  const int esz = p.dtype == LRM_BF16 ? 2 : 4;
  const int gch = p.h * esz / 16, pch = p.d * esz / 16;
  const int64_t kb = ((int64_t)p.K_cap + kBatch * kWavesPerBlock - 1) / (kBatch * kWavesPerBlock);
  const unsigned nblk = (unsigned)(kb < 4096 ? kb : 4096);
  const int64_t P = (int64_t)p.T * p.k;
  if (p.dtype == LRM_BF16)
    hipLaunchKernelGGL((compact_rows<true, 8, 4>), dim3(nblk), dim3(kBlock), 0, s, sel_row, row_pair,
                       cmp_off, p.E_loc, p.L_cap, p.K_cap, p.k, P, topk_w, (const uint4*)g,
                       (const uint4*)phi, gch, pch, (uint4*)Gc, (uint4*)Phic, sel_pair, err);
  else
    hipLaunchKernelGGL((compact_rows<false, 8, 4>), dim3(nblk), dim3(kBlock), 0, s, sel_row, row_pair,
                       cmp_off, p.E_loc, p.L_cap, p.K_cap, p.k, P, topk_w, (const uint4*)g,
                       (const uint4*)phi, gch, pch, (uint4*)Gc, (uint4*)Phic, sel_pair, err);
  return hipGetLastError();
}

}  // namespace lrm
