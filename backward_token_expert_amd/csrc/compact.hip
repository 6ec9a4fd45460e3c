// lrm_compact: physical compaction of the retained rows into contiguous expert-major segments.
//
// LRMoE (arXiv 2610.37720) Sec. 3.3 and 3.4, Fig. 4 (mask -> pack -> counts/offsets -> grouped
// GEMM): retained gradient rows and their matching saved activations are packed in pair order so
// that the grouped GEMMs run over the retained rows only, with no zero-masked padding.  The
// packed gradient is the weighted cotangent delta_u = alpha_u g_t of Appendix 7.1 Eq. (5), so the
// routing weight is applied here and never again.
//
// Two passes, so that each token's gradient row g_t crosses HBM once however many of its pairs
// are kept (a token has up to k retained pairs, in different experts' segments):
//   1. rows:   per retained row i, resolve r = sel_row[i] -> p = row_pair[r]; write sel_pair[i],
//              record i in a pair -> row map in the workspace, copy phi[r] to Phic[i];
//   2. tokens: per token t, look up its k pairs in the map; if any is kept, load g_t once and
//              write RNE(fl32(alpha_p * g_t)) to each kept row.
// The map is never cleared: an entry counts only if it points inside [0, K) at a row whose
// sel_pair (written by pass 1 of the same call) names the pair, so stale entries of earlier calls
// are ignored.  Pass 2 also checks that every kept row owns its map entry (row_pair injective).
#include "lrm_device.hpp"
#include "lrm_internal.hpp"

namespace lrm {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kBatch = 8;    // retained rows resolved together by one wavefront in pass 1
constexpr int kInFlight = 8; // 16-byte loads a lane issues before its stores

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

// Pass 1.  sel_row must be strictly ascending (lrm_select writes it so: ascending rows within a
// segment, and segments follow the expert-major forward layout); a violation, or a row / pair out
// of range, sets LRM_DEVERR_INDEX and the row gets sel_pair = -1 and no data.
__global__ __launch_bounds__(kBlock) void compact_rows_phi(
    const int32_t* __restrict__ sel_row, const int32_t* __restrict__ row_pair,
    const int32_t* __restrict__ cmp_off, int E_loc, int L_cap, int K_cap, int64_t P,
    const uint4* __restrict__ phi, int pch, uint4* __restrict__ Phic,
    int32_t* __restrict__ sel_pair, int32_t* __restrict__ inv, int32_t* __restrict__ err) {
  const int lane = lane_id();
  int K = cmp_off[E_loc];
  K = K < 0 ? 0 : (K > K_cap ? K_cap : K);
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  int bad = 0;
  for (int64_t b0 = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * kBatch; b0 < K;
       b0 += nw * kBatch) {
    int r = -1;
    if (lane < kBatch && b0 + lane < K) {
      const int64_t i = b0 + lane;
      const int rr = sel_row[i];
      const int prev = i > 0 ? sel_row[i - 1] : -1;
      int p = -1;
      if (rr >= 0 && rr < L_cap && rr > prev) {
        p = row_pair[rr];
        if (p < 0 || p >= P) p = -1;
      }
      if (p < 0) {
        bad = LRM_DEVERR_INDEX;
      } else {
        r = rr;
        inv[p] = (int32_t)i;
      }
      sel_pair[i] = p;
    }
    // Copy the batch's phi rows as one flat run of nb * pch 16-byte chunks.
    const int nb = K - b0 < kBatch ? (int)(K - b0) : kBatch;
    const int total = nb * pch;
    for (int f0 = lane; f0 < total; f0 += kInFlight * kWave) {
      uint4 v[kInFlight];
      int src[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int f = f0 + u * kWave;
        const int j = f < total ? f / pch : 0;
        const int rj = __shfl(r, j, kWave);
        src[u] = (f < total && rj >= 0) ? rj : -1;
        v[u] = src[u] >= 0 ? load_nt(phi + (int64_t)rj * pch + (f - j * pch)) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int f = f0 + u * kWave;
        if (src[u] >= 0) Phic[b0 * pch + f] = v[u];
      }
    }
  }
  if (bad) set_error(err, bad);
}

// Pass 2: one wavefront per token.  The row g_t is taken in groups of kGroup * 64 16-byte chunks:
// each group is loaded once (non-temporally, as nothing reads it again), kept in registers and
// written, scaled, to every kept row of the token.  Small groups keep the kernel at 8 waves per
// SIMD (holding a whole 8 KB row per lane left it at 3), which keeps more loads in flight.
constexpr int kGroup = 4;

template <bool kBF16>
__global__ __launch_bounds__(kBlock) void compact_tokens_g(
    const int32_t* __restrict__ inv, const int32_t* __restrict__ sel_pair,
    const int32_t* __restrict__ cmp_off, int E_loc, int K_cap, int T, int k,
    const float* __restrict__ topk_w, const uint4* __restrict__ g, int gch,
    uint4* __restrict__ Gc, int32_t* __restrict__ err) {
  const int lane = lane_id();
  int K = cmp_off[E_loc];
  K = K < 0 ? 0 : (K > K_cap ? K_cap : K);
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t w0 = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  for (int64_t t = w0; t < T; t += nw) {
    for (int j0 = 0; j0 < k; j0 += kWave) {
      const int j = j0 + lane;
      const int64_t p = t * k + j;
      int i = -1;
      float a = 0.0f;
      if (j < k) {
        const int v = inv[p];
        if (v >= 0 && v < K && sel_pair[v] == p) {
          i = v;
          a = topk_w[p];
        }
      }
      const uint64_t m = ballot(i >= 0);
      if (m == 0) continue;
      const uint4* gs = g + t * gch;
      for (int c0 = 0; c0 < gch; c0 += kGroup * kWave) {
        uint4 x[kGroup];
#pragma unroll
        for (int c = 0; c < kGroup; ++c) {
          const int ch = c0 + lane + c * kWave;
          x[c] = ch < gch ? load_nt(gs + ch) : make_uint4(0, 0, 0, 0);
        }
        for (uint64_t mm = m; mm; mm &= mm - 1) {
          const int jj = __builtin_ctzll(mm);
          const int ii = __shfl(i, jj, kWave);
          const float aa = __shfl(a, jj, kWave);
          uint4* gd = Gc + (int64_t)ii * gch;
#pragma unroll
          for (int c = 0; c < kGroup; ++c) {
            const int ch = c0 + lane + c * kWave;
            if (ch < gch) gd[ch] = scale_chunk<kBF16>(x[c], aa);
          }
        }
      }
    }
  }
  // Every kept row must own its map entry; otherwise two kept rows share a pair id (row_pair not
  // injective on the kept rows) and one of them was not written.
  int bad = 0;
  const int64_t nthreads = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < K; i += nthreads) {
    const int p = sel_pair[i];
    if (p >= 0 && inv[p] != i) bad = LRM_DEVERR_INDEX;
  }
  if (bad) set_error(err, bad);
}

template <bool kBF16>
void launch_tokens(const lrm_problem& p, const int32_t* inv, const int32_t* sel_pair,
                   const int32_t* cmp_off, const float* topk_w, const uint4* g, int gch, uint4* Gc,
                   int32_t* err, hipStream_t s) {
  const int64_t tb = ((int64_t)p.T + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned nblk = (unsigned)(tb < 16384 ? tb : 16384);
  hipLaunchKernelGGL((compact_tokens_g<kBF16>), dim3(nblk), dim3(kBlock), 0, s, inv, sel_pair,
                     cmp_off, p.E_loc, p.K_cap, p.T, p.k, topk_w, g, gch, Gc, err);
}

}  // namespace

hipError_t launch_compact(const lrm_problem& p, const int32_t* sel_row, const int32_t* row_pair,
                          const int32_t* cmp_off, const float* topk_w, const void* g,
                          const void* phi, void* Gc, void* Phic, int32_t* sel_pair, char* ws,
                          const WsLayout& wl, hipStream_t s) {
  int32_t* err = (int32_t*)(ws + wl.err);
  int32_t* inv = (int32_t*)(ws + wl.inv);
  const int esz = p.dtype == LRM_BF16 ? 2 : 4;
  const int gch = p.h * esz / 16, pch = p.d * esz / 16;
  const int64_t kb = ((int64_t)p.K_cap + kBatch * kWavesPerBlock - 1) / (kBatch * kWavesPerBlock);
  const unsigned nblk = (unsigned)(kb < 4096 ? kb : 4096);
  const int64_t P = (int64_t)p.T * p.k;
  hipLaunchKernelGGL(compact_rows_phi, dim3(nblk), dim3(kBlock), 0, s, sel_row, row_pair, cmp_off,
                     p.E_loc, p.L_cap, p.K_cap, P, (const uint4*)phi, pch, (uint4*)Phic, sel_pair,
                     inv, err);
  if (p.dtype == LRM_BF16)
    launch_tokens<true>(p, inv, sel_pair, cmp_off, topk_w, (const uint4*)g, gch, (uint4*)Gc, err, s);
  else
    launch_tokens<false>(p, inv, sel_pair, cmp_off, topk_w, (const uint4*)g, gch, (uint4*)Gc, err, s);
  return hipGetLastError();
}

}  // namespace lrm
