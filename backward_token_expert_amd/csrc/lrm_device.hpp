// Device-side helpers of liblrm (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrm {

constexpr int kWave = 64;

__device__ __forceinline__ void set_error(int32_t* err, int32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Bits of lanes strictly below the calling lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool v) { return __ballot(v); }

// Fixed-shape butterfly sum over the 64 lanes (the same tree for every wave and row).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (l >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum over the 1024 threads of a workgroup; returns the prefix, *total the sum.
// Every thread of the workgroup must call it (it holds barriers).
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* sh /* >= 17 ints */,
                                                         int* total) {
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = lane < 16 ? sh[lane] : 0;
    const int ti = wave_inclusive_scan(t);
    if (lane < 16) sh[lane] = ti - t;  // exclusive wave offsets
    if (lane == 15) sh[16] = ti;
  }
  __syncthreads();
  const int res = sh[w] + inc - v;
  *total = sh[16];
  __syncthreads();
  return res;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte streaming load of four floats (non-temporal hint: the data is read once).
__device__ __forceinline__ float4 load_nt(const float4* p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// 16-byte streaming store of four floats (non-temporal hint: the data is not read again here).
__device__ __forceinline__ void store_nt(float4* p, float4 v) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store((f32x4){v.x, v.y, v.z, v.w}, (f32x4*)p);
}

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (gfx950 hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace lrm
