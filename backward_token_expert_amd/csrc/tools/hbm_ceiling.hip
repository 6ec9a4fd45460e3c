// HBM throughput ceilings for the access mixes the path's memory stages use, measured with plain
// streaming kernels (16-byte accesses, non-temporal, grid-stride).  Not part of liblrm.so: the
// measurement tool backward_token_expert_amd/hbm_ceiling.py builds it into a library of its own.
//   read:  every 16-byte chunk of src read once (an XOR of the words keeps the loads alive)
//   write: every chunk of dst written once (non-temporal or plain stores)
//   mix R: every chunk of src read once and written to R places of dst (R = 1 is a copy)
// Every index stays below its buffer's chunk count (src n16, dst R * n16).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_stream(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <bool kNT>
__global__ __launch_bounds__(kThreads) void write_stream(u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = {(uint32_t)i, 1u, 2u, 3u};
    if (kNT)
      __builtin_nontemporal_store(v, dst + i);
    else
      dst[i] = v;
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void mix_stream(const u32x4* __restrict__ src,
                                                       u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
#pragma unroll
    for (int r = 0; r < R; ++r) __builtin_nontemporal_store(v, dst + (int64_t)r * n16 + i);
  }
}

// Mean over `reps` back-to-back launches after two untimed ones, in ms per launch.
template <typename F>
float time_launches(F launch, int reps) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0f;
  launch();
  launch();
  (void)hipEventRecord(a, 0);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(b, 0);
  (void)hipEventSynchronize(b);
  float ms = -1.0f;
  (void)hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (hipGetLastError() != hipSuccess) return -1.0f;
  return ms / reps;
}

}  // namespace

// kind 0: read, 1: write (non-temporal), 2..5: mix with R = kind - 1, 6: write (plain stores).  src holds n16 chunks, dst 4 * n16 (mix)
// or n16 (write), out one word per thread of `blocks` workgroups.  Returns ms per launch, or a
// negative value on an error (including an unknown kind).
extern "C" float hbm_ceiling_time(int kind, const void* src, void* dst, void* out, long long n16,
                                  int blocks, int reps) {
  const u32x4* s = (const u32x4*)src;
  u32x4* d = (u32x4*)dst;
  const dim3 g(blocks), t(kThreads);
  switch (kind) {
    case 0: return time_launches([&] { hipLaunchKernelGGL(read_stream, g, t, 0, 0, s, (int64_t)n16, (uint32_t*)out); }, reps);
    case 1: return time_launches([&] { hipLaunchKernelGGL(write_stream<true>, g, t, 0, 0, d, (int64_t)n16); }, reps);
    case 6: return time_launches([&] { hipLaunchKernelGGL(write_stream<false>, g, t, 0, 0, d, (int64_t)n16); }, reps);
    case 2: return time_launches([&] { hipLaunchKernelGGL(mix_stream<1>, g, t, 0, 0, s, d, (int64_t)n16); }, reps);
    case 3: return time_launches([&] { hipLaunchKernelGGL(mix_stream<2>, g, t, 0, 0, s, d, (int64_t)n16); }, reps);
    case 4: return time_launches([&] { hipLaunchKernelGGL(mix_stream<3>, g, t, 0, 0, s, d, (int64_t)n16); }, reps);
    case 5: return time_launches([&] { hipLaunchKernelGGL(mix_stream<4>, g, t, 0, 0, s, d, (int64_t)n16); }, reps);
  }
  return -1.0f;
}
