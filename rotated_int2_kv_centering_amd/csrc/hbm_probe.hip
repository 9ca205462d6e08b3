// HBM read-rate probe (measurement aid; declared in kvq_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u];
  }
  for (; i < n16; i += stride) x ^= src[i];
  uint32_t y = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) y ^= __shfl_xor(y, off);
  __shared__ uint32_t s_y[kThreads / 64];
  if ((threadIdx.x & 63) == 0) s_y[threadIdx.x >> 6] = y;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t z = 0;
    for (int w = 0; w < kThreads / 64; ++w) z ^= s_y[w];
    if (z == 0x9e3779b9u) sink[blockIdx.x] = z;
  }
}

}  // namespace

extern "C" int kvq_probe_read_stream(const void* src, size_t n_bytes, uint32_t* sink, int32_t n_workgroups,
                                     void* stream) {
  if (src == nullptr || sink == nullptr || n_workgroups < 1 || n_bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  if (n_bytes == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_stream_kernel, dim3(n_workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), n_bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
