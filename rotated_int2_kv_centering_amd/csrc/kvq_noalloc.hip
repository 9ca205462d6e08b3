// The decode workspace as a static device array, for kvq_decode_attn_noalloc:
// callers that cannot allocate device memory (code under stream capture,
// serving loops that forbid allocation) pass inputs and outputs only.
//
// Layout of `scratch` (one copy per GPU, held until the process ends): the
// merge tickets in a fixed prefix of kStaticTicketBytes (up to 16384
// (sequence, KV head) pairs), then the split partial rows and the window rows
// of the call, as in a caller's workspace.  Every completed call leaves the
// tickets at zero, so the array needs clearing once per device; calls that
// overlap on one GPU share it and race.
#include <mutex>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ void clear_words_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t static_scratch(void** out, hipStream_t stream) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device: the device address of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0) return hipErrorInvalidDevice;
  if (static_cast<size_t>(dev) >= addr.size()) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    // Set-up on this device (current): the array's name is a host-side stand-in
    // for the device copy; from here on only its device address is used.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // the tickets start at zero: cleared once by a fill kernel on the caller's
    // stream, ahead of the call's own kernel
    (void)hipGetLastError();
    hipLaunchKernelGGL(clear_words_kernel, dim3(16), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       static_cast<int>(kStaticTicketBytes / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace kvq
