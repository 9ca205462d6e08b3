// Decode kernels for nine to sixteen query heads per KV head (kvq_decode_kernel.h).
#include "kvq_decode_kernel.h"

namespace kvq {
template hipError_t launch_decode_quads<4>(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);
}  // namespace kvq
