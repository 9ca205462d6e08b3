// Decode attention read straight from the packed INT2 cache: the launcher, and
// the kernels for up to four query heads per KV head (the kernel itself is in
// kvq_decode_kernel.h).
#include "kvq_decode_kernel.h"

namespace kvq {

template hipError_t launch_decode_quads<1>(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);

hipError_t launch_decode(const DecodeParams& prm, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  (void)hipGetLastError();  // report only this call's launch errors, not stale ones
  hipError_t err;
  if (prm.g <= 4)
    err = launch_decode_quads<1>(prm, stream, ev_begin, ev_end);
  else if (prm.g <= 8)
    err = launch_decode_quads<2>(prm, stream, ev_begin, ev_end);
  else
    err = launch_decode_quads<4>(prm, stream, ev_begin, ev_end);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace kvq
