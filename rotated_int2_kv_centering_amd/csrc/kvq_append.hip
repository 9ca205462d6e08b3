// Quantize-append kernel: centre keys, rotate K and V, INT2-quantize, pack.
//
// OptR ("Output-Oriented Rotation for INT2 KV-Cache Quantization"), section 1:
// keys are centred by a fixed per-channel mean before rotation (every logit of
// a query then moves by one constant); section 3.1, Eq. (4): the cached vector
// z is stored as Q2(zR), here with Q2 asymmetric over groups of 32 rotated
// channels, fp16 scale/zero.
//
// Work decomposition: one workgroup of 256 threads per (tile of 16 tokens,
// KV head, tensor K or V).  For the rotation, thread (j, half) sums rows
// [64*half, 64*half + 64) of column j of R for all 16 tokens as two fma chains
// of 32 rows, with its 64 R loads issued up front (column j is read coalesced
// across threads); the two halves are added through LDS, which is the shared
// summation order of kvq_quant.h.  For quantization, each half takes 8 tokens
// and thread j owns rotated channel j (kvq_quant.h: q2_pack_channel).

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {

constexpr int kAppendTile = 16;
constexpr int kAppendThreads = 256;

template <int kIn>  // 0 = bf16 raw, 1 = fp32 raw, 2 = fp32 already centred and rotated
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    uint8_t* __restrict__ pool, int num_pages, int num_kv_heads, const void* __restrict__ k_in,
    const void* __restrict__ v_in, int n_tokens, const int32_t* __restrict__ slots, const float* __restrict__ mu,
    const float* __restrict__ r_k, const float* __restrict__ r_v, float* __restrict__ rot_out) {
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;  // 0: key, 1: value
  const int tid = threadIdx.x;
  const int j = tid & (kHeadDim - 1);  // channel
  const int half = tid >> 7;           // rotation: rows [64*half, +64) of R; packing: tokens [8*half, +8)
  const int n0 = tile * kAppendTile;
  const int nt = min(kAppendTile, n_tokens - n0);

  __shared__ float rows[kAppendTile][kHeadDim];    // centred inputs
  __shared__ float xpart[2][kAppendTile][kHeadDim];  // rotation partial sums, then rotated rows in [0]
  const void* src = tensor == 0 ? k_in : v_in;
  const float centre = (kIn != 2 && tensor == 0 && mu != nullptr) ? mu[h * kHeadDim + j] : 0.0f;
  for (int t = half; t < kAppendTile; t += 2) {
    float val = 0.0f;
    if (t < nt) {
      const size_t idx = (static_cast<size_t>(n0 + t) * num_kv_heads + h) * kHeadDim + j;
      val = kIn == 0 ? bf16_bits_to_f32(static_cast<const uint16_t*>(src)[idx]) : static_cast<const float*>(src)[idx];
      val = val - centre;  // key centering (fp32); values use centre = 0
    }
    rows[t][j] = val;
  }
  __syncthreads();

  if (kIn == 2) {
    for (int t = half; t < kAppendTile; t += 2) xpart[0][t][j] = rows[t][j];
  } else {
    // x[t][j] = sum_i rows[t][i] R[i][j]: this thread sums i in [64*half, 64*half + 64)
    const float* R = (tensor == 0 ? r_k : r_v) + (static_cast<size_t>(h) * kHeadDim + 64 * half) * kHeadDim + j;
    float rv[64];
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) rv[ii] = R[ii * kHeadDim];  // all loads in flight at once
    float x[kAppendTile];
#pragma unroll
    for (int t = 0; t < kAppendTile; ++t) x[t] = rot_chains<64>(&rows[t][64 * half], rv);
#pragma unroll
    for (int t = 0; t < kAppendTile; ++t) xpart[half][t][j] = x[t];
    __syncthreads();
    for (int t = half; t < kAppendTile; t += 2) xpart[0][t][j] = xpart[0][t][j] + xpart[1][t][j];
  }
  __syncthreads();

  // Quantize and pack: this half handles tokens 8*half .. 8*half + 7; within it,
  // wave w2 = (tid >> 6) & 1 holds channels 64*w2 .. 64*w2 + 63 (groups 2*w2, 2*w2 + 1).
#pragma unroll
  for (int tt = 0; tt < kAppendTile / 2; ++tt) {
    const int t = 8 * half + tt;
    const int n = n0 + t;
    const int slot = t < nt ? slots[n] : -1;
    if (slot < 0 || slot >= num_pages * kPage) continue;  // uniform over the half; bad slots are skipped
    const float xv = xpart[0][t][j];
    if (rot_out != nullptr) rot_out[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * kHeadDim + j] = xv;

    const int page = slot >> 4;
    uint8_t* block = pool + (static_cast<size_t>(page) * num_kv_heads + h) * kBlockBytes;
    (void)q2_pack_channel(xv, j, tensor, block, slot & 15);
  }
}

hipError_t launch_append(uint8_t* pool, int num_pages, int num_kv_heads, const void* k, const void* v, int in_kind,
                         int n_tokens, const int32_t* slots, const float* mu, const float* r_k, const float* r_v,
                         float* rot_out, hipStream_t stream) {
  const dim3 grid((n_tokens + kAppendTile - 1) / kAppendTile, num_kv_heads, 2);
  const dim3 block(kAppendThreads);
  (void)hipGetLastError();  // report only this call's launch errors, not stale ones
  switch (in_kind) {
    case 0:
      hipLaunchKernelGGL(append_kernel<0>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out);
      break;
    case 1:
      hipLaunchKernelGGL(append_kernel<1>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out);
      break;
    default:
      hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvq
