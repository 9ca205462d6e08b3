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
// [64*half, 64*half + 64) of column j of R for all 16 tokens, with its 64 R
// loads issued up front (column j is read coalesced across threads); the two
// halves are added through LDS.  For quantization, each half takes 8 tokens
// and thread j owns rotated channel j: groups of 32 channels are the two
// 32-lane halves of each wave, so min/max are shuffle reductions in a wave.
//
// Stores: a token's K code words belong to that token alone (plain stores);
// its metadata too.  A V code word holds 8 codes of each of two slots, so V
// words are updated with 32-bit atomic and/or of the token's own bits, which
// keeps concurrent appends to other slots of the same page correct.

#include "kvq_device.h"
#include "kvq_internal.h"

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
    for (int t = 0; t < kAppendTile; ++t) x[t] = 0.0f;
#pragma unroll
    for (int ii = 0; ii < 64; ++ii)
#pragma unroll
      for (int t = 0; t < kAppendTile; ++t) x[t] = fmaf(rows[t][64 * half + ii], rv[ii], x[t]);
#pragma unroll
    for (int t = 0; t < kAppendTile; ++t) xpart[half][t][j] = x[t];
    __syncthreads();
    for (int t = half; t < kAppendTile; t += 2) xpart[0][t][j] = xpart[0][t][j] + xpart[1][t][j];
  }
  __syncthreads();

  // Quantize and pack: this half handles tokens 8*half .. 8*half + 7; within it,
  // wave w2 = (tid >> 6) & 1 holds channels 64*w2 .. 64*w2 + 63 (groups 2*w2, 2*w2 + 1).
  const int lane = tid & 63;
  const int w2 = (tid >> 6) & 1;
  const int grp = j >> 5;
#pragma unroll
  for (int tt = 0; tt < kAppendTile / 2; ++tt) {
    const int t = 8 * half + tt;
    const int n = n0 + t;
    const int slot = t < nt ? slots[n] : -1;
    if (slot < 0 || slot >= num_pages * kPage) continue;  // uniform over the half; bad slots are skipped
    const float xv = xpart[0][t][j];
    if (rot_out != nullptr) rot_out[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * kHeadDim + j] = xv;

    // Q2 on the 32-channel group held by this 32-lane half-wave.
    float mn = xv, mx = xv;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, off));
      mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    const float s32 = (mx - mn) / 3.0f;
    const _Float16 s16 = static_cast<_Float16>(s32);
    const _Float16 z16 = static_cast<_Float16>(mn);
    const float sc = static_cast<float>(s16);
    const float z = static_cast<float>(z16);
    uint32_t code = 0;
    if (sc != 0.0f) {
      const float u = (xv - z) / sc;
      code = static_cast<uint32_t>(fminf(fmaxf(rintf(u), 0.0f), 3.0f));
    }

    const int page = slot >> 4;
    const int off = slot & 15;
    uint8_t* block = pool + (static_cast<size_t>(page) * num_kv_heads + h) * kBlockBytes;

    if (tensor == 0) {
      // K: channel j -> kk = j/32, a = (j%32)/8, e = j%8; record 16a + off,
      // word kk/2 (= w2), bit 2*(4*(kk%2) + e/2) + 16*(e%2).
      const int kk = grp, a = (j & 31) >> 3, e = j & 7;
      uint32_t w = code << (2 * (4 * (kk & 1) + (e >> 1)) + 16 * (e & 1));
      w |= __shfl_xor(w, 1);
      w |= __shfl_xor(w, 2);
      w |= __shfl_xor(w, 4);
      w |= __shfl_xor(w, 32);
      if ((lane & 39) == 0) {  // e == 0 and kk%2 == 0: lanes 0, 8, 16, 24
        *reinterpret_cast<uint32_t*>(block + 16 * (16 * a + off) + 4 * w2) = w;
      }
    } else {
      // V: channel j -> t = j/16, b = j%16; slot -> a = off/4, i = off%4;
      // record 16a + b, word V[i/2], bit 2t + 16*(i%2).
      const int t16 = j >> 4, b = j & 15, a = off >> 2, i = off & 3;
      const int shift = 16 * (i & 1);
      uint32_t w = code << (2 * t16 + shift);
      w |= __shfl_xor(w, 16);
      w |= __shfl_xor(w, 32);
      if (lane < 16) {
        uint32_t* word = reinterpret_cast<uint32_t*>(block + 16 * (16 * a + b) + 8 + 4 * (i >> 1));
        const uint32_t mask = 0xffu << (8 * w2 + shift);  // this wave's four tiles
        atomicAnd(word, ~mask);
        atomicOr(word, w);
      }
    }
    if ((j & 31) == 0) {
      const uint32_t pair = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
      const int rec = 4 * grp + (off >> 2);
      *reinterpret_cast<uint32_t*>(block + kCodeBytes + kMetaRecordBytes * rec + 16 * tensor + 4 * (off & 3)) = pair;
    }
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
