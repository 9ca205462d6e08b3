// Device-side helpers shared by the kvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_layout.h"

namespace kvq {

// Cache geometry (the only one the kernels implement).
constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kPage = 16;

// Decode split limits and the partial-result row stride (floats).
constexpr int kMaxPagesPerSplit = 2048;
constexpr int kMaxSplits = 512;
// Split partial row: [0,128) unnormalised rotated output, [128] max (log2
// units), [129] sum of weights.
constexpr int kPartStride = 132;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// DPP move inside 16-lane rows (ctrl is a gfx9 DPP control word).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
template <int kLane>
struct QuadBcast { static constexpr int ctrl = kLane | (kLane << 2) | (kLane << 4) | (kLane << 6); };
// quad_perm [1,0,3,2] and [2,3,0,1]: the lane paired by bit 0, by bit 1
struct QuadXor1 { static constexpr int ctrl = 1 | (0 << 2) | (3 << 4) | (2 << 6); };
struct QuadXor2 { static constexpr int ctrl = 2 | (3 << 2) | (0 << 4) | (1 << 6); };

// Sum over the lanes {n, n^4, n^8, n^12} of each 16-lane row (lane bits 2..3).
__device__ __forceinline__ float row_sum_stride4(float x) {
  x += dpp_f32<kDppRowRor8>(x);
  x += dpp_f32<kDppRowRor4>(x);
  return x;
}

// Pair lanes l and l^16 / l^32 with the gfx950 permlane swaps: the two returned
// words are x[l] and x[l ^ 16] (resp. ^32), in some order.
__device__ __forceinline__ void swap16(float x, float& u, float& v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& u, float& v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}
// Max / sum over the four 16-lane rows (lane bits 4..5).
__device__ __forceinline__ float rows_max(float x) {
  float u, v;
  swap16(x, u, v);
  x = fmaxf(u, v);
  swap32(x, u, v);
  return fmaxf(u, v);
}
__device__ __forceinline__ float rows_sum(float x) {
  float u, v;
  swap16(x, u, v);
  x = u + v;
  swap32(x, u, v);
  return u + v;
}
// Max / sum over the whole wave, returned to every lane: within each 16-lane
// row by DPP (quad pairs, then row rotations by 4 and 8), then over the rows.
__device__ __forceinline__ float wave_max_all(float x) {
  x = fmaxf(x, dpp_f32<QuadXor1::ctrl>(x));
  x = fmaxf(x, dpp_f32<QuadXor2::ctrl>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  return rows_max(x);
}
// Max / sum over each 16-lane row (lane bits 0..3), returned to every lane of the row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<QuadXor1::ctrl>(x));
  x = fmaxf(x, dpp_f32<QuadXor2::ctrl>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
  return fmaxf(x, dpp_f32<kDppRowRor8>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<QuadXor1::ctrl>(x);
  x += dpp_f32<QuadXor2::ctrl>(x);
  x += dpp_f32<kDppRowRor4>(x);
  return x + dpp_f32<kDppRowRor8>(x);
}
__device__ __forceinline__ int wave_sum_int(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, QuadXor1::ctrl, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, QuadXor2::ctrl, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowRor4, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowRor8, 0xf, 0xf, false);
  auto r = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  x = static_cast<int>(r[0] + r[1]);
  r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  return static_cast<int>(r[0] + r[1]);
}
__device__ __forceinline__ float wave_sum_all(float x) {
  x += dpp_f32<QuadXor1::ctrl>(x);
  x += dpp_f32<QuadXor2::ctrl>(x);
  x += dpp_f32<kDppRowRor4>(x);
  x += dpp_f32<kDppRowRor8>(x);
  return rows_sum(x);
}

}  // namespace kvq
