// Rotation x = a R of 32 tokens at a time on the matrix cores, for the bulk
// quantize-append (OptR, section 3.1, Eq. (4): the cache stores Q2(zR)).
//
// The product is taken transposed, x^T = R^T a^T, on v_mfma_f32_32x32x16_f16,
// so that every output lane holds one token: the quantizer then finds each
// token's groups in its own registers.
//
// Precision.  Both operands are split into fp16 pairs, a = a_hi + a_lo and
// R = R_hi + R_lo (each part rounded to nearest).  R (entries at most 1 in
// magnitude) is scaled by 2^10, so that the low parts of its entries stay
// normal down to 2^-13; each token row a is scaled by its own power of two
// 2^k, chosen so that the row's largest magnitude lands in [2^9, 2^10): any
// finite fp32 row then splits without overflow, and the low parts of the
// values that matter stay normal.  Both scalings are exact and are undone on
// the product (products stay below 2^20, sums of 128 below 2^27).  The product
// is R_hi a_hi + R_lo a_hi + R_hi a_lo accumulated in fp32; the dropped
// R_lo a_lo and the rounding of the parts are about 2^-21 of sum |a| |R|, far
// inside the fp32 error bound of a sequential dot product (about 2^-16 of
// that sum for 128 terms).  A bf16 row needs no low part: its 8-bit
// significands scaled by a power of two are exact in fp16, except entries
// below 2^-26 of the row's largest magnitude, which round to fp16's subnormal
// step (an error under 2^-34 of that magnitude); it takes the first two
// products only.
//
// Layouts (32x32x16 f16 MFMA, wave64; lane l = 32 h + n).  The contraction
// index of product ks, lane half h, element e is channel 64 h + 8 ks + e of
// the input row, so that lane (h, n) feeds token n's channels [64 h, 64 h + 64)
// from one contiguous 128-byte (bf16) piece of its row:
//   B operand (tokens), lane (h, n):  a[n][64 h + 8 ks + e], e = 0..7
//   A operand (R^T),    lane (h, m):  R[64 h + 8 ks + e][rot_channel(mt, m)]
//   C, lane (h, n), register 4 j + i of output tile mt (row m = 8 j + 4 h + i):
//     x[n][64 h + 16 mt + 4 j + i]
// so lane (h, n) ends up with channels [64 h, 64 h + 64) of token n, in
// register order 16 mt + 4 j + i.
#pragma once

#include "kvq_device.h"

namespace kvq {

typedef float float16v __attribute__((ext_vector_type(16)));

constexpr float kRotScale = 1024.0f;  // applied to R before the split

// The output channel of row m of output tile mt (m = 8 j + 4 h + i).
__device__ __forceinline__ int rot_channel(int mt, int m) {
  return 64 * ((m >> 2) & 1) + 16 * mt + 4 * (m >> 3) + (m & 3);
}

// The fp16 pair of v * scale (scale a power of two).
__device__ __forceinline__ void split_f16(float v, float scale, _Float16& hi, _Float16& lo) {
  const float s = v * scale;
  hi = static_cast<_Float16>(s);
  lo = static_cast<_Float16>(s - static_cast<float>(hi));
}

// The power of two that brings a row whose largest magnitude is amax into
// [2^9, 2^10) (1 for an all-zero row).
__device__ __forceinline__ float row_split_scale(float amax) {
  int ex = 0;
  frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
  return amax > 0.0f ? ldexpf(1.0f, 10 - ex) : 1.0f;
}

// The fp16 pair (hi, lo) of t * rs, each rounded to nearest once: hi is t rs
// rounded, lo is the exact t rs - hi rounded (one fused multiply-add to fp16).
// The empty asm keeps hi a single value that both the operand and lo use.
__device__ __forceinline__ void split_scaled(float t, float rs, _Float16& hi, _Float16& lo) {
  _Float16 h = static_cast<_Float16>(t * rs);
  asm volatile("" : "+v"(h));
  hi = h;
  lo = static_cast<_Float16>(fmaf(t, rs, -static_cast<float>(h)));
}

// R^T operands in LDS: op[((ks * 4 + mt) * 2 + part) * 64 + lane], part 0 =
// hi, 1 = lo; 64 KB for one 128 x 128 matrix.  Staged by the calling
// workgroup's waves (operand o = ks * 4 + mt taken by wave o % n_waves).
__device__ __forceinline__ void stage_rotation_t(const float* __restrict__ R, half8* op, int wave, int n_waves,
                                                 int lane) {
  const int m = lane & 31, h = lane >> 5;
  for (int o = wave; o < 32; o += n_waves) {
    const int ks = o >> 2, mt = o & 3;
    const float* src = R + (64 * h + 8 * ks) * kHeadDim + rot_channel(mt, m);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[e * kHeadDim];
    half8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 hh, ll;
      split_f16(v[e], kRotScale, hh, ll);
      hi[e] = hh;
      lo[e] = ll;
    }
    op[(o * 2 + 0) * 64 + lane] = hi;
    op[(o * 2 + 1) * 64 + lane] = lo;
  }
}

// x^T = R^T a^T for one 32-token tile: b_hi/b_lo[ks] are the token operands
// (B layout above), acc[mt] receives output tile mt (in units of the row
// scale times 2^10).  Every tile accumulates, for ks = 0..7 in order,
// R_hi a_hi, R_lo a_hi and (kLo) R_hi a_lo; the four tiles are interleaved so
// that consecutive MFMAs never depend on each other.
template <bool kLo>
__device__ __forceinline__ void rotate32(const half8 (&b_hi)[8], const half8 (&b_lo)[8], const half8* op, int lane,
                                         float16v (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    half8 r_hi[4], r_lo[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      r_hi[mt] = op[((ks * 4 + mt) * 2 + 0) * 64 + lane];
      r_lo[mt] = op[((ks * 4 + mt) * 2 + 1) * 64 + lane];
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r_hi[mt], b_hi[ks], acc[mt], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r_lo[mt], b_hi[ks], acc[mt], 0, 0, 0);
    if (kLo) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r_hi[mt], b_lo[ks], acc[mt], 0, 0, 0);
    }
  }
}

}  // namespace kvq
