// Rotation x = a R of 16 rows at a time on the matrix cores, for the bulk
// quantize-append (OptR, section 3.1, Eq. (4): the cache stores Q2(zR)).
//
// Precision.  Both operands are split into fp16 pairs, a = a_hi + a_lo and
// R = R_hi + R_lo (each part rounded to nearest).  R (entries at most 1 in
// magnitude) is scaled by 2^10, so that the low parts of its entries stay
// normal down to 2^-13; each row a is scaled by its own power of two 2^k,
// chosen so that the row's largest magnitude lands in [2^9, 2^10): any finite
// fp32 row then splits without overflow, and the low parts of the values that
// matter stay normal.  Both scalings are exact and are undone on the product
// (products stay below 2^20, sums of 128 below 2^27).  The product is
// a_hi R_hi + a_hi R_lo + a_lo R_hi accumulated in fp32 by
// v_mfma_f32_16x16x32_f16; the dropped a_lo R_lo and the rounding of the
// parts are about 2^-21 of sum |a| |R|, far inside the fp32 error bound of a
// sequential dot product (about 2^-16 of that sum for 128 terms).
//
// Layouts (16x16x32 f16 MFMA, wave64).  Output tile nt (columns 16 nt ..
// 16 nt + 15) accumulates over k-blocks kb (rows 32 kb .. 32 kb + 31 of R):
//   A operand, lane (kq = lane / 16, row = lane % 16): a[row][32 kb + 8 kq + e]
//   B operand, lane (kq, n = lane % 16):             R[32 kb + 8 kq + e][16 nt + n]
//   C, lane (a = lane / 16, col = lane % 16):        x[4 a + i][16 nt + col], i = 0..3
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr float kRotScale = 1024.0f;  // applied to R before the split

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

// R operands in LDS: op[((kb * 8 + nt) * 2 + part) * 64 + lane], part 0 = hi,
// 1 = lo; 64 KB for one 128 x 128 matrix.  Staged by the calling workgroup's
// waves (operand o = kb * 8 + nt taken by wave o % n_waves).
__device__ __forceinline__ void stage_rotation(const float* __restrict__ R, half8* op, int wave, int n_waves,
                                               int lane) {
  const int kq = lane >> 4, n = lane & 15;
  for (int o = wave; o < 32; o += n_waves) {
    const int kb = o >> 3, nt = o & 7;
    const float* src = R + (32 * kb + 8 * kq) * kHeadDim + 16 * nt + n;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[e * kHeadDim];
    half8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h, l;
      split_f16(v[e], kRotScale, h, l);
      hi[e] = h;
      lo[e] = l;
    }
    op[(o * 2 + 0) * 64 + lane] = hi;
    op[(o * 2 + 1) * 64 + lane] = lo;
  }
}

// x = a R for the 16 rows held in A-operand layout (a_hi/a_lo[kb] per lane);
// C[nt] receives output tile nt, multiplied by unscale[i] in row 4 (lane/16) + i
// (the inverse of that row's split scale times 2^-10).  Every tile accumulates
// hi*hi, hi*lo, lo*hi for kb = 0, 1, 2, 3 in that order; the tiles are
// interleaved so that consecutive MFMAs never depend on each other.
__device__ __forceinline__ void rotate16(const half8 (&a_hi)[4], const half8 (&a_lo)[4], const half8* op, int lane,
                                         const float (&unscale)[4], float4v (&C)[8]) {
  float4v acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const half8 r_hi = op[((kb * 8 + nt) * 2 + 0) * 64 + lane];
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[kb], r_hi, acc[nt], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const half8 r_lo = op[((kb * 8 + nt) * 2 + 1) * 64 + lane];
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[kb], r_lo, acc[nt], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const half8 r_hi = op[((kb * 8 + nt) * 2 + 0) * 64 + lane];
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[kb], r_hi, acc[nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) C[nt][i] = acc[nt][i] * unscale[i];
}

}  // namespace kvq
