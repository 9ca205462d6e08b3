// Rotation and Q2 quantize-pack of one token, shared by the append kernel and
// the fused decode step so that both write identical bytes.
//
// OptR ("Output-Oriented Rotation for INT2 KV-Cache Quantization"), section 3.1,
// Eq. (4): the cache stores Q2(zR).  Q2 here is asymmetric over groups of 32
// consecutive rotated channels: s = fp16(fp32(max - min) / 3), z = fp16(min),
// code = clamp(rint((x - z) / s), 0, 3) computed with the stored fp16 s and z
// (all codes 0 when s is 0); the dequantized level is z + s * code.  With a
// clip ratio c < 1, min and max are first scaled by c (fp32), which narrows
// the range the four levels span; values past it take the end codes.
#pragma once

#include "kvq_device.h"

namespace kvq {

// Rotation summation order.  Every rotated channel x[j] = sum_i a[i] R[i][j]
// is formed as four fma chains over the row ranges [0,32), [32,64), [64,96),
// [96,128) (each started from 0 and taken in row order), added as
// (c0 + c1) + (c2 + c3).  Both kernels follow it, so a token's rotated fp32
// value, and hence its codes, do not depend on which kernel appended it.
template <int kRows>  // 32 or 64 consecutive rows of R held by this thread, starting at row 32*chain0
__device__ __forceinline__ float rot_chains(const float* a, const float* r) {
  static_assert(kRows == 32 || kRows == 64, "one or two chains");
  float c0 = 0.0f;
#pragma unroll
  for (int ii = 0; ii < 32; ++ii) c0 = fmaf(a[ii], r[ii], c0);
  if (kRows == 32) return c0;
  float c1 = 0.0f;
#pragma unroll
  for (int ii = 32; ii < kRows; ++ii) c1 = fmaf(a[ii], r[ii], c1);
  return c0 + c1;
}

// Randomized Hadamard rotation R = diag(s) H / sqrt(128) (H Sylvester's
// Hadamard matrix, H[i][j] = (-1)^popcount(i & j)): x R = WHT(x * s) / sqrt(128)
// and y R^T = s * WHT(y) / sqrt(128).  wht128 is the unnormalised Walsh-Hadamard
// transform of a 128-vector held one element per thread by two whole waves
// (element c = 64 * wave-pair index + lane): stage k = 0..6 turns the pair
// (c, c ^ 2^k) with bit k of c clear into (x_c + x_c', x_c - x_c'); stages 0..5
// shuffle within the wave, stage 6 crosses the two waves through `xch` (128
// floats per vector).  Every thread of the workgroup calls it (it holds two
// barriers); threads without a vector pass xch = nullptr.  One fixed order, so
// the append and the fused decode step round identically.
constexpr float kInvSqrt128 = 0.0883883476483184405f;

__device__ __forceinline__ float wht128(float x, int c, float* xch) {
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const float p = __shfl_xor(x, 1 << k);
    x = (c & (1 << k)) ? p - x : x + p;
  }
  if (xch != nullptr) xch[c] = x;
  __syncthreads();
  const float p = xch != nullptr ? xch[c ^ 64] : 0.0f;
  __syncthreads();  // xch free again
  return (c & 64) ? p - x : x + p;
}

// Range (min, max) of the Q2 group of channel j over the lanes of the calling
// wave, for one token's rotated vector held as in q2_pack_channel: G = 32 is a
// half-wave, G = 64 the whole wave; a G = 128 group spans both waves, whose
// ranges the caller combines (min and max are exact in any order).
__device__ __forceinline__ float2 q2_wave_range(float xv, int gsize) {
  float mn = xv, mx = xv;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (gsize > 32) {
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
  }
  return float2{mn, mx};
}

// Quantizes channel j of one token's rotated vector and packs it into a block.
// Called by the 128 threads j = 0..127 of one (token, KV head, tensor), laid
// out as two whole waves (j = 64 * w2 + lane), with (mn, mx) the unclipped
// range of channel j's group (q2_wave_range).  `block` is the (page, KV head)
// block to write, or null to only compute; `off` is the slot within the page
// (0..15); tensor 0 = K, 1 = V.  The block keeps one metadata pair per group
// of G channels (gsize).  kbits (vbits) = 3 or 4 quantizes the key (value) to
// 8 or 16 levels: its low two bits go where a 2-bit code would, the rest to
// the tensor's plane (kvq_device.h).  Returns the dequantized level of channel j.
//
// K code of slot s, channel c (kk = c/32, a = (c%32)/8, e = c%8): record
// 16a + s, word K[kk/2], bit 2(4(kk%2) + e/2) + 16(e%2).  V code (t = c/16,
// b = c%16, a = s/4, i = s%4): record 16a + b, word V[i/2], bit 2t + 16(i%2).
// Metadata of slot s, group grp (of G channels): record 4grp + s/4 at byte
// 1024 + 32*record, K pair at +4(s%4), V pair at +16 + 4(s%4), each (fp16
// scale, fp16 zero).  A K code word and a metadata pair belong to one slot
// (plain stores); a V code word holds codes of two slots, so it is updated
// with atomic and/or of this slot's bits only, which keeps concurrent writes
// to other slots intact; so is a 3-bit plane word, which holds bits of both
// K words of a record (each wave writes its own alternate bits) or of four
// value slots.
__device__ __forceinline__ float q2_pack_channel(float xv, int j, int tensor, uint8_t* block, int off, float clip,
                                                float mn, float mx, int kbits = 2, int vbits = 2, int gsize = 32) {
  const int bits = tensor == 0 ? kbits : vbits;
  const float n_lv = static_cast<float>((1 << bits) - 1);
  const int lane = j & 63;
  const int w2 = j >> 6;
  mn *= clip;
  mx *= clip;
  // c*min and c*max are rounded to fp32 before anything else uses them (the
  // fp16 zero included): without this the compiler may round c*min straight
  // to fp16 in one mixed-precision multiply, which differs at fp16 ties.
  asm volatile("" : "+v"(mn), "+v"(mx));
  const float s32 = (mx - mn) / n_lv;
  const _Float16 s16 = static_cast<_Float16>(s32);
  const _Float16 z16 = static_cast<_Float16>(mn);
  const float sc = static_cast<float>(s16);
  const float z = static_cast<float>(z16);
  uint32_t code = 0;
  if (sc != 0.0f) {
    const float u = (xv - z) / sc;
    code = static_cast<uint32_t>(fminf(fmaxf(rintf(u), 0.0f), n_lv));
  }

  if (tensor == 0) {
    const int kk = j >> 5, a = (j & 31) >> 3, e = j & 7;
    const int sh = 2 * (4 * (kk & 1) + (e >> 1)) + 16 * (e & 1);
    uint32_t w = (code & 3u) << sh;
    // wide keys: the high bits at the same position (4 bits), or the high bit
    // at the position plus the word index w2 (3 bits)
    uint32_t wh = bits == 4 ? (code >> 2) << sh : (code >> 2) << (sh + w2);
    w |= __shfl_xor(w, 1);
    w |= __shfl_xor(w, 2);
    w |= __shfl_xor(w, 4);
    w |= __shfl_xor(w, 32);
    if (bits > 2) {
      wh |= __shfl_xor(wh, 1);
      wh |= __shfl_xor(wh, 2);
      wh |= __shfl_xor(wh, 4);
      wh |= __shfl_xor(wh, 32);
    }
    if (block != nullptr && (lane & 39) == 0) {  // e == 0, kk even: lanes 0, 8, 16, 24 hold both groups' words
      *reinterpret_cast<uint32_t*>(block + 16 * (16 * a + off) + 4 * w2) = w;
      if (bits == 4) {
        *reinterpret_cast<uint32_t*>(block + k_hi_plane(gsize) + 8 * (16 * a + off) + 4 * w2) = wh;
      } else if (bits == 3) {  // this wave's alternate bits of the record's plane word
        uint32_t* pw = reinterpret_cast<uint32_t*>(block + k_hi_plane(gsize) + 4 * (16 * a + off));
        atomicAnd(pw, ~(0x55555555u << w2));
        atomicOr(pw, wh);
      }
    }
  } else {
    const int t16 = j >> 4, b = j & 15, a = off >> 2, i = off & 3;
    const int shift = 16 * (i & 1);
    uint32_t w = (code & 3u) << (2 * t16 + shift);
    // wide values: the high bits at the same position (4 bits), or the high
    // bit at bit 8 i + t16 of the record's plane word (3 bits)
    uint32_t wh = bits == 4 ? (code >> 2) << (2 * t16 + shift) : (code >> 2) << (8 * i + t16);
    w |= __shfl_xor(w, 16);
    w |= __shfl_xor(w, 32);
    if (bits > 2) {
      wh |= __shfl_xor(wh, 16);
      wh |= __shfl_xor(wh, 32);
    }
    if (block != nullptr && lane < 16) {
      uint32_t* word = reinterpret_cast<uint32_t*>(block + 16 * (16 * a + b) + 8 + 4 * (i >> 1));
      const uint32_t mask = 0xffu << (8 * w2 + shift);  // this wave's four tiles of this slot
      atomicAnd(word, ~mask);
      atomicOr(word, w);
      if (bits == 4) {  // the plane's words are shared by slots as the V words are
        uint32_t* hword =
            reinterpret_cast<uint32_t*>(block + v_hi_plane(kbits, gsize) + 8 * (16 * a + b) + 4 * (i >> 1));
        atomicAnd(hword, ~mask);
        atomicOr(hword, wh);
      } else if (bits == 3) {  // this wave's four tiles of slot i: a nibble of byte i
        uint32_t* hword = reinterpret_cast<uint32_t*>(block + v_hi_plane(kbits, gsize) + 4 * (16 * a + b));
        atomicAnd(hword, ~(0xfu << (8 * i + 4 * w2)));
        atomicOr(hword, wh);
      }
    }
  }
  if (block != nullptr && (j & (gsize - 1)) == 0) {
    const uint32_t pair = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
    const int rec = 4 * (j / gsize) + (off >> 2);
    *reinterpret_cast<uint32_t*>(block + kCodeBytes + kMetaRecordBytes * rec + 16 * tensor + 4 * (off & 3)) = pair;
  }
  return fmaf(sc, static_cast<float>(code), z);
}

// Q2 of the 32 channels [32 g, 32 g + 32) of one token held by one lane (the
// bulk path), lane 4 r + g for token r: the same result as q2_pack_channel's
// arithmetic.  For G = 64 and 128 the range is combined over lanes g ^ 1 and
// g ^ 2 (all lanes of the wave call it).  The code of each element is
// rint(fl(t / s)) clamped to 0..3 with t = fl(x - z); it is taken from
// q = fl(t * fl(1 / s)), which lies within 3 * 2^-24 |q| of fl(t / s), unless
// q is within 2^-19 of a half-integer, where the two could round apart: such a
// lane recomputes its group with the IEEE division.
__device__ __forceinline__ void q2_group32(const float (&x)[32], float clip, int gsize, uint32_t& pair,
                                           uint32_t (&code)[32], float n_lv = 3.0f) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int c = 1; c < 32; ++c) {
    mn = fminf(mn, x[c]);
    mx = fmaxf(mx, x[c]);
  }
  if (gsize > 32) {
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
  }
  if (gsize > 64) {
    mn = fminf(mn, __shfl_xor(mn, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
  }
  mn *= clip;
  mx *= clip;
  // c*min and c*max are rounded to fp32 before anything else uses them (the
  // fp16 zero included): without this the compiler may round c*min straight
  // to fp16 in one mixed-precision multiply, which differs at fp16 ties.
  asm volatile("" : "+v"(mn), "+v"(mx));
  const float s32 = (mx - mn) / n_lv;  // n_lv = 3, or 7 / 15 for 3- / 4-bit codes
  const _Float16 s16 = static_cast<_Float16>(s32);
  const _Float16 z16 = static_cast<_Float16>(mn);
  const float sc = static_cast<float>(s16);
  const float z = static_cast<float>(z16);
  pair = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
  bool near = false;
  const float rcp = sc != 0.0f ? 1.0f / sc : 0.0f;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const float q = (x[c] - z) * rcp;
    const float k = rintf(q);
    near = near || fabsf(q - k) > 0.5f - 0x1p-19f;
    code[c] = static_cast<uint32_t>(__builtin_amdgcn_fmed3f(k, 0.0f, n_lv));
  }
  if (__builtin_amdgcn_ballot_w64(near) != 0 && near) {  // exact path, rarely taken
#pragma unroll
    for (int c = 0; c < 32; ++c)
      code[c] = static_cast<uint32_t>(fminf(fmaxf(rintf((x[c] - z) / sc), 0.0f), n_lv));
  }
}

}  // namespace kvq
