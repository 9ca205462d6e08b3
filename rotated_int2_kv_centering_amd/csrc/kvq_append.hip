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

#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"
#include "kvq_rot.h"

namespace kvq {

constexpr int kAppendTile = 16;
constexpr int kAppendThreads = 256;
// Appends of at least this many raw tokens take the bulk (matrix-core) path.
constexpr int kBulkMin = 64;

template <int kIn>  // 0 = bf16 raw, 1 = fp32 raw, 2 = fp32 already centred and rotated
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    uint8_t* __restrict__ pool, int num_pages, int num_kv_heads, const void* __restrict__ k_in,
    const void* __restrict__ v_in, int n_tokens, const int32_t* __restrict__ slots, const float* __restrict__ mu,
    const float* __restrict__ r_k, const float* __restrict__ r_v, float* __restrict__ rot_out, float clip,
    int rot_kind, int gsize, float* __restrict__ sq_err, int kbits, int vbits) {
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
  } else if (rot_kind == 1) {
    // x = WHT(a * s) / sqrt(128): this half transforms tokens 8*half .. 8*half + 7
    __shared__ float xch[2][kHeadDim];
    const float sg = (tensor == 0 ? r_k : r_v)[h * kHeadDim + j];
#pragma unroll 1
    for (int tt = 0; tt < kAppendTile / 2; ++tt) {
      const int t = (kAppendTile / 2) * half + tt;
      xpart[0][t][j] = wht128(rows[t][j] * sg, j, xch[half]) * kInvSqrt128;
    }
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

  // G = 128: a group spans both waves of a half; each wave's range of each token first
  __shared__ float2 s_rng[kAppendTile][2];
  if (gsize == 128) {
    for (int tt = 0; tt < kAppendTile / 2; ++tt) {
      const int t = (kAppendTile / 2) * half + tt;
      const float2 r = q2_wave_range(xpart[0][t][j], 64);
      if ((j & 63) == 0) s_rng[t][j >> 6] = r;
    }
    __syncthreads();
  }

  // Quantize and pack: this half handles tokens 8*half .. 8*half + 7; within it,
  // wave w2 = (tid >> 6) & 1 holds channels 64*w2 .. 64*w2 + 63 (groups 2*w2, 2*w2 + 1).
#pragma unroll
  for (int tt = 0; tt < kAppendTile / 2; ++tt) {
    const int t = (kAppendTile / 2) * half + tt;
    const int n = n0 + t;
    const int slot = t < nt ? slots[n] : -1;
    if (slot < 0 || slot >= num_pages * kPage) continue;  // uniform over the half; bad slots are skipped
    const float xv = xpart[0][t][j];
    if (rot_out != nullptr) rot_out[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * kHeadDim + j] = xv;

    const int page = slot >> 4;
    uint8_t* block = pool + (static_cast<size_t>(page) * num_kv_heads + h) * block_bytes(kbits, vbits, gsize);
    float2 r;
    if (gsize == 128) {
      const float2 a = s_rng[t][0], b = s_rng[t][1];
      r = float2{fminf(a.x, b.x), fmaxf(a.y, b.y)};
    } else {
      r = q2_wave_range(xv, gsize);
    }
    const float lvl = q2_pack_channel(xv, j, tensor, block, slot & 15, clip, r.x, r.y, kbits, vbits, gsize);
    if (sq_err != nullptr) {  // squared error over this wave's 64 channels
      float e = (xv - lvl) * (xv - lvl);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o);
      if ((j & 63) == 0) sq_err[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * 2 + (j >> 6)] = e;
    }
  }
}

// ---------------------------------------------------------------------------
// Bulk path (n_tokens >= kBulkMin, raw bf16/fp32 input).
//
// Workgroups of 8 waves, each bound to one KV head, with R_K and R_V staged
// once in LDS as split-fp16 MFMA operands (kvq_rot.h; a Hadamard R needs
// none).  A wave takes 32 tokens at a time and runs their keys, then their
// values:
//   1. lane l = 32 h + n loads channels [64 h, 64 h + 64) of token n (one
//      contiguous piece of its row) and centres keys (fp32);
//   2. the wave rotates the 32 rows on the matrix cores (kvq_rot.h), or, for
//      a Hadamard R, runs the seven butterfly stages of wht128 in the same
//      order: stages 0-5 inside the lane, stage 6 across the lane halves.
//      Either way lane (h, n) ends up with channels [64 h, 64 h + 64) of the
//      rotated token n, which are its Q2 groups 2h and 2h + 1 (G = 32);
//   3. the lane quantizes them in registers (bulk_params, bulk_codes) and
//      packs the codes straight into the block's words: a slot's K words are
//      whole in one lane; its V half-words take one exchange across the lane
//      halves, and the two slots of a V word one between neighbouring lanes;
//   4. 2-bit codes: the lanes write the tile's two blocks into the wave's LDS
//      image, which is copied out as whole 16-byte chunks (whole lines) when
//      the tile fills two pages in order, else slot by slot; 3- and 4-bit
//      codes are stored slot by slot.  Slot by slot, a V word whose other slot
//      is not the neighbouring token of the same tile is written as this
//      slot's 16-bit half only.
//   Tiles are dealt to the workgroup's waves from an LDS counter, so a wave
//   that is issued less often takes fewer of them.
// ---------------------------------------------------------------------------
constexpr int kBulkThreads = 512;
constexpr int kBulkWaves = kBulkThreads / 64;
constexpr int kBulkTok = 32;                  // tokens per wave tile
constexpr float kMagic = 12582912.0f;         // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4b400000u;  // its bits: fl(q + kMagic) keeps rint(q) in the low bits
// sum of kMagicBits << p over the sixteen 2-bit fields p = 0, 2, .., 30 of a word
constexpr uint32_t magic_fields() {
  uint32_t s = 0;
  for (int p = 0; p < 32; p += 2) s += kMagicBits << p;
  return s;
}
constexpr uint32_t kMagicFields = magic_fields();

__device__ __forceinline__ uint32_t dpp_xor1_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), QuadXor1::ctrl, 0xf, 0xf, false));
}

// Q2 of one token's channels [64 h, 64 h + 64), held by one lane as c[v]
// (v = channel - 64 h) in units of 1/u (u a power of two: x = c u exactly);
// groups g = 0, 1 are v in [32 g, 32 g + 32).  The arithmetic is that of
// q2_pack_channel (kvq_quant.h): s = fp16(fp32(max - min) / n_lv) and
// z = fp16(min) after the clip, code = clamp(rint(fl(fl(x - z) / s)), 0, n_lv),
// all codes 0 where s is 0.
struct BulkGroups {
  float sc[2], z[2];  // fp16 scale and zero of groups 0, 1 (as fp32)
  float zn[2], top[2], r_lo[2], r_hi[2];
  uint32_t pair[2];  // metadata words: fp16 scale | fp16 zero << 16
};

// d / b rounded to nearest, for b = 3, 7 or 15 and y = 1/b rounded to nearest:
// Markstein's correction q1 = q0 + (d - q0 b) y of q0 = d y, whose residual
// d - q0 b the fused multiply-add forms exactly, is the correctly rounded
// quotient (for d normal or zero; a subnormal d gives a quotient that fp16
// flushes to 0 either way).
__device__ __forceinline__ float div_exact(float d, float b, float y) {
  const float q0 = d * y;
  const float r = fmaf(-q0, b, d);
  return fmaf(r, y, q0);
}

__device__ __forceinline__ BulkGroups bulk_params(const float (&c)[64], float u, float clip, int gsize, float n_lv) {
  const float inv_lv = n_lv == 3.0f ? 1.0f / 3.0f : (n_lv == 7.0f ? 1.0f / 7.0f : 1.0f / 15.0f);
  float mn[2], mx[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    mn[g] = c[32 * g];
    mx[g] = c[32 * g];
#pragma unroll
    for (int v = 32 * g + 1; v < 32 * g + 32; ++v) {
      mn[g] = fminf(mn[g], c[v]);
      mx[g] = fmaxf(mx[g], c[v]);
    }
  }
  if (gsize > 32) {  // G = 64: both groups of the lane
    mn[0] = mn[1] = fminf(mn[0], mn[1]);
    mx[0] = mx[1] = fmaxf(mx[0], mx[1]);
  }
  if (gsize > 64) {  // G = 128: and the other lane half
    float p, q;
    swap32(mn[0], p, q);
    mn[0] = mn[1] = fminf(p, q);
    swap32(mx[0], p, q);
    mx[0] = mx[1] = fmaxf(p, q);
  }
  BulkGroups G;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float lo = mn[g] * u, hi = mx[g] * u;  // exact: u is a power of two
    lo *= clip;
    hi *= clip;
    // c*min and c*max are rounded to fp32 before anything else uses them
    asm volatile("" : "+v"(lo), "+v"(hi));
    const float s32 = div_exact(hi - lo, n_lv, inv_lv);
    const _Float16 s16 = static_cast<_Float16>(s32);
    const _Float16 z16 = static_cast<_Float16>(lo);
    G.sc[g] = static_cast<float>(s16);
    G.z[g] = static_cast<float>(z16);
    G.pair[g] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s16)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, z16)) << 16);
    G.zn[g] = -G.z[g];
    G.top[g] = G.sc[g] * n_lv;  // exact: an 11-bit by 4-bit product
    const float rcp = G.sc[g] != 0.0f ? __builtin_amdgcn_rcpf(G.sc[g]) : 0.0f;
    G.r_lo[g] = rcp * (1.0f - 0x1p-20f);
    G.r_hi[g] = rcp * (1.0f + 0x1p-20f);
  }
  return G;
}

// The codes of the 64 values as y = kMagicBits + code, passed to pack(v, y);
// with kErr, err(v, x, level) also sees each value and its dequantized level.
//
// The fast path (kExact false) divides nothing.  With t = fl(x - z) clamped
// to [0, n_lv s] (n_lv s is exact, and clamping t clamps the code),
// q1 = t r_lo and q2 = t r_hi bracket fl(t / s): r_lo and r_hi are 1/s moved
// 2^-20 down and up, more than the reciprocal's error plus that of the rounded
// quotient.  rint is monotone, so where rint(q1) = rint(q2) that is the code.
// Each rint is taken inside the fused multiply-add that forms q, by adding
// 1.5 * 2^23: the sum keeps the integer in its low bits.  The return value is
// nonzero where some q1 and q2 round apart (fl(t / s) within about 2^-20 of a
// half-integer, ties included); the caller then takes this lane's codes again
// with kExact, the IEEE division.
template <bool kExact, bool kErr, typename Pack, typename Err>
__device__ __forceinline__ uint32_t bulk_codes(const float (&c)[64], float u, float n_lv, const BulkGroups& G,
                                               Pack&& pack, Err&& err) {
  uint32_t apart = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const int g = v >> 5;
    const float t = fmaf(c[v], u, G.zn[g]);
    uint32_t y;
    if (kExact) {
      const float q = G.sc[g] != 0.0f ? fminf(fmaxf(rintf(t / G.sc[g]), 0.0f), n_lv) : 0.0f;
      y = kMagicBits + static_cast<uint32_t>(q);
    } else {
      const float tc = __builtin_amdgcn_fmed3f(t, 0.0f, G.top[g]);
      const float y1 = fmaf(tc, G.r_lo[g], kMagic);
      const float y2 = fmaf(tc, G.r_hi[g], kMagic);
      apart += __float_as_uint(y1) ^ __float_as_uint(y2);
      y = __float_as_uint(y1);
    }
    pack(v, y);
    if (kErr) err(v, c[v] * u, fmaf(G.sc[g], static_cast<float>(y - kMagicBits), G.z[g]));
  }
  return apart;
}

// K code word a (record 16 a + slot, word h) gets value v = 16 mt + 4 j + i of
// the lane when a = 2 (mt & 1) + j / 2, at bit 2 (4 (mt / 2) + 2 (j & 1) +
// i / 2) + 16 (i & 1): channel 64 h + v is c = 32 kk + 8 a + e with kk = 2 h +
// mt / 2 and e = 4 (j & 1) + i (kvq_quant.h).  The lane's byte h of V
// half-word b = 4 j + i (t = c / 16 = 4 h + mt) is byte i of word j, at bit
// 8 i + 2 mt.
__device__ __forceinline__ int kword_of(int v) { return 2 * ((v >> 4) & 1) + ((v >> 3) & 1); }
__device__ __forceinline__ int kbit_of(int v) {
  return 2 * (4 * (v >> 5) + 2 * ((v >> 2) & 1) + ((v & 3) >> 1)) + 16 * (v & 1);
}
__device__ __forceinline__ int vword_of(int v) { return (v >> 2) & 3; }
__device__ __forceinline__ int vbit_of(int v) { return 8 * (v & 3) + 2 * (v >> 4); }

// The 16-bit V half-words of this lane's token for b = 8 h + 2 q, 8 h + 2 q + 1
// (word q, low and high half) from the byte words D[j] of both lane halves:
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes
// 0..31 of its second, so each lane receives, in this order, the h = 0 and the
// h = 1 byte words of the j it keeps (lower half: j = 0, 1; upper: 2, 3).
__device__ __forceinline__ void v_halfwords(const uint32_t (&D)[4], uint32_t (&E)[4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const auto r = __builtin_amdgcn_permlane32_swap(D[p], D[p + 2], false, false);
    E[2 * p] = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);      // bytes P0 Q0 P1 Q1
    E[2 * p + 1] = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // bytes P2 Q2 P3 Q3
  }
}

// The V words of the slot pair of this lane's token and its neighbour in the
// tile (lane ^ 1): the even token of the pair assembles b = 8 h .. 8 h + 3,
// the odd one b = 8 h + 4 .. 8 h + 7 (W[q] for b0 + q), each word holding the
// even slot's half-word low; `odd_slot` tells which of the two slots is this
// lane's.  Every lane takes part (a DPP exchange).
__device__ __forceinline__ int v_pair(const uint32_t (&E)[4], bool tok_odd, bool odd_slot, int h, uint32_t (&W)[4]) {
  const uint32_t send0 = tok_odd ? E[0] : E[2], send1 = tok_odd ? E[1] : E[3];
  const uint32_t own0 = tok_odd ? E[2] : E[0], own1 = tok_odd ? E[3] : E[1];
  const uint32_t recv0 = dpp_xor1_u32(send0), recv1 = dpp_xor1_u32(send1);
  const uint32_t s_lo = odd_slot ? 0x01000504u : 0x05040100u;
  const uint32_t s_hi = odd_slot ? 0x03020706u : 0x07060302u;
  W[0] = __builtin_amdgcn_perm(recv0, own0, s_lo);
  W[1] = __builtin_amdgcn_perm(recv0, own0, s_hi);
  W[2] = __builtin_amdgcn_perm(recv1, own1, s_lo);
  W[3] = __builtin_amdgcn_perm(recv1, own1, s_hi);
  return 8 * h + (tok_odd ? 4 : 0);
}

// Stores the V half-words E of this lane's token (slot `slot`; pslot that of
// the neighbouring token) into the block's plane at byte offset `plane`,
// record stride `rec_stride`: the assembled words where the neighbour holds
// the other slot of each word, else this slot's 16-bit halves only.
__device__ __forceinline__ void v_store(uint8_t* block, bool ok, int slot, int pslot, bool tok_odd, int h,
                                        const uint32_t (&E)[4], int plane, int rec_stride) {
  uint32_t W[4];
  const int b0 = v_pair(E, tok_odd, (slot & 1) != 0, h, W);
  if (!ok) return;
  const int off = slot & 15;
  uint8_t* base = block + plane + rec_stride * 16 * (off >> 2) + 4 * ((off & 3) >> 1);
  if (pslot == (slot ^ 1)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(base + rec_stride * (b0 + q)) = W[q];
  } else {
    uint8_t* half = base + 2 * (off & 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint16_t*>(half + rec_stride * (8 * h + 2 * q)) = static_cast<uint16_t>(E[q] & 0xffffu);
      *reinterpret_cast<uint16_t*>(half + rec_stride * (8 * h + 2 * q + 1)) = static_cast<uint16_t>(E[q] >> 16);
    }
  }
}

// Quantize-pack-store one tensor of a 32-token tile from the lane's 64 values
// c (in units of 1/u).  kT = 0: keys, 1: values; `slot` is the lane's token's
// slot (-1 past the end).  kImg (2-bit keys and values): the words go to the
// wave's LDS image `img` of two blocks, token n of the tile at slot n % 16 of
// image block n / 16, for the caller to copy out; otherwise they are stored
// slot by slot into the pool.
template <int kT, int kBits, bool kImg>
__device__ __forceinline__ void bulk_store(const float (&c)[64], float u, uint8_t* __restrict__ pool, int num_pages,
                                           int num_kv_heads, int hd, int n, int slot, float* __restrict__ rot_out,
                                           float clip, int gsize, float* __restrict__ sq_err, int kbits, int vbits,
                                           int lane, uint8_t* img) {
  constexpr bool kWide = kBits > 2;
  const int h = lane >> 5;
  const float n_lv = static_cast<float>((1 << kBits) - 1);
  const BulkGroups G = bulk_params(c, u, clip, gsize, n_lv);
  // words: K code words a = 0..3 (kWide: + their high bits), or V byte words j = 0..3
  uint32_t w[4], wh[4];
  float e_sum = 0.0f;
  auto reset = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = kWide ? 0u : 0u - kMagicFields;  // 2-bit: the magic's bits cancel once all 16 fields are in
      wh[q] = 0u;
    }
    e_sum = 0.0f;
  };
  constexpr int bits = kBits;
  auto pack = [&](int v, uint32_t y) {
    const int q = kT == 0 ? kword_of(v) : vword_of(v);
    const int b = kT == 0 ? kbit_of(v) : vbit_of(v);
    if (kWide) {
      w[q] |= (y & 3u) << b;
      if (bits == 4)  // the high bits at the low bits' position
        wh[q] |= ((y >> 2) & 3u) << b;
      else  // 3 bits: keys at the position plus the word index h; values: bit 8 (b % 4) + tile of byte b % 4
        wh[q] |= ((y >> 2) & 1u) << (kT == 0 ? b + h : 8 * (v & 3) + 4 * h + (v >> 4));
    } else {
      w[q] += y << b;
    }
  };
  auto err = [&](int, float x, float lvl) {
    const float d = x - lvl;
    e_sum = fmaf(d, d, e_sum);
  };
  auto run = [&](auto exact_tag) {
    constexpr bool kExact = decltype(exact_tag)::value;
    return sq_err != nullptr ? bulk_codes<kExact, true>(c, u, n_lv, G, pack, err)
                             : bulk_codes<kExact, false>(c, u, n_lv, G, pack, err);
  };
  reset();
  if (run(std::false_type{}) != 0) {  // this lane: recompute with the division
    reset();
    run(std::true_type{});
  }

  const bool tok_odd = (lane & 1) != 0;
  const bool ok = slot >= 0 && slot < num_pages * kPage;
  const int shift = meta_shift(gsize);
  uint32_t E[4], EH[4];
  if (kT == 1) {
    v_halfwords(w, E);
    if (kWide && bits == 4) v_halfwords(wh, EH);
  }
  if (kWide && bits == 3) {  // 3-bit planes: both lane halves' bits of each word
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float p0, p1;
      swap32(__uint_as_float(wh[q]), p0, p1);
      wh[q] = __float_as_uint(p0) | __float_as_uint(p1);
    }
  }
  if (kImg) {
    uint8_t* ib = img + kBlockBytes * ((lane & 31) >> 4);
    const int io = lane & 15;  // the token's slot in the image
    if (kT == 0) {
#pragma unroll
      for (int a = 0; a < 4; ++a) *reinterpret_cast<uint32_t*>(ib + 16 * (16 * a + io) + 4 * h) = w[a];
    } else {
      uint32_t W[4];
      const int b0 = v_pair(E, tok_odd, tok_odd, h, W);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint32_t*>(ib + 8 + 16 * (16 * (io >> 2) + b0 + q) + 4 * ((io & 3) >> 1)) = W[q];
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)  // 32-channel group 2 h + g: a pair where a group of G channels starts
      if (((2 * h + g) & ((1 << shift) - 1)) == 0)
        *reinterpret_cast<uint32_t*>(ib + kCodeBytes + kMetaRecordBytes * (4 * ((2 * h + g) >> shift) + (io >> 2)) +
                                     16 * kT + 4 * (io & 3)) = G.pair[g];
    if (!ok) return;
  } else {
    const int pslot = static_cast<int>(dpp_xor1_u32(static_cast<uint32_t>(slot)));
    uint8_t* block =
        pool + (static_cast<size_t>(ok ? slot >> 4 : 0) * num_kv_heads + hd) * block_bytes(kbits, vbits, gsize);
    const int off = slot & 15;
    if (kT == 1) {
      v_store(block, ok, slot, pslot, tok_odd, h, E, 8, 16);
      if (kWide && bits == 4) v_store(block, ok, slot, pslot, tok_odd, h, EH, v_hi_plane(kbits, gsize), 8);
    }
    if (!ok) return;
    if (kT == 0) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        *reinterpret_cast<uint32_t*>(block + 16 * (16 * a + off) + 4 * h) = w[a];
        if (kWide && bits == 4) *reinterpret_cast<uint32_t*>(block + k_hi_plane(gsize) + 8 * (16 * a + off) + 4 * h) = wh[a];
      }
      if (kWide && bits == 3) {  // the record's plane word (both K words' bits), records 2h, 2h + 1 by this lane
#pragma unroll
        for (int a = 2 * h; a < 2 * h + 2; ++a)
          *reinterpret_cast<uint32_t*>(block + k_hi_plane(gsize) + 4 * (16 * a + off)) = wh[a];
      }
    } else if (kWide && bits == 3) {  // byte off % 4 of plane record 16 (off / 4) + b, b = 8h .. 8h + 7 by this lane
#pragma unroll
      for (int b = 8 * h; b < 8 * h + 8; ++b)
        block[v_hi_plane(kbits, gsize) + 4 * (16 * (off >> 2) + b) + (off & 3)] =
            static_cast<uint8_t>(wh[b >> 2] >> (8 * (b & 3)));
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)  // 32-channel group 2 h + g: a pair where a group of G channels starts
      if (((2 * h + g) & ((1 << shift) - 1)) == 0)
        *reinterpret_cast<uint32_t*>(block + kCodeBytes + kMetaRecordBytes * (4 * ((2 * h + g) >> shift) + (off >> 2)) +
                                     16 * kT + 4 * (off & 3)) = G.pair[g];
  }
  const size_t row = (static_cast<size_t>(n) * num_kv_heads + hd) * 2 + kT;
  if (sq_err != nullptr) sq_err[row * 2 + h] = e_sum;  // channels [64 h, 64 h + 64)
  if (rot_out != nullptr) {
    float* dst = rot_out + row * kHeadDim + 64 * h;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      *reinterpret_cast<float4v*>(dst + 4 * q) =
          float4v{c[4 * q] * u, c[4 * q + 1] * u, c[4 * q + 2] * u, c[4 * q + 3] * u};
  }
}

typedef uint16_t uint16_v2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16_v2 __attribute__((ext_vector_type(2)));

// One bf16 element of a packed pair (hi selects the upper one) times a power
// of two given as bf16 bits, by the bf16 dot product with (s, 0) or (0, s)
// plus 0: the product is exact while it stays a normal fp32, so the dot
// product's own rounding never acts (its addition is not IEEE-rounded, which
// is why the key centering is a plain fp32 subtraction instead).
__device__ __forceinline__ float bf16_pick_scale(uint32_t pair, bool hi, uint32_t scale_bits) {
  const bf16_v2 sel = __builtin_bit_cast(bf16_v2, hi ? scale_bits << 16 : scale_bits);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16_v2, pair), sel, 0.0f, false);
}

template <int kIn>
struct BulkRaw {
  uint4v w[kIn == 0 ? 8 : 16];  // channels [64 h, 64 h + 64) of the lane's token: bf16 or fp32
};

template <int kIn>
__device__ __forceinline__ void bulk_load(BulkRaw<kIn>& r, const void* __restrict__ src, int n, int n_tokens,
                                          int num_kv_heads, int hd, int h) {
  const size_t base = (static_cast<size_t>(min(n, n_tokens - 1)) * num_kv_heads + hd) * kHeadDim + 64 * h;
#pragma unroll
  for (int q = 0; q < (kIn == 0 ? 8 : 16); ++q)
    r.w[q] = kIn == 0 ? *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(src) + base + 8 * q)
                      : *reinterpret_cast<const uint4v*>(static_cast<const float*>(src) + base + 4 * q);
}

// Rotates (and quantizes, packs, stores) one tensor of the lane's token;
// next() issues the loads of the next tensor once the rotation is done (the
// point of fewest live registers that still leaves the quantizer's work to
// cover their latency).
template <int kIn, int kRot, int kT, bool kImg, typename Next>
__device__ __forceinline__ void bulk_tensor(const BulkRaw<kIn>& raw, const half8* op, const float* centre,
                                            const float* sgn, uint8_t* __restrict__ pool, int num_pages,
                                            int num_kv_heads, int hd, int n, int slot, float* __restrict__ rot_out,
                                            float clip, int gsize, float* __restrict__ sq_err, int kbits, int vbits,
                                            int lane, uint8_t* img, Next&& next) {
  const int h = lane >> 5;
  // bf16 values scale exactly into fp16: they need no low part (kvq_rot.h)
  constexpr bool kBf16Values = kIn == 0 && kT == 1 && kRot == 0;
  float a[64];  // channel 64 h + v of the token, centred for keys (unused for bf16 values)
  if (!kBf16Values) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float4v m4 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kT == 0) m4 = *reinterpret_cast<const float4v*>(centre + 64 * h + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * q + e;
        const uint32_t word = kIn == 0 ? raw.w[v >> 3][(v & 7) >> 1] : raw.w[q][e];
        const float x = kIn == 0 ? __uint_as_float((v & 1) ? (word & 0xffff0000u) : (word << 16)) : __uint_as_float(word);
        a[v] = x - m4[e];  // key centering (fp32); values use centre 0
      }
    }
  }
  float c[64];
  float u = 1.0f;
  if (kRot == 0) {
    float amax;
    if (kBf16Values) {  // the largest magnitude from the bf16 bits (sign cleared, compared as integers)
      uint16_v2 m2 = {0, 0};
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(uint16_v2, raw.w[q][i] & 0x7fff7fffu));
      amax = __uint_as_float(static_cast<uint32_t>(m2[0] > m2[1] ? m2[0] : m2[1]) << 16);
    } else {
      amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 64; ++v) amax = fmaxf(amax, fabsf(a[v]));
    }
    float p, q;
    swap32(amax, p, q);
    const float rs = row_split_scale(fmaxf(p, q));
    u = 1.0f / (rs * kRotScale);  // a power of two: exact
    constexpr bool kLo = !kBf16Values;
    half8 b_hi[8], b_lo[8];
    if (kBf16Values) {
      // rs as a bf16 in either half: the dot product with it scales one element exactly
      const uint32_t rs_bits = __float_as_uint(rs) >> 16;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          b_hi[ks][e] = static_cast<_Float16>(bf16_pick_scale(raw.w[ks][e >> 1], (e & 1) != 0, rs_bits));
          b_lo[ks][e] = 0;
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          _Float16 hh, ll;
          split_scaled(a[8 * ks + e], rs, hh, ll);
          b_hi[ks][e] = hh;
          b_lo[ks][e] = ll;
        }
    }
    float16v acc[4];
    rotate32<kLo>(b_hi, b_lo, op, lane, acc);
#pragma unroll
    for (int v = 0; v < 64; ++v) c[v] = acc[v >> 4][v & 15];
  } else {
    // x = WHT(a * s) / sqrt(128), the stages of wht128 in its order
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float4v s4 = *reinterpret_cast<const float4v*>(sgn + 64 * h + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[4 * q + e] = a[4 * q + e] * s4[e];
    }
#pragma unroll
    for (int k = 0; k < 6; ++k)  // channel bits 0-5: inside the lane
#pragma unroll
      for (int v = 0; v < 64; ++v)
        if ((v & (1 << k)) == 0) {
          const float lo = c[v], hi = c[v | (1 << k)];
          c[v] = lo + hi;
          c[v | (1 << k)] = lo - hi;
        }
    const float sg = h ? -1.0f : 1.0f;  // channel bit 6: the lane halves
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      float lo, hi;  // the h = 0 and the h = 1 element of the pair
      swap32(c[v], lo, hi);
      c[v] = fmaf(hi, sg, lo) * kInvSqrt128;
    }
  }
  next();
  const int bits = kT == 0 ? kbits : vbits;
  if (!kImg && bits == 4)
    bulk_store<kT, 4, false>(c, u, pool, num_pages, num_kv_heads, hd, n, slot, rot_out, clip, gsize, sq_err, kbits,
                             vbits, lane, img);
  else if (!kImg && bits == 3)
    bulk_store<kT, 3, false>(c, u, pool, num_pages, num_kv_heads, hd, n, slot, rot_out, clip, gsize, sq_err, kbits,
                             vbits, lane, img);
  else
    bulk_store<kT, 2, kImg>(c, u, pool, num_pages, num_kv_heads, hd, n, slot, rot_out, clip, gsize, sq_err, kbits,
                            vbits, lane, img);
}

// kNarrow: 2-bit keys and values (the tile goes through the wave's LDS
// image); otherwise 3- or 4-bit codes in either tensor, stored slot by slot.
template <int kIn, int kRot, bool kNarrow>  // kIn: 0 = bf16, 1 = fp32; kRot: 0 = dense R, 1 = Hadamard signs
__global__ __launch_bounds__(kBulkThreads) void append_bulk_kernel(
    uint8_t* __restrict__ pool, int num_pages, int num_kv_heads, const void* __restrict__ k_in,
    const void* __restrict__ v_in, int n_tokens, const int32_t* __restrict__ slots, const float* __restrict__ mu,
    const float* __restrict__ r_k, const float* __restrict__ r_v, float* __restrict__ rot_out, float clip, int gsize,
    float* __restrict__ sq_err, int kbits, int vbits) {
  const int hd = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  constexpr int kOps = 32 * 2 * 64;  // half8 operands of one R
  __shared__ half8 s_op[kRot == 0 ? 2 * kOps : 1];  // R_K then R_V, 128 KB (dense R only)
  __shared__ float s_vec[3][kHeadDim];              // key centre; Hadamard signs of K and V
  constexpr int kImgChunks = kNarrow ? 2 * kBlockBytes / 16 : 1;
  __shared__ uint4v s_img[kBulkWaves][kImgChunks];  // each wave's image of two 2-bit blocks
  __shared__ int s_next;                            // the workgroup's next unclaimed tile index j
  if (tid == 0) s_next = kBulkWaves;

  if (kRot == 0) {
    stage_rotation_t(r_k + static_cast<size_t>(hd) * kHeadDim * kHeadDim, s_op, wave, kBulkWaves, lane);
    stage_rotation_t(r_v + static_cast<size_t>(hd) * kHeadDim * kHeadDim, s_op + kOps, wave, kBulkWaves, lane);
  }
  for (int i = tid; i < 3 * kHeadDim; i += kBulkThreads) {
    const int which = i / kHeadDim, j = i % kHeadDim;
    float val = 0.0f;
    if (which == 0)
      val = mu != nullptr ? mu[hd * kHeadDim + j] : 0.0f;
    else if (kRot == 1)
      val = (which == 1 ? r_k : r_v)[hd * kHeadDim + j];
    s_vec[which][j] = val;
  }
  __syncthreads();

  const int n_tiles = (n_tokens + kBulkTok - 1) / kBulkTok;
  const int stride = gridDim.x * kBulkWaves;
  // The workgroup's tiles are blockIdx.x * 8 + (j % 8) + stride * (j / 8),
  // j = 0, 1, ..; its waves start with j = wave and then claim the next j
  // from an LDS counter, so a wave that issues less often takes fewer tiles.
  auto tile_of = [&](int j) { return blockIdx.x * kBulkWaves + j % kBulkWaves + stride * (j / kBulkWaves); };
  int tile = tile_of(wave);
  if (tile >= n_tiles) return;  // no barrier follows
  const int nl = lane & 31;
  uint8_t* img = reinterpret_cast<uint8_t*>(&s_img[wave][0]);
  // bf16 rows are loaded one tensor ahead (32 registers); fp32 rows, twice
  // the registers, where they are used.  A tile's slots come with its key
  // rows, so that no wait for them also waits for stores issued later.
  constexpr bool kAhead = kIn == 0;
  BulkRaw<kIn> rk, rv;
  int slot = 0;
  auto load_keys = [&](int t) {
    const int n = kBulkTok * t + nl;
    slot = n < n_tokens ? slots[n] : -1;
    bulk_load<kIn>(rk, k_in, n, n_tokens, num_kv_heads, hd, h);
  };
  if (kAhead) load_keys(tile);
  // The tile's image is copied out at the top of the next tile (and after the
  // last), once that tile's rows have arrived: the copy-out's stores then
  // come after the wait for those loads, and no later wait for loads finds
  // them still in flight.
  auto copy_out = [&](int sl) {
    // the image was written by this wave only: order those LDS writes before
    // the reads that copy it out
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Whole pages: the tile's 32 tokens fill two distinct pages in order
    // (token n at slot 16 page + n % 16); each block is then stored as whole
    // lines, 16 B per lane (chunks 0..63, then 64..95).
    const int s0 = __builtin_amdgcn_readlane(sl, 0), s16 = __builtin_amdgcn_readlane(sl, 16);
    const int page = nl < 16 ? (s0 >> 4) : (s16 >> 4);
    const bool mine = sl >= 0 && sl < num_pages * kPage && sl == kPage * page + (nl & 15);
    if ((s0 >> 4) != (s16 >> 4) && __ballot(mine) == ~0ull) {
      constexpr int kImgBlk = kBlockBytes / 16;  // image chunks per block (96)
      const int nb = block_bytes(2, 2, gsize);   // 1536, 1280 or 1152 bytes stored
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint4v* dst = reinterpret_cast<uint4v*>(pool + (static_cast<size_t>((b ? s16 : s0) >> 4) * num_kv_heads + hd) * nb);
        dst[lane] = s_img[wave][b * kImgBlk + lane];
        if (lane < nb / 16 - 64) dst[64 + lane] = s_img[wave][b * kImgBlk + 64 + lane];
      }
    } else if (sl >= 0 && sl < num_pages * kPage) {
      // Otherwise each token's own bytes go to its slot: lane (h, n) copies
      // K records 2h, 2h + 1, V half-words b = 8h .. 8h + 7 and the metadata
      // of groups 2h, 2h + 1 (16-bit V stores keep the other slot of a word).
      // (addresses formed here from an opaque lane index: hoisted out of the
      // tile loop they would only take registers from the common path)
      int lid = lane;
      asm volatile("" : "+v"(lid));
      const int hh = lid >> 5, ln = lid & 31;
      const uint8_t* ib = img + kBlockBytes * (ln >> 4);
      const int io = ln & 15, off = sl & 15;
      uint8_t* blk = pool + (static_cast<size_t>(sl >> 4) * num_kv_heads + hd) * block_bytes(2, 2, gsize);
      const int shift = meta_shift(gsize);
#pragma unroll
      for (int a = 2 * hh; a < 2 * hh + 2; ++a)
        *reinterpret_cast<uint2*>(blk + 16 * (16 * a + off)) = *reinterpret_cast<const uint2*>(ib + 16 * (16 * a + io));
#pragma unroll
      for (int b = 8 * hh; b < 8 * hh + 8; ++b)
        *reinterpret_cast<uint16_t*>(blk + 16 * (16 * (off >> 2) + b) + 8 + 4 * ((off & 3) >> 1) + 2 * (off & 1)) =
            *reinterpret_cast<const uint16_t*>(ib + 16 * (16 * (io >> 2) + b) + 8 + 4 * ((io & 3) >> 1) +
                                               2 * (io & 1));
#pragma unroll
      for (int g = 2 * hh; g < 2 * hh + 2; ++g)  // the pairs of the groups of G channels starting at 32 g
        if ((g & ((1 << shift) - 1)) == 0)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            *reinterpret_cast<uint32_t*>(blk + kCodeBytes + kMetaRecordBytes * (4 * (g >> shift) + (off >> 2)) +
                                         16 * t + 4 * (off & 3)) =
                *reinterpret_cast<const uint32_t*>(ib + kCodeBytes + kMetaRecordBytes * (4 * (g >> shift) + (io >> 2)) +
                                                   16 * t + 4 * (io & 3));
    }
    // the next tile's image writes come after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int prev_slot = -1;
  bool have_prev = false;
  for (;;) {
    const int n = kBulkTok * tile + nl;
    if (!kAhead) load_keys(tile);
    const int cur_slot = slot;
    // this tile's rows and slots are here (s_waitcnt vmcnt(0), every other
    // counter left alone) before the previous tile's stores are issued
    if (kNarrow) __builtin_amdgcn_s_waitcnt(0x0f70);
    if (kNarrow && have_prev) copy_out(prev_slot);
    int next_tile = n_tiles;
    bulk_tensor<kIn, kRot, 0, kNarrow>(rk, s_op, s_vec[0], s_vec[1], pool, num_pages, num_kv_heads, hd, n, cur_slot,
                                       rot_out, clip, gsize, sq_err, kbits, vbits, lane, img, [&]() {
                                         if (kAhead) bulk_load<kIn>(rv, v_in, n, n_tokens, num_kv_heads, hd, h);
                                       });
    if (!kAhead) bulk_load<kIn>(rv, v_in, n, n_tokens, num_kv_heads, hd, h);
    bulk_tensor<kIn, kRot, 1, kNarrow>(rv, s_op + kOps, s_vec[0], s_vec[2], pool, num_pages, num_kv_heads, hd, n,
                                       cur_slot, rot_out, clip, gsize, sq_err, kbits, vbits, lane, img, [&]() {
                                         int j = 0;
                                         if (lane == 0) j = atomicAdd(&s_next, 1);
                                         next_tile = tile_of(__builtin_amdgcn_readfirstlane(j));
                                         if (kAhead && next_tile < n_tiles) load_keys(next_tile);
                                       });
    prev_slot = cur_slot;
    have_prev = true;
    if (next_tile >= n_tiles) break;
    tile = next_tile;
  }
  if (kNarrow) copy_out(prev_slot);
}

hipError_t launch_append(uint8_t* pool, int num_pages, int num_kv_heads, const void* k, const void* v, int in_kind,
                         int n_tokens, const int32_t* slots, const float* mu, const float* r_k, const float* r_v,
                         float* rot_out, float clip, int rot_kind, int gsize, float* sq_err, int kbits, int vbits,
                         hipStream_t stream) {
  (void)hipGetLastError();  // report only this call's launch errors, not stale ones
  if (in_kind != 2 && n_tokens >= kBulkMin) {
    // about one workgroup per compute unit in all (each stages R_K and R_V of its
    // head once, 128 KB of LDS: one 8-wave workgroup fills a compute unit), and
    // no more workgroups per head than it has 32-token tiles for their waves
    const int n_tiles = (n_tokens + kBulkTok - 1) / kBulkTok;
    const int per = std::max(1, std::min((n_tiles + kBulkWaves - 1) / kBulkWaves,
                                         (256 + num_kv_heads - 1) / num_kv_heads));
    const dim3 bgrid(per, num_kv_heads);
    const bool narrow = kbits == 2 && vbits == 2;
    auto kern = narrow ? (in_kind == 0 ? (rot_kind == 0 ? append_bulk_kernel<0, 0, true> : append_bulk_kernel<0, 1, true>)
                                       : (rot_kind == 0 ? append_bulk_kernel<1, 0, true> : append_bulk_kernel<1, 1, true>))
                       : (in_kind == 0 ? (rot_kind == 0 ? append_bulk_kernel<0, 0, false> : append_bulk_kernel<0, 1, false>)
                                       : (rot_kind == 0 ? append_bulk_kernel<1, 0, false> : append_bulk_kernel<1, 1, false>));
    hipLaunchKernelGGL(kern, bgrid, dim3(kBulkThreads), 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens, slots,
                       mu, r_k, r_v, rot_out, clip, gsize, sq_err, kbits, vbits);
    return hipGetLastError();
  }
  const dim3 grid((n_tokens + kAppendTile - 1) / kAppendTile, num_kv_heads, 2);
  const dim3 block(kAppendThreads);
  switch (in_kind) {
    case 0:
      hipLaunchKernelGGL(append_kernel<0>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out, clip, rot_kind, gsize, sq_err, kbits, vbits);
      break;
    case 1:
      hipLaunchKernelGGL(append_kernel<1>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out, clip, rot_kind, gsize, sq_err, kbits, vbits);
      break;
    default:
      hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, pool, num_pages, num_kv_heads, k, v, n_tokens,
                         slots, mu, r_k, r_v, rot_out, clip, rot_kind, gsize, sq_err, kbits, vbits);
      break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ exact window
// The BF16 window kept next to the INT2 history (OptR section 3.1): one
// workgroup per token copies its key and value rows of every KV head into the
// window slot of its position, when that position is a window position of its
// sequence (t < sinks, or T - recent <= t < T).  16 bytes (8 bf16) per thread
// and step; fp32 input is rounded to bf16, nearest even.
constexpr int kFillThreads = 128;

__global__ __launch_bounds__(kFillThreads) void window_fill_kernel(uint16_t* __restrict__ buf, int batch, int H,
                                                                   int sinks, int recent, const void* __restrict__ k,
                                                                   const void* __restrict__ v, int in_kind,
                                                                   const int32_t* __restrict__ seq_ids,
                                                                   const int32_t* __restrict__ positions,
                                                                   const int32_t* __restrict__ seq_lens) {
  const int n = blockIdx.x;
  const int b = seq_ids[n];
  const int t = positions[n];
  if (b < 0 || b >= batch || t < 0) return;
  const int T = seq_lens[b];
  if (t >= T || (t >= sinks && t < T - recent)) return;  // not a window position
  const int slot = t < sinks ? t : sinks + t % recent;   // recent > 0 here
  const int n_slots = sinks + recent;
  for (int e = threadIdx.x; e < H * 2 * 16; e += kFillThreads) {
    const int h = e >> 5, kv = (e >> 4) & 1, j = e & 15;
    const size_t src = (static_cast<size_t>(n) * H + h) * kHeadDim + 8 * j;
    uint4v w;
    if (in_kind == 0) {
      w = *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(kv ? v : k) + src);
    } else {
      const float* f = static_cast<const float*>(kv ? v : k) + src;
      const float4v lo = *reinterpret_cast<const float4v*>(f);
      const float4v hi = *reinterpret_cast<const float4v*>(f + 4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        w[i] = f32_to_bf16_bits(lo[2 * i]) | (static_cast<uint32_t>(f32_to_bf16_bits(lo[2 * i + 1])) << 16);
        w[2 + i] = f32_to_bf16_bits(hi[2 * i]) | (static_cast<uint32_t>(f32_to_bf16_bits(hi[2 * i + 1])) << 16);
      }
    }
    *reinterpret_cast<uint4v*>(buf + ((static_cast<size_t>(b) * H + h) * n_slots + slot) * 2 * kHeadDim +
                               kv * kHeadDim + 8 * j) = w;
  }
}

hipError_t launch_window_fill(uint16_t* buf, int batch, int num_kv_heads, int sinks, int recent, const void* k,
                              const void* v, int in_kind, int n_tokens, const int32_t* seq_ids,
                              const int32_t* positions, const int32_t* seq_lens, hipStream_t stream) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(window_fill_kernel, dim3(n_tokens), dim3(kFillThreads), 0, stream, buf, batch, num_kv_heads,
                     sinks, recent, k, v, in_kind, seq_ids, positions, seq_lens);
  return hipGetLastError();
}

}  // namespace kvq
