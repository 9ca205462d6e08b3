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
    uint8_t* block = pool + (static_cast<size_t>(page) * num_kv_heads + h) * block_bytes(kbits, vbits);
    float2 r;
    if (gsize == 128) {
      const float2 a = s_rng[t][0], b = s_rng[t][1];
      r = float2{fminf(a.x, b.x), fmaxf(a.y, b.y)};
    } else {
      r = q2_wave_range(xv, gsize);
    }
    const float lvl = q2_pack_channel(xv, j, tensor, block, slot & 15, clip, r.x, r.y, kbits, vbits);
    if (sq_err != nullptr) {  // squared error over this wave's 64 channels
      float e = (xv - lvl) * (xv - lvl);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o);
      if ((j & 63) == 0) sq_err[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * 2 + (j >> 6)] = e;
    }
  }
}

// ---------------------------------------------------------------------------
// Bulk path (n_tokens >= kBulkMin, raw bf16/fp32 input): workgroups of 8
// waves, each bound to one (KV head, tensor) and striding over its tiles of
// 512 tokens.  Dense R (kRot = 0) is staged once in LDS
// as split-fp16 MFMA operands (kvq_rot.h); each wave rotates 16 tokens at a
// time on the matrix cores.  A Hadamard R (kRot = 1) is applied in registers:
// lane (row, kq) holds columns 32 kb + 8 kq + e of one token, so the seven
// butterfly stages run on column bits 0-2 (e) and 5-6 (kb) inside the lane and
// on bits 3-4 (kq) across lanes 16 and 32 apart, in the stage order of wht128,
// which makes the result bitwise that of the tiled kernel.  Either way the
// wave passes the rotated rows through its own LDS rows and quantizes them
// with one lane per (token, 32-channel group) (kvq_quant.h: q2_group32),
// packing the K and V words across lanes.
constexpr int kBulkThreads = 512;
constexpr int kBulkWaves = kBulkThreads / 64;
constexpr int kBulkRounds = 4;                        // 16-token tiles per wave
constexpr int kBulkTile = 16 * kBulkWaves * kBulkRounds;  // tokens per workgroup

template <int kIn, int kRot>  // kIn: 0 = bf16, 1 = fp32; kRot: 0 = dense R, 1 = Hadamard signs
__global__ __launch_bounds__(kBulkThreads) void append_bulk_kernel(
    uint8_t* __restrict__ pool, int num_pages, int num_kv_heads, const void* __restrict__ k_in,
    const void* __restrict__ v_in, int n_tokens, const int32_t* __restrict__ slots, const float* __restrict__ mu,
    const float* __restrict__ r_k, const float* __restrict__ r_v, float* __restrict__ rot_out, float clip, int gsize,
    float* __restrict__ sq_err, int kbits, int vbits) {
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;  // 0: key, 1: value
  const int bits = tensor == 0 ? kbits : vbits;
  const bool wide = bits > 2;  // this workgroup packs 3- or 4-bit codes (high bits in the tensor's plane)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  __shared__ half8 s_op[kRot == 0 ? 32 * 2 * 64 : 1];          // R operands, 64 KB (dense R only)
  __shared__ float s_x[kBulkWaves][16][kHeadDim + 4];          // rotated rows of each wave's 16 tokens

  if (kRot == 0)
    stage_rotation((tensor == 0 ? r_k : r_v) + static_cast<size_t>(h) * kHeadDim * kHeadDim, s_op, wave, kBulkWaves,
                   lane);
  // this lane's A columns 32 kb + 8 kq + e; key centre (fp32) or 0, and the Hadamard signs
  const int kq = lane >> 4, row = lane & 15;
  float cen[4][8], sgn[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cen[kb][e] = (tensor == 0 && mu != nullptr) ? mu[h * kHeadDim + 32 * kb + 8 * kq + e] : 0.0f;
      sgn[kb][e] = kRot == 1 ? (tensor == 0 ? r_k : r_v)[h * kHeadDim + 32 * kb + 8 * kq + e] : 0.0f;
    }
  __syncthreads();

  const void* src = tensor == 0 ? k_in : v_in;
  const int n_tiles = (n_tokens + kBulkTile - 1) / kBulkTile;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int n0 = tile * kBulkTile;
    // raw A rows of the wave's 16-token tile m, loaded one tile ahead: row `row`
    // (clamped; rows past the end are never stored), columns 32 kb + 8 kq ..
    constexpr int kRawWords = kIn == 0 ? 4 : 8;  // uint4v per lane: 4 kb x 8 bf16, or 4 kb x 8 fp32
    auto load_raw = [&](int m, uint4v (&raw)[kRawWords]) {
      const int r0 = n0 + 16 * (kBulkWaves * m + wave);
      const size_t base = (static_cast<size_t>(min(r0 + row, n_tokens - 1)) * num_kv_heads + h) * kHeadDim;
  #pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const size_t off = base + 32 * kb + 8 * kq;
        if (kIn == 0) {
          raw[kb] = *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(src) + off);
        } else {
          raw[2 * kb] = *reinterpret_cast<const uint4v*>(static_cast<const float*>(src) + off);
          raw[2 * kb + 1] = *reinterpret_cast<const uint4v*>(static_cast<const float*>(src) + off + 4);
        }
      }
    };
    uint4v raw[kRawWords], next[kRawWords];
    load_raw(0, raw);
    for (int m = 0; m < kBulkRounds; ++m) {
      const int r0 = n0 + 16 * (kBulkWaves * m + wave);  // this wave's first token
      if (m + 1 < kBulkRounds) load_raw(m + 1, next);
      half8 a_hi[4], a_lo[4];
      float ah[4][8];  // the centred row values (Hadamard: also sign-flipped)
  #pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float a[8];
        if (kIn == 0) {
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[2 * e] = __uint_as_float(raw[kb][e] << 16);
            a[2 * e + 1] = __uint_as_float(raw[kb][e] & 0xffff0000u);
          }
        } else {
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = __uint_as_float(raw[2 * kb][e]);
            a[4 + e] = __uint_as_float(raw[2 * kb + 1][e]);
          }
        }
  #pragma unroll
        for (int e = 0; e < 8; ++e)  // key centering (fp32); values use centre 0
          ah[kb][e] = kRot == 0 ? a[e] - cen[kb][e] : (a[e] - cen[kb][e]) * sgn[kb][e];
      }
      if (kRot == 0) {
        // the row's split scale from its largest magnitude (its 128 values over
        // the four lanes 16 kq + row), and the unscale of output rows 4 (lane/16) + i
        float amax = 0.0f;
  #pragma unroll
        for (int kb = 0; kb < 4; ++kb)
  #pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(ah[kb][e]));
        float u0, u1;
        swap16(amax, u0, u1);
        amax = fmaxf(u0, u1);
        swap32(amax, u0, u1);
        amax = fmaxf(u0, u1);
        const float rs = row_split_scale(amax);
  #pragma unroll
        for (int kb = 0; kb < 4; ++kb)
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            _Float16 hh, ll;
            split_f16(ah[kb][e], rs, hh, ll);
            a_hi[kb][e] = hh;
            a_lo[kb][e] = ll;
          }
        const float inv = 1.0f / (rs * kRotScale);  // a power of two: exact
        float unscale[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i) unscale[i] = __shfl(inv, 4 * (lane >> 4) + i);  // lane r holds row r
        float4v C[8];
        rotate16(a_hi, a_lo, s_op, lane, unscale, C);
  #pragma unroll
        for (int nt = 0; nt < 8; ++nt)
  #pragma unroll
          for (int i = 0; i < 4; ++i) s_x[wave][4 * (lane >> 4) + i][16 * nt + (lane & 15)] = C[nt][i];
      } else {
        // stage k pairs column c (bit k clear) with c + 2^k: (lo, hi) -> (lo + hi, lo - hi)
  #pragma unroll
        for (int k = 0; k < 3; ++k)  // column bits 0-2: e
  #pragma unroll
          for (int kb = 0; kb < 4; ++kb)
  #pragma unroll
            for (int e = 0; e < 8; ++e)
              if ((e & (1 << k)) == 0) {
                const float lo = ah[kb][e], hi = ah[kb][e | (1 << k)];
                ah[kb][e] = lo + hi;
                ah[kb][e | (1 << k)] = lo - hi;
              }
  #pragma unroll
        for (int k = 3; k < 5; ++k) {  // column bits 3-4: kq, lane bits 4-5
          const int lb = 16 << (k - 3);
  #pragma unroll
          for (int kb = 0; kb < 4; ++kb)
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pv = __shfl_xor(ah[kb][e], lb);
              ah[kb][e] = (lane & lb) ? pv - ah[kb][e] : ah[kb][e] + pv;
            }
        }
  #pragma unroll
        for (int k = 5; k < 7; ++k)  // column bits 5-6: kb
  #pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            if ((kb & (1 << (k - 5))) == 0) {
  #pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float lo = ah[kb][e], hi = ah[kb | (1 << (k - 5))][e];
                ah[kb][e] = lo + hi;
                ah[kb | (1 << (k - 5))][e] = lo - hi;
              }
            }
  #pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float* dst = &s_x[wave][row][32 * kb + 8 * kq];
          *reinterpret_cast<float4v*>(dst) = float4v{ah[kb][0] * kInvSqrt128, ah[kb][1] * kInvSqrt128,
                                                     ah[kb][2] * kInvSqrt128, ah[kb][3] * kInvSqrt128};
          *reinterpret_cast<float4v*>(dst + 4) = float4v{ah[kb][4] * kInvSqrt128, ah[kb][5] * kInvSqrt128,
                                                         ah[kb][6] * kInvSqrt128, ah[kb][7] * kInvSqrt128};
        }
      }

      // Quantize-pack this wave's 16 tokens: lane (token r, group g) holds the
      // 32 channels of group g of token r.  The rows were written by this wave
      // only; the barrier orders those LDS writes before the reads.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int r = lane >> 2, g = lane & 3;
      const int n = r0 + r;
      float x[32];
  #pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float4v q4 = *reinterpret_cast<const float4v*>(&s_x[wave][r][32 * g + 4 * u]);
        x[4 * u] = q4[0];
        x[4 * u + 1] = q4[1];
        x[4 * u + 2] = q4[2];
        x[4 * u + 3] = q4[3];
      }
      uint32_t pair, code[32];
      q2_group32(x, clip, gsize, pair, code, static_cast<float>((1 << bits) - 1));
      const int slot = n < n_tokens ? slots[n] : -1;
      const bool ok = slot >= 0 && slot < num_pages * kPage;  // same for the token's four lanes
      if (sq_err != nullptr) {  // squared error of groups g and g ^ 1: channels [64 (g / 2), +64)
        const float sc = __builtin_bit_cast(_Float16, static_cast<uint16_t>(pair & 0xffffu));
        const float zr = __builtin_bit_cast(_Float16, static_cast<uint16_t>(pair >> 16));
        float e = 0.0f;
  #pragma unroll
        for (int c = 0; c < 32; ++c) {
          const float d = x[c] - fmaf(sc, static_cast<float>(code[c]), zr);
          e = fmaf(d, d, e);
        }
        e += __shfl_xor(e, 1);
        if (ok && (g & 1) == 0) sq_err[((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * 2 + (g >> 1)] = e;
      }
      if (rot_out != nullptr && n < n_tokens) {
        float* dst = rot_out + ((static_cast<size_t>(n) * num_kv_heads + h) * 2 + tensor) * kHeadDim + 32 * g;
  #pragma unroll
        for (int u = 0; u < 8; ++u)
          *reinterpret_cast<float4v*>(dst + 4 * u) = float4v{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
      }
      // Slots 2k and 2k + 1 of a page share their V words.  The partner of this
      // token's slot is held by token r - 1 or r + 1 of the tile when this call
      // writes it there (lane 4 pr + g, the same group).
      const int pr = (slot & 1) ? r - 1 : r + 1;
      const int plane = 4 * (pr & 15) + g;
      const int pslot = __shfl(slot, plane);
      const bool paired = ok && pr >= 0 && pr < 16 && pslot == (slot ^ 1);
      const int off = slot & 15;
      uint8_t* block =  // the block stride follows the cache format (key and value bits)
          pool + (static_cast<size_t>(ok ? slot >> 4 : 0) * num_kv_heads + h) * block_bytes(kbits, vbits);
      if (ok) {  // metadata pair of (token, group): record 4g + off/4
        *reinterpret_cast<uint32_t*>(block + kCodeBytes + kMetaRecordBytes * (4 * g + (off >> 2)) + 16 * tensor +
                                     4 * (off & 3)) = pair;
      }
      if (tensor == 0) {
        // K: channel 32g + 8ak + e -> record 16ak + off, word K[g/2], bit 2(4(g%2) + e/2) + 16(e%2)
        uint32_t kw[4];
        uint32_t khw[4];  // 4-bit keys: the high bits, same positions, in the plane at kKHiPlane
  #pragma unroll
        for (int ak = 0; ak < 4; ++ak) {
          uint32_t w = 0, wh = 0;
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int sh = 2 * (4 * (g & 1) + (e >> 1)) + 16 * (e & 1);
            w |= (code[8 * ak + e] & 3u) << sh;
            wh |= (code[8 * ak + e] >> 2) << sh;
          }
          kw[ak] = w | __shfl_xor(w, 1);  // both groups of the word
          khw[ak] = wh | __shfl_xor(wh, 1);
        }
        if (ok && (g & 1) == 0) {
  #pragma unroll
          for (int ak = 0; ak < 4; ++ak) {
            *reinterpret_cast<uint32_t*>(block + 16 * (16 * ak + off) + 4 * (g >> 1)) = kw[ak];
            if (wide) *reinterpret_cast<uint32_t*>(block + kKHiPlane + 8 * (16 * ak + off) + 4 * (g >> 1)) = khw[ak];
          }
        }
      } else {
        // V: channel 32g + 16tt + b -> record 16(off/4) + b, word V[(off%4)/2],
        // bit 2(2g + tt) + 16(off%2); the token's bits of word b after the group OR
        // The high bits of wide values go to the same positions of the values'
        // plane: record 16(off/4) + b at v_hi_plane + 8 record, word VH[(off%4)/2].
        const int hs = 16 * (off & 1);
  #pragma unroll 1
        for (int part = 0; part < (wide ? 2 : 1); ++part) {
          const int dn = 2 * part;  // part 0: bits 0-1 of each code, part 1: bits 2-3
          uint32_t vw[16];
  #pragma unroll
          for (int bb = 0; bb < 16; ++bb) {
            uint32_t w = (((code[bb] >> dn) & 3u) << (4 * g + hs)) | (((code[16 + bb] >> dn) & 3u) << (4 * g + 2 + hs));
            w |= __shfl_xor(w, 1);
            w |= __shfl_xor(w, 2);
            vw[bb] = w;
          }
          auto word_at = [&](int bb) {
            const int rec = 16 * (off >> 2) + bb;
            return reinterpret_cast<uint32_t*>(block + (part == 0 ? 16 * rec + 8 : v_hi_plane(kbits) + 8 * rec) +
                                               4 * ((off & 3) >> 1));
          };
          // Both slots of a word written by this tile: the even slot's lane stores
          // the combined word whole.  Otherwise the partner slot may be written
          // concurrently by another tile (or keeps an older token): only this
          // slot's half, with atomic and/or.
          const uint32_t mask = 0xffffu << hs;
  #pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t mine = vw[4 * g + u];
            const uint32_t other = __shfl(mine, plane);
            if (paired) {
              if ((slot & 1) == 0) *word_at(4 * g + u) = mine | other;
            } else if (ok) {
              uint32_t* word = word_at(4 * g + u);
              atomicAnd(word, ~mask);
              atomicOr(word, mine);
            }
          }
        }
      }
  #pragma unroll
      for (int u = 0; u < kRawWords; ++u) raw[u] = next[u];
    }
  }  // tiles
}

hipError_t launch_append(uint8_t* pool, int num_pages, int num_kv_heads, const void* k, const void* v, int in_kind,
                         int n_tokens, const int32_t* slots, const float* mu, const float* r_k, const float* r_v,
                         float* rot_out, float clip, int rot_kind, int gsize, float* sq_err, int kbits, int vbits,
                         hipStream_t stream) {
  (void)hipGetLastError();  // report only this call's launch errors, not stale ones
  if (in_kind != 2 && n_tokens >= kBulkMin) {
    // about one workgroup per compute unit in all (each staging its dense R once;
    // over 128 VGPRs per lane, one 8-wave workgroup fills a compute unit)
    const int n_tiles = (n_tokens + kBulkTile - 1) / kBulkTile;
    const int per = std::max(1, std::min(n_tiles, (256 + 2 * num_kv_heads - 1) / (2 * num_kv_heads)));
    const dim3 bgrid(per, num_kv_heads, 2);
    auto kern = in_kind == 0 ? (rot_kind == 0 ? append_bulk_kernel<0, 0> : append_bulk_kernel<0, 1>)
                             : (rot_kind == 0 ? append_bulk_kernel<1, 0> : append_bulk_kernel<1, 1>);
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
