// Output-error evaluator (OptR section 3.2, Eq. (6)-(10)) at the decode position
// of each sequence, read from the packed cache.
//
// For query head j of sequence b (KV head h = j / g) over the positions s < T_b
// on present pages, with c = sm_scale * log2(e):
//   exact      a_s  = c <q_j, k_s>                 p  = softmax(a)
//   INT2 keys  a~_s = c <q_j R_K, x_hat_s>          p~ = softmax(a~)
// (the effective key is x_hat R_K^T + mu; <q_j, mu> shifts every a~_s equally
// and drops out of p~).  Three readouts:
//   A = sum p v,   B = sum p~ v,   C = (sum p~ w_hat) R_V^T
// so that dO_K = B - A (key-induced, Eq. (8) before W_O) and dO_V = C - B
// (value-induced).  eval_attn_kernel computes them with one workgroup per
// (split of pages, KV head, sequence) and a last-workgroup merge;
// eval_project_kernel then applies W_O,j (dy = dO W_O,j^T) and forms
// E_out = ||dy_K + dy_V||^2 (Eq. (10)).  E_rec (Eq. (9)) sums the per-token
// squared quantization errors the append wrote (rotated basis, which R
// preserves).
//
// This is a calibration-time diagnostic, written for clarity on the vector
// ALUs: per page a wave stages the 16 tokens' exact rows and the packed block in
// LDS; lane (token, head quad) forms both logits of its heads, then lane
// (channel pair) accumulates the three readouts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kEvWaves = 4;
constexpr int kEvThreads = 64 * kEvWaves;
constexpr int kRowPad = kHeadDim + 4;  // LDS row stride (floats) of staged exact rows: conflict-free row reads
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrt128f = 0.0883883476483184405f;

__device__ __forceinline__ float ld_ag(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// R[i][c] of KV head h: a dense row-major matrix, or diag(s) H / sqrt(128) from the signs s.
__device__ __forceinline__ float rot_elem(const float* r, int rot_kind, int h, int i, int c) {
  if (rot_kind == 0) return r[(static_cast<size_t>(h) * kHeadDim + i) * kHeadDim + c];
  const float s = r[h * kHeadDim + i];
  return (__popc(i & c) & 1) ? -s * kInvSqrt128f : s * kInvSqrt128f;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One page's global data held in registers while the previous page is computed.
template <bool kF32>
struct PageRegs {
  static constexpr int kRowWords = kF32 ? 8 : 4;  // uint4 per lane for 16 rows of k (or v)
  uint4v k[kRowWords], v[kRowWords], blk[3];  // the block as 16-byte chunks lane, 64 + lane, 128 + lane
  float4v err;  // this lane's token's squared errors, K and V (lanes 0..15)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// kPlanes: high-bit planes per block (3- or 4-bit keys, values); kMfma: the matrix-core page loop (bf16 k and
// v, 2-bit codes), else the vector-ALU one
template <int kNH, bool kF32, int kPlanes, bool kMfma>
__global__ __launch_bounds__(kEvThreads) __attribute__((amdgpu_waves_per_eu(2))) void eval_attn_kernel(
    const EvalParams p) {
  static_assert(!kMfma || (!kF32 && kPlanes == 0), "the MFMA page loop reads bf16 rows and 2-bit codes");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = p.num_kv_heads;
  const int b = blockIdx.y;
  const int h = blockIdx.x % H;
  const int split = blockIdx.x / H;
  const int hc = blockIdx.z;                           // chunk of at most kEvHeads query heads of KV head h
  const int n_hc = gridDim.z;
  const int g = min(kEvHeads, p.g - kEvHeads * hc);    // query heads of this workgroup
  const int T = min(max(p.seq_lens[b], 0), p.len_cap);
  const int n_pages = (T + kPage - 1) / kPage;
  const int n_valid = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  const size_t row_j0 =  // output row of (b, j = h g_kv + kEvHeads hc)
      static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(h) * p.g + kEvHeads * hc;
  const size_t slot = (static_cast<size_t>(b) * H + h) * n_hc + hc;  // counter and partial block
  if (n_valid == 0) {  // nothing attended: no differences and no reconstruction error
    if (split == 0) {
      for (int idx = tid; idx < g * 2 * kHeadDim; idx += kEvThreads) p.dobuf[row_j0 * 2 * kHeadDim + idx] = 0.0f;
      if (tid == 0 && hc == 0) p.e_rec[b * H + h] = 0.0f;
    }
    return;
  }
  if (split >= n_valid) return;

  __shared__ float s_q[kNH][kHeadDim];   // q * c
  __shared__ float s_qh[kNH][kHeadDim];  // q R_K * c
  __shared__ float s_qs[kNH][4];         // per-32-channel sums of s_qh
  // per-wave page staging, reused by the merges
  constexpr int kBlk = kBlockBytes + 512 * kPlanes;  // the largest block of this plane count (G = 32, 4 bits)
  constexpr int kBlkWords = kBlk / 4;
  const int nb = block_bytes(p.kbits, p.vbits, p.gsize);  // this pool's block: its stride and size
  const int nb_chunks = nb / 16;
  const int msh = meta_shift(p.gsize);                // metadata record of 32-channel group c: 4 (c >> msh) + slot / 4
  constexpr int kStage = 2 * kPage * kRowPad + kBlkWords + 2 * kNH * kPage + 2 * kNH;
  const bool kwide = kPlanes > 0 && p.kbits > 2;     // the keys' high-bit plane after the metadata
  const bool vwide = kPlanes > 0 && p.vbits > 2;     // the values' plane after it
  const bool k3 = p.kbits == 3, v3 = p.vbits == 3;   // 3-bit planes: one word per record
  const int kpw = k_hi_plane(p.gsize) / 4;           // word index of the keys' plane
  const int vpw = v_hi_plane(p.kbits, p.gsize) / 4;  // word index of the values' plane
  constexpr int kMergeW = kEvWaves * kNH * (3 * kHeadDim + 4) + kEvWaves;
  constexpr int kBuf = kEvWaves * kStage > kMergeW ? kEvWaves * kStage : kMergeW;
  __shared__ __align__(16) float s_buf[kBuf];
  __shared__ float s_fq[kNH];  // MFMA path: the INT2 query scale f per head
  __shared__ int s_ticket;

  // ---- queries, scaled by c, and their rotation q R_K
  const float c_log2 = p.sm_scale * kLog2e;
  for (int idx = tid; idx < kNH * kHeadDim; idx += kEvThreads) {
    const int jj = idx / kHeadDim, c = idx % kHeadDim;
    float qv = 0.0f;
    if (jj < g) {
      const size_t qi = (row_j0 + jj) * kHeadDim + c;
      qv = p.q_kind == 0 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.q)[qi]) : static_cast<const float*>(p.q)[qi];
    }
    s_q[jj][c] = qv * c_log2;
  }
  __syncthreads();
  for (int idx = tid; idx < kNH * kHeadDim; idx += kEvThreads) {
    const int jj = idx / kHeadDim, c = idx % kHeadDim;
    float acc = 0.0f;
    for (int i = 0; i < kHeadDim; ++i) acc = fmaf(s_q[jj][i], rot_elem(p.r_k, p.rot_kind, h, i, c), acc);
    s_qh[jj][c] = acc;
  }
  __syncthreads();
  if (tid < kNH * 4) {
    const int jj = tid / 4, grp = tid % 4;
    float s = 0.0f;
    for (int c = 0; c < 32; ++c) s += s_qh[jj][32 * grp + c];
    s_qs[jj][grp] = s;
  }
  __syncthreads();

  const int p_first = split * p.pages_per_split;
  const int p_end = min(p_first + p.pages_per_split, n_pages);
  const int64_t row0 = p.row0[b];
  // the waves' rows for the merge: [wave][head][A | B | C (128 each) | m_a l_a m_q l_q], then [wave] errors
  constexpr int kWRow = 3 * kHeadDim + 4;
  float* const s_mw = s_buf;
  float* const s_merr = s_buf + kEvWaves * kNH * kWRow;

  if constexpr (!kMfma) {
  // ---- this wave's pages: first + wave, + kEvWaves, ...
  float* const st = s_buf + wave * kStage;
  float* const s_k = st;                                   // [16][kRowPad]
  float* const s_v = st + kPage * kRowPad;                 // [16][kRowPad]
  uint32_t* const s_blk = reinterpret_cast<uint32_t*>(st + 2 * kPage * kRowPad);  // the block: up to 384, 512 or 640 words
  float* const s_p = st + 2 * kPage * kRowPad + kBlkWords;  // [2][kNH][16]
  float* const s_al = s_p + 2 * kNH * kPage;                      // [2][kNH]

  constexpr int kHQ = kNH / 4;  // heads per lane in the logit phase: j = jq + 4 u
  const int t_l = lane & 15, jq = lane >> 4;
  float m_a[kHQ], l_a[kHQ], m_q[kHQ], l_q[kHQ];
#pragma unroll
  for (int u = 0; u < kHQ; ++u) {
    m_a[u] = -INFINITY;
    m_q[u] = -INFINITY;
    l_a[u] = 0.0f;
    l_q[u] = 0.0f;
  }
  float accA[kNH][2], accB[kNH][2], accC[kNH][2];
#pragma unroll
  for (int jj = 0; jj < kNH; ++jj)
#pragma unroll
    for (int e = 0; e < 2; ++e) accA[jj][e] = accB[jj][e] = accC[jj][e] = 0.0f;
  float e_acc = 0.0f;

  // the table entry of page pg of the split (-1 past the split), loaded ahead and checked at use
  // (a check in the loading block would wait for the load there)
  auto page_of = [&](int pg) -> int {
    return pg < p_end ? p.page_table[static_cast<size_t>(b) * p.max_pages + pg] : -1;
  };
  auto present = [&](int id) { return id >= 0 && id < p.num_pages; };
  auto load_page = [&](int pg, int id, PageRegs<kF32>& r) {
    const int nt = min(kPage, T - kPage * pg);
    const uint8_t* blk = p.pool + (static_cast<size_t>(id) * H + h) * nb;
#pragma unroll
    for (int u = 0; u < 3; ++u)
      r.blk[u] = 64 * u + lane < nb_chunks ? *reinterpret_cast<const uint4v*>(blk + 16 * (64 * u + lane))
                                           : uint4v{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < PageRegs<kF32>::kRowWords; ++u) {
      const int idx = u * 64 + lane;
      const int t = kF32 ? idx >> 5 : idx >> 4;
      const int part = kF32 ? idx & 31 : idx & 15;
      if (t < nt) {
        const size_t e0 = (static_cast<size_t>(row0 + kPage * pg + t) * H + h) * kHeadDim + (kF32 ? 4 : 8) * part;
        if (kF32) {
          r.k[u] = *reinterpret_cast<const uint4v*>(static_cast<const float*>(p.k) + e0);
          r.v[u] = *reinterpret_cast<const uint4v*>(static_cast<const float*>(p.v) + e0);
        } else {
          r.k[u] = *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(p.k) + e0);
          r.v[u] = *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(p.v) + e0);
        }
      } else {
        r.k[u] = uint4v{0u, 0u, 0u, 0u};
        r.v[u] = uint4v{0u, 0u, 0u, 0u};
      }
    }
    // this lane's token's squared errors (lanes 0..15), summed when the page is consumed
    r.err = p.sq_err != nullptr && lane < nt
                ? *reinterpret_cast<const float4v*>(p.sq_err + (static_cast<size_t>(row0 + kPage * pg + lane) * H + h) * 4)
                : float4v{0.0f, 0.0f, 0.0f, 0.0f};
  };
  auto stage_page = [&](const PageRegs<kF32>& r) {
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (64 * u + lane < nb_chunks) reinterpret_cast<uint4v*>(s_blk)[64 * u + lane] = r.blk[u];
#pragma unroll
    for (int u = 0; u < PageRegs<kF32>::kRowWords; ++u) {
      const int idx = u * 64 + lane;
      const int t = kF32 ? idx >> 5 : idx >> 4;
      const int part = kF32 ? idx & 31 : idx & 15;
      if (kF32) {
        *reinterpret_cast<uint4v*>(s_k + t * kRowPad + 4 * part) = r.k[u];
        *reinterpret_cast<uint4v*>(s_v + t * kRowPad + 4 * part) = r.v[u];
      } else {
        const uint4v kw = r.k[u], vw = r.v[u];
        float* kd = s_k + t * kRowPad + 8 * part;
        float* vd = s_v + t * kRowPad + 8 * part;
        *reinterpret_cast<float4v*>(kd) = float4v{__uint_as_float(kw[0] << 16), __uint_as_float(kw[0] & 0xffff0000u),
                                                  __uint_as_float(kw[1] << 16), __uint_as_float(kw[1] & 0xffff0000u)};
        *reinterpret_cast<float4v*>(kd + 4) = float4v{__uint_as_float(kw[2] << 16), __uint_as_float(kw[2] & 0xffff0000u),
                                                      __uint_as_float(kw[3] << 16), __uint_as_float(kw[3] & 0xffff0000u)};
        *reinterpret_cast<float4v*>(vd) = float4v{__uint_as_float(vw[0] << 16), __uint_as_float(vw[0] & 0xffff0000u),
                                                  __uint_as_float(vw[1] << 16), __uint_as_float(vw[1] & 0xffff0000u)};
        *reinterpret_cast<float4v*>(vd + 4) = float4v{__uint_as_float(vw[2] << 16), __uint_as_float(vw[2] & 0xffff0000u),
                                                      __uint_as_float(vw[3] << 16), __uint_as_float(vw[3] & 0xffff0000u)};
      }
    }
  };

  // Pages pg = p_first + wave, + kEvWaves, ...: the page's data is loaded one
  // page ahead and its id two pages ahead, so neither latency is waited on
  // in line; an absent page is skipped after its (masked) turn.
  int pg = p_first + wave;
  int id_cur = page_of(pg);
  PageRegs<kF32> cur;
  if (present(id_cur)) load_page(pg, id_cur, cur);
  int id_nxt = page_of(pg + kEvWaves);
  for (; pg < p_end; pg += kEvWaves) {
    const int nt = min(kPage, T - kPage * pg);
    const bool here = present(id_cur);
    if (here) {
      stage_page(cur);
      e_acc += (cur.err[0] + cur.err[1]) + (cur.err[2] + cur.err[3]);
    }
    PageRegs<kF32> nxt;
    if (present(id_nxt)) load_page(pg + kEvWaves, id_nxt, nxt);
    const int id_2 = page_of(pg + 2 * kEvWaves);  // issued last: no wait below covers it
    id_cur = id_nxt;
    id_nxt = id_2;
    if (!here) {
      cur = nxt;
      continue;
    }
    wave_sync();

    // ---- logits: lane (token t_l, head quad jq) forms a and a~ of heads jq + 4 u
    float ea[kHQ], eq[kHQ];
    {
      float dq[kHQ][4];
#pragma unroll
      for (int u = 0; u < kHQ; ++u) {
        ea[u] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) dq[u][kk] = 0.0f;
      }
      const float* krow = s_k + t_l * kRowPad;
      float ea2[kHQ][2];  // two interleaved sums: shorter dependency chains
#pragma unroll
      for (int u = 0; u < kHQ; ++u) ea2[u][0] = ea2[u][1] = 0.0f;
#pragma unroll 4
      for (int c4 = 0; c4 < kHeadDim / 4; ++c4) {
        const float4v kv = *reinterpret_cast<const float4v*>(krow + 4 * c4);
#pragma unroll
        for (int u = 0; u < kHQ; ++u) {
          const float4v qv = *reinterpret_cast<const float4v*>(&s_q[jq + 4 * u][4 * c4]);
          ea2[u][c4 & 1] = fmaf(qv[0], kv[0], fmaf(qv[1], kv[1], fmaf(qv[2], kv[2], fmaf(qv[3], kv[3], ea2[u][c4 & 1]))));
        }
      }
#pragma unroll
      for (int u = 0; u < kHQ; ++u) ea[u] = ea2[u][0] + ea2[u][1];
      // K codes of slot t_l: record 16 a + t_l holds words K0 (groups 0, 1) and K1 (groups 2, 3);
      // channel 32 kk + 8 a + e sits at bit 2 (4 (kk % 2) + e / 2) + 16 (e % 2)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t w01[2] = {s_blk[4 * (16 * a + t_l)], s_blk[4 * (16 * a + t_l) + 1]};
        // wide keys: the high bits of record 16 a + t_l at the positions of their low bits, from the
        // plane's words H0, H1 (4 bits) or from its one word, H0's bits even and H1's odd (3 bits)
        uint32_t h01[2] = {0u, 0u};
        if (kwide) {
          if (k3) {
            const uint32_t P = s_blk[kpw + 16 * a + t_l];
            h01[0] = P & 0x55555555u;
            h01[1] = (P >> 1) & 0x55555555u;
          } else {
            h01[0] = s_blk[kpw + 2 * (16 * a + t_l)];
            h01[1] = s_blk[kpw + 2 * (16 * a + t_l) + 1];
          }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t w = w01[kk >> 1], wh = h01[kk >> 1];
          float cf[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int sh = 2 * (4 * (kk & 1) + (e >> 1)) + 16 * (e & 1);
            cf[e] = static_cast<float>(((w >> sh) & 3u) | (((wh >> sh) & 3u) << 2));
          }
#pragma unroll
          for (int u = 0; u < kHQ; ++u) {
            const float4v q0 = *reinterpret_cast<const float4v*>(&s_qh[jq + 4 * u][32 * kk + 8 * a]);
            const float4v q1 = *reinterpret_cast<const float4v*>(&s_qh[jq + 4 * u][32 * kk + 8 * a + 4]);
            dq[u][kk] = fmaf(q0[0], cf[0], fmaf(q0[1], cf[1], fmaf(q0[2], cf[2], fmaf(q0[3], cf[3], dq[u][kk]))));
            dq[u][kk] = fmaf(q1[0], cf[4], fmaf(q1[1], cf[5], fmaf(q1[2], cf[6], fmaf(q1[3], cf[7], dq[u][kk]))));
          }
        }
      }
      // a~ = sum over groups of s * <q_hat, codes> + z * sum(q_hat): K (scale, zero) of (group kk, slot t_l)
#pragma unroll
      for (int u = 0; u < kHQ; ++u) {
        float acc = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t pr = s_blk[(kCodeBytes + kMetaRecordBytes * (4 * (kk >> msh) + (t_l >> 2))) / 4 + (t_l & 3)];
          acc = fmaf(f16_lo(pr), dq[u][kk], fmaf(f16_hi(pr), s_qs[jq + 4 * u][kk], acc));
        }
        eq[u] = acc;
        if (t_l >= nt) {
          ea[u] = -INFINITY;
          eq[u] = -INFINITY;
        }
      }
    }

    // ---- online softmax per head over this page's 16 tokens (lanes sharing jq)
#pragma unroll
    for (int u = 0; u < kHQ; ++u) {
      const int jj = jq + 4 * u;
      const float ma = row16_max(ea[u]), mq = row16_max(eq[u]);
      const float na = fmaxf(m_a[u], ma), nq = fmaxf(m_q[u], mq);
      const float ala = __builtin_amdgcn_exp2f(m_a[u] - na), alq = __builtin_amdgcn_exp2f(m_q[u] - nq);
      const float pa = __builtin_amdgcn_exp2f(ea[u] - na), pq = __builtin_amdgcn_exp2f(eq[u] - nq);
      const float sa = row16_sum(pa), sq = row16_sum(pq);
      l_a[u] = fmaf(l_a[u], ala, sa);
      l_q[u] = fmaf(l_q[u], alq, sq);
      m_a[u] = na;
      m_q[u] = nq;
      // heads past g weigh nothing (their sums are never stored)
      s_p[jj * kPage + t_l] = jj < g ? pa : 0.0f;
      s_p[(kNH + jj) * kPage + t_l] = jj < g ? pq : 0.0f;
      if (t_l == 0) {
        s_al[jj] = jj < g ? ala : 1.0f;
        s_al[kNH + jj] = jj < g ? alq : 1.0f;
      }
    }
    wave_sync();

    // ---- readouts: lane (channels c0, c0 + 1)
    {
      const int c0 = 2 * lane;
#pragma unroll
      for (int jj = 0; jj < kNH; ++jj) {
        const float ala = s_al[jj], alq = s_al[kNH + jj];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          accA[jj][e] *= ala;
          accB[jj][e] *= alq;
          accC[jj][e] *= alq;
        }
      }
      // V code of slot t, channel c: record 16 (t / 4) + c % 16, word V[(t % 4) / 2], bit 2 (c / 16) + 16 (t % 2);
      // V (scale, zero) of (channel c, slot t): record 4 (c / G) + t / 4, at +16 + 4 (t % 4)
      // (a full page runs four tokens per step, so their LDS reads are issued ahead of their uses)
      const int tile = c0 >> 4, b0 = c0 & 15, grp = (c0 >> 5) >> msh;
      auto token = [&](int t) {
        const int wsel = 2 + ((t & 3) >> 1);
        const int sh = 2 * tile + 16 * (t & 1);
        const uint32_t w0 = s_blk[4 * (16 * (t >> 2) + b0) + wsel];
        const uint32_t w1 = s_blk[4 * (16 * (t >> 2) + b0 + 1) + wsel];
        uint32_t cv0 = (w0 >> sh) & 3u, cv1 = (w1 >> sh) & 3u;
        if (vwide) {
          if (v3) {  // the high bit: bit 8 (t % 4) + c / 16 of the record's plane word
            const int hb = 8 * (t & 3) + tile;
            cv0 |= ((s_blk[vpw + 16 * (t >> 2) + b0] >> hb) & 1u) << 2;
            cv1 |= ((s_blk[vpw + 16 * (t >> 2) + b0 + 1] >> hb) & 1u) << 2;
          } else {  // the high bits: the same record and bit of the values' plane, word VH[(t % 4) / 2]
            const int hsel = (t & 3) >> 1;
            cv0 |= ((s_blk[vpw + 2 * (16 * (t >> 2) + b0) + hsel] >> sh) & 3u) << 2;
            cv1 |= ((s_blk[vpw + 2 * (16 * (t >> 2) + b0 + 1) + hsel] >> sh) & 3u) << 2;
          }
        }
        const uint32_t pr = s_blk[(kCodeBytes + kMetaRecordBytes * (4 * grp + (t >> 2)) + 16) / 4 + (t & 3)];
        const float sv = f16_lo(pr), zv = f16_hi(pr);
        const float wh0 = fmaf(sv, static_cast<float>(cv0), zv);
        const float wh1 = fmaf(sv, static_cast<float>(cv1), zv);
        const float v0 = s_v[t * kRowPad + c0], v1 = s_v[t * kRowPad + c0 + 1];
#pragma unroll
        for (int jj = 0; jj < kNH; ++jj) {
          const float pa = s_p[jj * kPage + t], pq = s_p[(kNH + jj) * kPage + t];
          accA[jj][0] = fmaf(pa, v0, accA[jj][0]);
          accA[jj][1] = fmaf(pa, v1, accA[jj][1]);
          accB[jj][0] = fmaf(pq, v0, accB[jj][0]);
          accB[jj][1] = fmaf(pq, v1, accB[jj][1]);
          accC[jj][0] = fmaf(pq, wh0, accC[jj][0]);
          accC[jj][1] = fmaf(pq, wh1, accC[jj][1]);
        }
      };
      if (nt == kPage) {
#pragma unroll 4
        for (int t = 0; t < kPage; ++t) token(t);
      } else {
        for (int t = 0; t < nt; ++t) token(t);
      }
    }
    wave_sync();  // staging free for the next page
    cur = nxt;
  }

  // ---- this wave's rows of s_mw
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < kNH; ++jj) {
    if (jj < g) {
      float* row = s_mw + (wave * kNH + jj) * kWRow;
      row[2 * lane] = accA[jj][0];
      row[2 * lane + 1] = accA[jj][1];
      row[kHeadDim + 2 * lane] = accB[jj][0];
      row[kHeadDim + 2 * lane + 1] = accB[jj][1];
      row[2 * kHeadDim + 2 * lane] = accC[jj][0];
      row[2 * kHeadDim + 2 * lane + 1] = accC[jj][1];
    }
  }
#pragma unroll
  for (int u = 0; u < kHQ; ++u) {
    const int jj = jq + 4 * u;
    if (jj < g && t_l == 0) {
      float* row = s_mw + (wave * kNH + jj) * kWRow + 3 * kHeadDim;
      row[0] = m_a[u];
      row[1] = l_a[u];
      row[2] = m_q[u];
      row[3] = l_q[u];
    }
  }
  const float e_w = wave_sum(lane < kPage ? e_acc : 0.0f);
  if (lane == 0) s_merr[wave] = e_w;
  } else {
    // ---- MFMA path (bf16 k and v, 2-bit codes): lane (a = lane / 16, col = lane % 16).
    // Every product below is a 16 x 16 tile whose output lane (a, col) holds rows 4a + i:
    //   exact logits   C[token][head]   = k rows (A, token = col of the A operand) x q in three bf16
    //                                     parts (B, column = head)                 (16x16x32 bf16)
    //   INT2 logits    C[token][4grp+j] = key codes as fp16 subnormals x the block-diagonal fp16
    //                                     hi/lo of q_hat f, as in the decode kernel (16x16x32 f16)
    //   A, B readouts  C[head][ch]      = p (A: row = head, k = tokens 4a..4a+3 the lane holds)
    //                                     in two bf16 parts x v (B, tokens x 16 channels)    (16x16x16 bf16)
    //   C readout      C[4grp+j][ch]    = p~ s_v 2^-e in two fp16 parts x value codes    (16x16x16 f16)
    // so the weights formed in the logit layout feed the readouts with no transposition.
    constexpr int kNQ = kNH / 4;
    constexpr int kQpRow = kHeadDim + 8;   // bf16 per (part, head) row of the q parts (conflict-light B reads)
    constexpr int kVbRow = kHeadDim + 8;   // bf16 per staged v row
    constexpr int kQpFloats = 3 * 16 * kQpRow / 2;
    constexpr int kVbFloats = kPage * kVbRow / 2;
    constexpr int kQbFloats = kNQ * 4 * 2 * 64 * 4;  // INT2 query operands [quad][kk][hi, lo][lane], one copy
    static_assert(kQpFloats + kEvWaves * kVbFloats + kQbFloats <= kBuf, "MFMA staging fits the page buffer");
    uint16_t* const s_qp = reinterpret_cast<uint16_t*>(s_buf);                                    // [3][16][kQpRow]
    uint16_t* const s_vb = reinterpret_cast<uint16_t*>(s_buf + kQpFloats + wave * kVbFloats);  // [16][kVbRow]
    uint4v* const s_qb = reinterpret_cast<uint4v*>(s_buf + kQpFloats + kEvWaves * kVbFloats);
    const int a = lane >> 4, col = lane & 15, grp = col >> 2, jj = col & 3;
    // the three bf16 parts of q c (truncation; columns past g are zero), and the INT2 scale f per head
    for (int idx = tid; idx < 16 * kHeadDim; idx += kEvThreads) {
      const int n = idx / kHeadDim, c = idx % kHeadDim;
      float r = n < g ? s_q[n][c] : 0.0f;
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const uint32_t t = __float_as_uint(r) & 0xffff0000u;
        s_qp[(sp * 16 + n) * kQpRow + c] = static_cast<uint16_t>(t >> 16);
        r -= __uint_as_float(t);
      }
    }
    for (int jh = wave; jh < kNH; jh += kEvWaves) {
      const float am = wave_max_all(fmaxf(fabsf(s_qh[jh][lane]), fabsf(s_qh[jh][lane + 64])));
      if (lane == 0) {
        int e = 0;
        frexpf(am, &e);  // am in [2^(e-1), 2^e)
        s_fq[jh] = am > 0.0f ? ldexpf(1.0f, 14 - e) : 1.0f;
      }
    }
    __syncthreads();
    // INT2 query operands of quad Q, column 4 grp + jj: head 4 Q + jj on group grp's 32 channels, element
    // e divided by 4^(e/2) (the factor its key code carries), as fp16 hi + lo of q_hat c f; the lane's
    // operands (the same in every wave) are kept in LDS by wave 0 and read back per page, so they hold
    // no registers across the loop
    float qz[kNQ], c1[kNQ];
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      const int jl = 4 * Q + jj;
      const float f = s_fq[jl];
      half8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sc = s_qh[jl][32 * grp + 8 * a + e] * f * (1.0f / static_cast<float>(1 << (2 * (e >> 1))));
        const _Float16 hh = static_cast<_Float16>(sc);
        hi[e] = hh;
        lo[e] = static_cast<_Float16>(sc - static_cast<float>(hh));
      }
      c1[Q] = 16777216.0f / f;  // the code's 2^-24 and f undone
      qz[Q] = s_qs[jl][grp] / c1[Q];
      const half8 zero = {};
      if (wave == 0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          s_qb[((Q * 4 + kk) * 2 + 0) * 64 + lane] = __builtin_bit_cast(uint4v, grp == kk ? hi : zero);
          s_qb[((Q * 4 + kk) * 2 + 1) * 64 + lane] = __builtin_bit_cast(uint4v, grp == kk ? lo : zero);
        }
      }
    }
    __syncthreads();

    // state: exact softmax per head col, INT2 per (quad, head jj); accumulators in the output layouts
    float m_a = -INFINITY, l_a = 0.0f;
    float m_q[kNQ], l_q[kNQ], z_run[kNQ];
    float4v accA[8], accB[8], accC[kNQ][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) accA[t] = accB[t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      m_q[Q] = -INFINITY;
      l_q[Q] = 0.0f;
      z_run[Q] = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) accC[Q][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float e_acc = 0.0f;
    // lane values broadcast by readlane, picked by the lane's row a
    auto lane_val = [](float x, int k) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k)); };

    struct PageM {
      uint4v k[4], v[4];  // k: the A operand of k-step u (token col, channels 32 u + 8 a ..); v: staged rows
      uint4v rec, km, vm; // this lane's code record, its K and V metadata records
      float4v err;        // this lane's token's squared errors (lanes 0..15)
    };
    auto page_of = [&](int pg) -> int {
      return pg < p_end ? p.page_table[static_cast<size_t>(b) * p.max_pages + pg] : -1;
    };
    auto present = [&](int id) { return id >= 0 && id < p.num_pages; };
    auto load_page = [&](int pg, int id, PageM& r) {
      const int nt = min(kPage, T - kPage * pg);
      const uint16_t* kb = static_cast<const uint16_t*>(p.k);
      const uint16_t* vb = static_cast<const uint16_t*>(p.v);
      const size_t rowk = static_cast<size_t>(row0 + kPage * pg + min(col, nt - 1)) * H + h;
#pragma unroll
      for (int u = 0; u < 4; ++u) r.k[u] = *reinterpret_cast<const uint4v*>(kb + rowk * kHeadDim + 32 * u + 8 * a);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * 64 + lane, t = idx >> 4, part = idx & 15;
        r.v[u] = t < nt ? *reinterpret_cast<const uint4v*>(
                              vb + (static_cast<size_t>(row0 + kPage * pg + t) * H + h) * kHeadDim + 8 * part)
                        : uint4v{0u, 0u, 0u, 0u};
      }
      const uint8_t* blk = p.pool + (static_cast<size_t>(id) * H + h) * nb;
      r.rec = *reinterpret_cast<const uint4v*>(blk + 16 * lane);
      const uint8_t* meta = blk + kCodeBytes + kMetaRecordBytes * (4 * (grp >> msh) + a);
      r.km = *reinterpret_cast<const uint4v*>(meta);
      r.vm = *reinterpret_cast<const uint4v*>(meta + 16);
      r.err = p.sq_err != nullptr && lane < nt
                  ? *reinterpret_cast<const float4v*>(p.sq_err +
                                                      (static_cast<size_t>(row0 + kPage * pg + lane) * H + h) * 4)
                  : float4v{0.0f, 0.0f, 0.0f, 0.0f};
    };

    int pg = p_first + wave;
    int id_cur = page_of(pg);
    PageM cur;
    if (present(id_cur)) load_page(pg, id_cur, cur);
    int id_nxt = page_of(pg + kEvWaves);
    for (; pg < p_end; pg += kEvWaves) {
      const int nt = min(kPage, T - kPage * pg);
      const bool here = present(id_cur);
      if (here) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = u * 64 + lane;
          *reinterpret_cast<uint4v*>(s_vb + (idx >> 4) * kVbRow + 8 * (idx & 15)) = cur.v[u];
        }
        e_acc += (cur.err[0] + cur.err[1]) + (cur.err[2] + cur.err[3]);
      }
      PageM nxt;
      if (present(id_nxt)) load_page(pg + kEvWaves, id_nxt, nxt);
      const int id_2 = page_of(pg + 2 * kEvWaves);  // issued last: no wait below covers it
      id_cur = id_nxt;
      id_nxt = id_2;
      if (!here) {
        cur = nxt;
        continue;
      }
      const PageM& P = cur;

      // ---- logits, lane (a, col): tokens 4a + i
      float4v E = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 kA = __builtin_bit_cast(bf16x8, P.k[u]);
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const uint4v qb = *reinterpret_cast<const uint4v*>(s_qp + (sp * 16 + col) * kQpRow + 32 * u + 8 * a);
          E = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8, qb), E, 0, 0, 0);
        }
      }
      // key operands: a code at bits 2q (+16) of a word is the fp16 subnormal code 4^q 2^-24
      const uint32_t kw[4] = {P.rec[0], P.rec[0] >> 8, P.rec[1], P.rec[1] >> 8};
      half8 kA2[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint4v rr;
#pragma unroll
        for (int q = 0; q < 4; ++q) rr[q] = kw[kk] & (0x00030003u << (2 * q));
        kA2[kk] = __builtin_bit_cast(half8, rr);
      }
      bool live[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) live[i] = 4 * a + i < nt;
      float ea[4], eq[kNQ][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ea[i] = live[i] ? E[i] : -INFINITY;
#pragma unroll
      for (int Q = 0; Q < kNQ; ++Q) {
        float4v C = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const half8 qh = __builtin_bit_cast(half8, s_qb[((Q * 4 + kk) * 2 + 0) * 64 + lane]);
          const half8 ql = __builtin_bit_cast(half8, s_qb[((Q * 4 + kk) * 2 + 1) * 64 + lane]);
          C = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA2[kk], qh, C, 0, 0, 0);
          C = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA2[kk], ql, C, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // s_grp <codes, q_hat> + z_grp sum(q_hat), summed over the four groups of the row
          const float s = fmaf(C[i], f16_lo(P.km[i]), f16_hi(P.km[i]) * qz[Q]);
          const float lg = row_sum_stride4(s) * c1[Q];
          eq[Q][i] = live[i] ? lg : -INFINITY;
        }
      }

      // ---- online softmax: exact per head col; INT2 per head jj of each quad (the group lanes agree)
      const float pm = rows_max(fmaxf(fmaxf(ea[0], ea[1]), fmaxf(ea[2], ea[3])));
      const float na = fmaxf(m_a, pm);
      const float ala = __builtin_amdgcn_exp2f(m_a - na);
      float pa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = col < g ? __builtin_amdgcn_exp2f(ea[i] - na) : 0.0f;
      l_a = fmaf(l_a, ala, rows_sum((pa[0] + pa[1]) + (pa[2] + pa[3])));
      m_a = na;
      float pq[kNQ][4], alq[kNQ];
#pragma unroll
      for (int Q = 0; Q < kNQ; ++Q) {
        const float qm = rows_max(fmaxf(fmaxf(eq[Q][0], eq[Q][1]), fmaxf(eq[Q][2], eq[Q][3])));
        const float nq = fmaxf(m_q[Q], qm);
        alq[Q] = __builtin_amdgcn_exp2f(m_q[Q] - nq);
        const bool hq = 4 * Q + jj < g;
#pragma unroll
        for (int i = 0; i < 4; ++i) pq[Q][i] = hq ? __builtin_amdgcn_exp2f(eq[Q][i] - nq) : 0.0f;
        l_q[Q] = fmaf(l_q[Q], alq[Q], rows_sum((pq[Q][0] + pq[Q][1]) + (pq[Q][2] + pq[Q][3])));
        m_q[Q] = nq;
      }
      // rescale the sums kept against the old maxima (wave-uniform skip when nothing moved)
      bool moved = ala != 1.0f;
#pragma unroll
      for (int Q = 0; Q < kNQ; ++Q) moved = moved || alq[Q] != 1.0f;
      if (__ballot(moved) != 0) {
        // accA / accB rows 4a + i are heads 4a + i: their factors come from lane 4a + i (row 0)
        float fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float xa = 1.0f, xb = 1.0f;
#pragma unroll
          for (int Q = 0; Q < kNQ; ++Q) {
            const float va = lane_val(ala, 4 * Q + i), vb = lane_val(alq[Q], i);
            xa = a == Q ? va : xa;
            xb = a == Q ? vb : xb;
          }
          fa[i] = xa;
          fb[i] = xb;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accA[t][i] *= fa[i];
            accB[t][i] *= fb[i];
          }
#pragma unroll
        for (int Q = 0; Q < kNQ; ++Q) {
          // accC[Q] rows 4 grp + i are head 4 Q + i: the factor of lane i
          float fc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) fc[i] = lane_val(alq[Q], i);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) accC[Q][t][i] *= fc[i];
          z_run[Q] *= alq[Q];
        }
      }

      // ---- readouts A = sum p v, B = sum p~ v (rows = heads), C = sum p~ w_hat (rows 4 grp + j per quad)
      wave_sync();  // the staged v rows are visible to the whole wave
      // x = hi + lo + r by truncation, |r| < 2^-16 |x| (the weights are finite and nonnegative)
      auto split_bf16 = [](const float (&x)[4], short4v& hi, short4v& lo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t t = __float_as_uint(x[i]) & 0xffff0000u;
          hi[i] = static_cast<short>(t >> 16);
          lo[i] = static_cast<short>(__float_as_uint(x[i] - __uint_as_float(t)) >> 16);
        }
      };
      short4v pa_hi, pa_lo, pb_hi, pb_lo;
      split_bf16(pa, pa_hi, pa_lo);
      float pbv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.0f;  // row col of the B readout: head col = 4 Q + jj, this lane's jj
#pragma unroll
        for (int Q = 0; Q < kNQ; ++Q) x = (col >> 2) == Q ? pq[Q][i] : x;
        pbv[i] = x;
      }
      split_bf16(pbv, pb_hi, pb_lo);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        short4v vB;
#pragma unroll
        for (int i = 0; i < 4; ++i) vB[i] = static_cast<short>(s_vb[(4 * a + i) * kVbRow + 16 * t + col]);
        accA[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, vB, accA[t], 0, 0, 0);
        accA[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, vB, accA[t], 0, 0, 0);
        accB[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb_hi, vB, accB[t], 0, 0, 0);
        accB[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb_lo, vB, accB[t], 0, 0, 0);
      }
      // value scales and zeros of the lane's tokens (masked slots: 0, whatever bits they hold);
      // the page's unit 2^e per group brings its largest scale into [1/2, 1)
      float sv[4], zv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = live[i] ? f16_lo(P.vm[i]) : 0.0f;
        zv[i] = live[i] ? f16_hi(P.vm[i]) : 0.0f;
      }
      const float smax = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      int ex = 0;
      frexpf(smax, &ex);  // smax in [2^(ex-1), 2^ex)
      if (!(smax > 0.0f)) ex = 0;
      const float unit_in = ldexpf(1.0f, -ex);
      // the output rows 4 a + i belong to group a: its unit comes from lane 4 a (group a's lanes agree)
      float eo = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = lane_val(static_cast<float>(ex), 4 * k);
        eo = a == k ? v : eo;
      }
      const float unit_out = ldexpf(16777216.0f, static_cast<int>(eo));  // the codes' 2^-24 and the unit undone
      // value code operands of tile t: record 16 a + col, words V0 (tokens 4a, 4a + 1) and V1 (4a + 2, 4a + 3),
      // bits 2 (t % 4) (+16), tiles 4..7 in the upper byte: codes times 4^(t % 4)
      const uint32_t vw[4] = {P.rec[2], P.rec[3], P.rec[2] >> 8, P.rec[3] >> 8};
#pragma unroll
      for (int Q = 0; Q < kNQ; ++Q) {
        float x[4];
        half4 xh, xl;
        float zq = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = pq[Q][i] * sv[i] * unit_in;
          xh[i] = static_cast<_Float16>(x[i]);
          xl[i] = static_cast<_Float16>(x[i] - static_cast<float>(xh[i]));
          zq = fmaf(pq[Q][i], zv[i], zq);
        }
        z_run[Q] += rows_sum(zq);  // lane (., grp, jj): sum of p~ z_v over the page for (head 4Q + jj, grp)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t m = 0x00030003u << (2 * (t & 3));
          uint32_t w2[2] = {vw[2 * (t >> 2)] & m, vw[2 * (t >> 2) + 1] & m};
          const half4 cB = __builtin_bit_cast(half4, w2);
          float4v pc = {0.0f, 0.0f, 0.0f, 0.0f};
          pc = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, cB, pc, 0, 0, 0);
          pc = __builtin_amdgcn_mfma_f32_16x16x16f16(xl, cB, pc, 0, 0, 0);
          const float fct = unit_out * (1.0f / static_cast<float>(1 << (2 * (t & 3))));
#pragma unroll
          for (int i = 0; i < 4; ++i) accC[Q][t][i] = fmaf(pc[i], fct, accC[Q][t][i]);
        }
      }
      wave_sync();  // staging free for the next page
      cur = nxt;
    }

    // ---- this wave's rows of s_mw
    __syncthreads();  // every wave is done with its staging (s_mw overlays it)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = 4 * a + i;  // accA / accB row
      if (a < kNQ && hd < g) {
        float* row = s_mw + (wave * kNH + hd) * kWRow;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          row[16 * t + col] = accA[t][i];
          row[kHeadDim + 16 * t + col] = accB[t][i];
        }
      }
    }
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // zero part of head 4 Q + i, group a: lane 4 a + i
        float zi = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = lane_val(z_run[Q], 4 * k + i);
          zi = a == k ? v : zi;
        }
        const int hd = 4 * Q + i;
        if (hd < g) {
          float* row = s_mw + (wave * kNH + hd) * kWRow + 2 * kHeadDim;
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if ((t >> 1) == a) row[16 * t + col] = accC[Q][t][i] + zi;
        }
      }
      if (lane < 4 && 4 * Q + lane < g) {
        float* row = s_mw + (wave * kNH + 4 * Q + lane) * kWRow + 3 * kHeadDim;
        row[2] = m_q[Q];
        row[3] = l_q[Q];
      }
    }
    if (lane < g) {
      float* row = s_mw + (wave * kNH + lane) * kWRow + 3 * kHeadDim;
      row[0] = m_a;
      row[1] = l_a;
    }
    const float e_w = wave_sum(lane < kPage ? e_acc : 0.0f);
    if (lane == 0) s_merr[wave] = e_w;
  }

  __syncthreads();

  float* const part_base = p.part + slot * p.n_splits * kEvHeads * kEvPartStride;
  for (int idx = tid; idx < g * kHeadDim; idx += kEvThreads) {
    const int jj = idx / kHeadDim, c = idx % kHeadDim;
    float Ma = -INFINITY, Mq = -INFINITY;
#pragma unroll
    for (int w = 0; w < kEvWaves; ++w) {
      const float* st4 = s_mw + (w * kNH + jj) * kWRow + 3 * kHeadDim;
      Ma = fmaxf(Ma, st4[0]);
      Mq = fmaxf(Mq, st4[2]);
    }
    float A = 0.0f, B = 0.0f, C = 0.0f, La = 0.0f, Lq = 0.0f;
#pragma unroll
    for (int w = 0; w < kEvWaves; ++w) {
      const float* row = s_mw + (w * kNH + jj) * kWRow;
      const float fa = Ma == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(row[3 * kHeadDim] - Ma);
      const float fq = Mq == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(row[3 * kHeadDim + 2] - Mq);
      A = fmaf(fa, row[c], A);
      B = fmaf(fq, row[kHeadDim + c], B);
      C = fmaf(fq, row[2 * kHeadDim + c], C);
      La = fmaf(fa, row[3 * kHeadDim + 1], La);
      Lq = fmaf(fq, row[3 * kHeadDim + 3], Lq);
    }
    float* dst = part_base + (static_cast<size_t>(split) * g + jj) * kEvPartStride;
    st_ag(dst + c, A);
    st_ag(dst + kHeadDim + c, B);
    st_ag(dst + 2 * kHeadDim + c, C);
    if (c == 0) {
      st_ag(dst + 3 * kHeadDim, Ma);
      st_ag(dst + 3 * kHeadDim + 1, La);
      st_ag(dst + 3 * kHeadDim + 2, Mq);
      st_ag(dst + 3 * kHeadDim + 3, Lq);
      if (jj == 0) st_ag(dst + 3 * kHeadDim + 4, (s_merr[0] + s_merr[1]) + (s_merr[2] + s_merr[3]));
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_ticket = __hip_atomic_fetch_add(p.counters + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != n_valid - 1) return;

  // ---- the last workgroup of (b, h) merges the splits
  float* const s_st = s_buf;                              // [split][head][4]
  float* const s_se = s_buf + n_valid * g * 4;             // [split]
  float* const s_crot = s_se + n_valid;                    // [head][128] C in the rotated basis
  float* const s_oa = s_crot + g * kHeadDim;               // [head][128] A
  float* const s_ob = s_oa + g * kHeadDim;                 // [head][128] B
  static_assert(kMaxEvalSplits * kNH * 4 + kMaxEvalSplits + 3 * kNH * kHeadDim <= kBuf, "split merge fits the buffer");
  for (int idx = tid; idx < n_valid * g; idx += kEvThreads) {
    const float* src = part_base + static_cast<size_t>(idx) * kEvPartStride + 3 * kHeadDim;
#pragma unroll
    for (int e = 0; e < 4; ++e) s_st[4 * idx + e] = ld_ag(src + e);
    if (idx % g == 0) s_se[idx / g] = ld_ag(src + 4);
  }
  __syncthreads();
  for (int idx = tid; idx < g * kHeadDim; idx += kEvThreads) {
    const int jj = idx / kHeadDim, c = idx % kHeadDim;
    float Ma = -INFINITY, Mq = -INFINITY;
    for (int s = 0; s < n_valid; ++s) {
      Ma = fmaxf(Ma, s_st[4 * (s * g + jj)]);
      Mq = fmaxf(Mq, s_st[4 * (s * g + jj) + 2]);
    }
    float A = 0.0f, B = 0.0f, C = 0.0f, La = 0.0f, Lq = 0.0f;
    for (int s = 0; s < n_valid; ++s) {
      const float* st4 = s_st + 4 * (s * g + jj);
      const float fa = Ma == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st4[0] - Ma);
      const float fq = Mq == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st4[2] - Mq);
      const float* row = part_base + (static_cast<size_t>(s) * g + jj) * kEvPartStride;
      A = fmaf(fa, ld_ag(row + c), A);
      B = fmaf(fq, ld_ag(row + kHeadDim + c), B);
      C = fmaf(fq, ld_ag(row + 2 * kHeadDim + c), C);
      La = fmaf(fa, st4[1], La);
      Lq = fmaf(fq, st4[3], Lq);
    }
    s_oa[idx] = La > 0.0f ? A / La : 0.0f;
    s_ob[idx] = Lq > 0.0f ? B / Lq : 0.0f;
    s_crot[idx] = Lq > 0.0f ? C / Lq : 0.0f;
  }
  __syncthreads();
  for (int idx = tid; idx < g * kHeadDim; idx += kEvThreads) {
    const int jj = idx / kHeadDim, i = idx % kHeadDim;
    float C = 0.0f;  // (C_rot R_V^T)_i = sum_c C_rot[c] R_V[i][c]
    for (int c = 0; c < kHeadDim; ++c) C = fmaf(s_crot[jj * kHeadDim + c], rot_elem(p.r_v, p.rot_kind, h, i, c), C);
    float* d = p.dobuf + (row_j0 + jj) * 2 * kHeadDim;
    d[i] = s_ob[idx] - s_oa[idx];     // key-induced: B - A
    d[kHeadDim + i] = C - s_ob[idx];  // value-induced: C - B
  }
  if (tid == 0) {
    float e = 0.0f;
    for (int s = 0; s < n_valid; ++s) e += s_se[s];
    if (hc == 0) p.e_rec[b * H + h] = p.sq_err != nullptr ? e : 0.0f;
    __hip_atomic_store(p.counters + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// dy = dO W_O,j^T for every sequence: workgroup (head j, chunk of kProjRows rows
// of W_O), one thread per row r reading its 128 weights (a 256 or 512 B
// contiguous run; a wave's 64 runs stay in L1 while it walks them) against dO
// rows broadcast from LDS, so no cross-lane sums are needed and dy stores are
// coalesced.  E_out = ||dy_K + dy_V||^2: per-chunk sums, added in chunk order by
// the last workgroup of head j.
template <bool kWF32>
__global__ __launch_bounds__(kEvThreads) void eval_project_kernel(const EvalParams p) {
  static_assert(kProjRows == kEvThreads, "one row per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = blockIdx.x;
  const int chunk = blockIdx.y;
  const int Hq = p.num_q_heads;
  const int B = p.batch;
  __shared__ float s_do[kMaxEvalBatch][2 * kHeadDim];
  __shared__ float s_e[kEvWaves][kMaxEvalBatch];
  __shared__ int s_ticket;
  for (int idx = tid; idx < B * 2 * kHeadDim; idx += kEvThreads) {
    const int bb = idx / (2 * kHeadDim), c = idx % (2 * kHeadDim);
    s_do[bb][c] = p.dobuf[(static_cast<size_t>(bb) * Hq + j) * 2 * kHeadDim + c];
  }
  __syncthreads();
  const int r = chunk * kProjRows + tid;
  const bool live = r < p.d_model;
  const size_t w0i = static_cast<size_t>(live ? r : 0) * Hq * kHeadDim + static_cast<size_t>(j) * kHeadDim;
  for (int bb0 = 0; bb0 < B; bb0 += 4) {  // four sequences per pass over the row
    float ak[4] = {0.0f, 0.0f, 0.0f, 0.0f}, av[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c8 = 0; c8 < kHeadDim / 8; ++c8) {
      float w[8];
      if (kWF32) {
        const float4v a = *reinterpret_cast<const float4v*>(static_cast<const float*>(p.w_o) + w0i + 8 * c8);
        const float4v b = *reinterpret_cast<const float4v*>(static_cast<const float*>(p.w_o) + w0i + 8 * c8 + 4);
        for (int e = 0; e < 4; ++e) {
          w[e] = a[e];
          w[4 + e] = b[e];
        }
      } else {
        const uint4v a = *reinterpret_cast<const uint4v*>(static_cast<const uint16_t*>(p.w_o) + w0i + 8 * c8);
        for (int e = 0; e < 4; ++e) {
          w[2 * e] = __uint_as_float(a[e] << 16);
          w[2 * e + 1] = __uint_as_float(a[e] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (bb0 + u < B) {
          const float* dk = s_do[bb0 + u] + 8 * c8;
          const float* dv = s_do[bb0 + u] + kHeadDim + 8 * c8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ak[u] = fmaf(dk[e], w[e], ak[u]);
            av[u] = fmaf(dv[e], w[e], av[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bb = bb0 + u;
      if (bb < B) {
        if (live) {
          const size_t oi = (static_cast<size_t>(bb) * Hq + j) * p.d_model + r;
          p.dy_k[oi] = ak[u];
          p.dy_v[oi] = av[u];
        }
        const float dy = ak[u] + av[u];
        const float e = wave_sum(live ? dy * dy : 0.0f);
        if (lane == 0) s_e[wave][bb] = e;
      }
    }
  }
  __syncthreads();
  float* const e_chunk = p.e_chunk + static_cast<size_t>(j) * p.n_chunks * kMaxEvalBatch;
  if (tid < B) st_ag(e_chunk + static_cast<size_t>(chunk) * kMaxEvalBatch + tid,
                     (s_e[0][tid] + s_e[1][tid]) + (s_e[2][tid] + s_e[3][tid]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_ticket = __hip_atomic_fetch_add(p.proj_counters + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != p.n_chunks - 1) return;
  if (tid < B) {
    float e = 0.0f;
    for (int ch = 0; ch < p.n_chunks; ++ch) e += ld_ag(e_chunk + static_cast<size_t>(ch) * kMaxEvalBatch + tid);
    p.e_out[static_cast<size_t>(tid) * Hq + j] = e;
  }
  if (tid == 0) __hip_atomic_store(p.proj_counters + j, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int kNH, int kPlanes>
hipError_t launch_attn(const EvalParams& p, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads * p.n_splits, p.batch, (p.g + kEvHeads - 1) / kEvHeads);
  if (p.kv_kind == 1)
    hipLaunchKernelGGL((eval_attn_kernel<kNH, true, kPlanes, false>), grid, dim3(kEvThreads), 0, stream, p);
  else if constexpr (kPlanes == 0)
    hipLaunchKernelGGL((eval_attn_kernel<kNH, false, 0, true>), grid, dim3(kEvThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((eval_attn_kernel<kNH, false, kPlanes, false>), grid, dim3(kEvThreads), 0, stream, p);
  return hipGetLastError();
}

template <int kPlanes>
hipError_t launch_attn_g(const EvalParams& p, hipStream_t stream) {
  return p.g <= 4 ? launch_attn<4, kPlanes>(p, stream) : launch_attn<kEvHeads, kPlanes>(p, stream);
}

}  // namespace

hipError_t launch_eval(const EvalParams& p, hipStream_t stream) {
  (void)hipGetLastError();  // report only this call's launch errors
  const int planes = (p.kbits > 2) + (p.vbits > 2);  // 3- and 4-bit codes of a tensor share one block layout
  hipError_t e = planes == 0 ? launch_attn_g<0>(p, stream)
                             : (planes == 1 ? launch_attn_g<1>(p, stream) : launch_attn_g<2>(p, stream));
  if (e != hipSuccess) return e;
  const dim3 pgrid(p.num_q_heads, p.n_chunks);
  if (p.w_kind == 1)
    hipLaunchKernelGGL(eval_project_kernel<true>, pgrid, dim3(kEvThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(eval_project_kernel<false>, pgrid, dim3(kEvThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
