// Decode attention read straight from the packed INT2 cache.
//
// OptR ("Output-Oriented Rotation for INT2 KV-Cache Quantization"), section 3,
// Eq. (1)-(2) and section 3.2, Eq. (5): softmax attention of each query head
// over the effective (dequantized) keys and values of its KV head.  Since the
// cache holds Q2(zR) and R is orthogonal, the query is rotated once
// (q_hat = q R_K), logits are <q_hat, x_hat_s>, the value sum is formed in the
// rotated basis and mapped back once with R_V^T (section 3.1, Eq. (4)).
//
// Three kernels per call:
//   qrot_kernel   q_hat = q R_K * sm_scale * log2(e)  (fp32), plus a power of
//                 two that brings max|q_hat| into [2^13, 2^14) for fp16.
//   split_kernel  one workgroup (4 waves) per (split, KV head, sequence); each
//                 wave streams page pairs, forms logits and the P.V product on
//                 the matrix cores, keeps an online softmax, and the waves
//                 merge through LDS into one partial (max, sum, acc[128]).
//   merge_kernel  log-sum-exp merge of the partials, divide, o = o_rot R_V^T.
//
// Logits on the matrix cores (per page, per quad of query heads).  A group's
// dequantized key is z + s*c with codes c in {0..3}, so
//   <q_hat, x_hat> = sum_grp s_grp * <q_hat_grp, c_grp> + z_grp * sum(q_hat_grp).
// The inner products <q_hat_grp, c_grp> come from v_mfma_f32_16x16x32_f16 with
// A = the page's 16 tokens x 32 codes and B = a block-diagonal query operand:
// column n = 4*grp + j holds q_hat_j on group grp's channels and 0 elsewhere,
// so the four chunks of 32 channels fill all 16 columns.  Codes enter as the
// raw fp16 bit patterns c (subnormals c * 2^-24, exact in the MFMA); the
// query enters as an fp16 hi/lo pair of q_hat * 2^k, so the products carry
// about 22 bits.  The per-group scale/zero are applied in fp32 and the 4
// groups summed with two DPP row rotations.
// P.V on the matrix cores (per page pair).  A = p * s_v as fp16 with rows
// n = 4*grp + j and 32 token columns (the 2 x 16 tokens the lane already
// holds), B = value codes (subnormal bit patterns) of 32 tokens x 16 channels;
// rows whose group does not own the tile's channels are discarded.  The
// zero-point part sum_s p_s z_v,s is accumulated in fp32.

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima
constexpr float kTwo24 = 16777216.0f;

// --------------------------------------------------------------- q rotation
template <int kQIn>  // 0 bf16, 1 fp32
__global__ __launch_bounds__(128) void qrot_kernel(const void* __restrict__ q, const float* __restrict__ r_k,
                                                   int num_q_heads, int g, float logit_scale,
                                                   float* __restrict__ qhat) {
  const int row = blockIdx.x;  // b * num_q_heads + j
  const int j = row % num_q_heads;
  const int h = j / g;
  const int c = threadIdx.x;
  __shared__ float qs[kHeadDim];
  __shared__ float wmax[2];
  const size_t base = static_cast<size_t>(row) * kHeadDim;
  qs[c] = kQIn == 0 ? bf16_bits_to_f32(static_cast<const uint16_t*>(q)[base + c]) : static_cast<const float*>(q)[base + c];
  __syncthreads();
  const float* R = r_k + static_cast<size_t>(h) * kHeadDim * kHeadDim;
  float acc = 0.0f;
  for (int i = 0; i < kHeadDim; ++i) acc = fmaf(qs[i], R[i * kHeadDim + c], acc);
  acc *= logit_scale;
  float am = fabsf(acc);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((c & 63) == 0) wmax[c >> 6] = am;
  __syncthreads();
  am = fmaxf(wmax[0], wmax[1]);
  float* dst = qhat + static_cast<size_t>(row) * kQhatStride;
  dst[c] = acc;
  if (c == 0) {
    int e = 0;
    frexpf(am, &e);  // am in [2^(e-1), 2^e)
    dst[128] = am > 0.0f ? ldexpf(1.0f, 14 - e) : 1.0f;
  }
}

// ------------------------------------------------------------- split kernel
template <int kNQ>  // quads of query heads per KV head: g <= 4 * kNQ
__global__ __launch_bounds__(256) void split_kernel(const uint8_t* __restrict__ pool, int num_kv_heads,
                                                    int num_pages, const float* __restrict__ qhat,
                                                    const int32_t* __restrict__ page_table, int max_pages,
                                                    const int32_t* __restrict__ seq_lens, int num_q_heads, int g,
                                                    int pages_per_split, int n_splits, float* __restrict__ part) {
  constexpr int kNH = 4 * kNQ;
  __shared__ float s_acc[4][kNH][kHeadDim];
  __shared__ float s_m[4][kNH];
  __shared__ float s_l[4][kNH];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  // Pages past the table row are never read (a length beyond max_pages*16 is cut).
  const int T = min(seq_lens[b], max_pages * kPage);
  const int n_pages = (T + kPage - 1) / kPage;
  const int p0 = split * pages_per_split;
  if (p0 >= n_pages) return;  // whole workgroup
  const int p1 = min(p0 + pages_per_split, n_pages);
  const int npairs = (p1 - p0 + 1) >> 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int a = lane >> 4;    // row of 16 lanes: token quad (QK) / channel octet
  const int col = lane & 15;  // MFMA column: 4*grp + jj
  const int grp = col >> 2;
  const int jj = col & 3;

  // ---- block-diagonal query operands (fp16 hi/lo of q_hat * f)
  half8 qhi[kNQ][4], qlo[kNQ][4];
  float qz[kNQ], c1[kNQ];
#pragma unroll
  for (int Q = 0; Q < kNQ; ++Q) {
    const int jl = 4 * Q + jj;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = 0.0f;
    float f = 1.0f;
    if (jl < g) {
      const float* row = qhat + (static_cast<size_t>(b) * num_q_heads + h * g + jl) * kQhatStride;
      f = row[128];
      const float4v u0 = *reinterpret_cast<const float4v*>(row + 32 * grp + 8 * a);
      const float4v u1 = *reinterpret_cast<const float4v*>(row + 32 * grp + 8 * a + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[e] = u0[e];
        qv[e + 4] = u1[e];
      }
    }
    half8 hi, lo;
    float qsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sc = qv[e] * f;
      const _Float16 hh = static_cast<_Float16>(sc);
      hi[e] = hh;
      lo[e] = static_cast<_Float16>(sc - static_cast<float>(hh));
      qsum += qv[e];
    }
    qsum = rows_sum(qsum);  // sum of q_hat over group grp's 32 channels
    c1[Q] = kTwo24 / f;
    qz[Q] = qsum / c1[Q];
    const half8 zero = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qhi[Q][kk] = (grp == kk) ? hi : zero;
      qlo[Q][kk] = (grp == kk) ? lo : zero;
    }
  }

  float m_run[kNQ], l_run[kNQ], z_run[kNQ];
  float4v acc[kNQ][8];
#pragma unroll
  for (int Q = 0; Q < kNQ; ++Q) {
    m_run[Q] = kNegBig;
    l_run[Q] = 0.0f;
    z_run[Q] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[Q][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int32_t* pt = page_table + static_cast<size_t>(b) * max_pages;
  const int meta_off = kCodeBytes + kMetaRecordBytes * (4 * grp + a);

  for (int pair = wave; pair < npairs; pair += 4) {
    const int lp0 = p0 + 2 * pair;
    int ph0 = pt[lp0];
    int ph1 = lp0 + 1 < p1 ? pt[lp0 + 1] : ph0;
    // A page id outside the pool is read as page 0 and all its tokens are masked.
    const bool ok0 = ph0 >= 0 && ph0 < num_pages;
    const bool has1 = lp0 + 1 < p1 && ph1 >= 0 && ph1 < num_pages;
    ph0 = ok0 ? ph0 : 0;
    ph1 = has1 ? ph1 : ph0;
    const uint8_t* blk0 = pool + (static_cast<size_t>(ph0) * num_kv_heads + h) * kBlockBytes;
    const uint8_t* blk1 = pool + (static_cast<size_t>(ph1) * num_kv_heads + h) * kBlockBytes;
    const uint4v rec0 = *reinterpret_cast<const uint4v*>(blk0 + 16 * lane);
    const uint4v rec1 = *reinterpret_cast<const uint4v*>(blk1 + 16 * lane);
    const uint4v km0 = *reinterpret_cast<const uint4v*>(blk0 + meta_off);
    const uint4v vm0 = *reinterpret_cast<const uint4v*>(blk0 + meta_off + 16);
    const uint4v km1 = *reinterpret_cast<const uint4v*>(blk1 + meta_off);
    const uint4v vm1 = *reinterpret_cast<const uint4v*>(blk1 + meta_off + 16);

    // ---- logits (log2 units, divided by c1) for both pages
    float sp[kNQ][2][4];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const uint4v rec = X ? rec1 : rec0;
      const uint4v km = X ? km1 : km0;
      half8 kA[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t w = kk < 2 ? rec[0] : rec[1];
        const int sh = 8 * (kk & 1);
        uint4v r;
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = (w >> (sh + 2 * q)) & 0x00030003u;
        kA[kk] = __builtin_bit_cast(half8, r);
      }
      float sk[4], zk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sk[i] = f16_lo(km[i]);
        zk[i] = f16_hi(km[i]);
      }
      const int pos0 = (lp0 + X) * kPage + 4 * a;
      const bool page_ok = X == 0 ? ok0 : has1;
#pragma unroll
      for (int Q = 0; Q < kNQ; ++Q) {
        float4v C = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          C = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qhi[Q][kk], C, 0, 0, 0);
          C = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qlo[Q][kk], C, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = fmaf(C[i], sk[i], zk[i] * qz[Q]);
          s = row_sum_stride4(s);
          sp[Q][X][i] = (page_ok && pos0 + i < T) ? s : -INFINITY;
        }
      }
    }

    // ---- value operands: tile t holds channels 16t..16t+15
    half8 vB[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint4v r;
      r[0] = (rec0[2] >> (2 * t)) & 0x00030003u;
      r[1] = (rec0[3] >> (2 * t)) & 0x00030003u;
      r[2] = (rec1[2] >> (2 * t)) & 0x00030003u;
      r[3] = (rec1[3] >> (2 * t)) & 0x00030003u;
      vB[t] = __builtin_bit_cast(half8, r);
    }
    float sv[2][4], zv[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[0][i] = f16_lo(vm0[i]);
      zv[0][i] = f16_hi(vm0[i]);
      sv[1][i] = f16_lo(vm1[i]);
      zv[1][i] = f16_hi(vm1[i]);
    }

    // ---- online softmax and P.V per quad
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      float mloc = -INFINITY;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sp[Q][X][i]);
      mloc = rows_max(mloc);
      const float m_new = fmaxf(m_run[Q], mloc * c1[Q]);
      if (__ballot(m_new > m_run[Q]) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[Q] - m_new);
        const float al0 = dpp_f32<QuadBcast<0>::ctrl>(alpha);
        const float al1 = dpp_f32<QuadBcast<1>::ctrl>(alpha);
        const float al2 = dpp_f32<QuadBcast<2>::ctrl>(alpha);
        const float al3 = dpp_f32<QuadBcast<3>::ctrl>(alpha);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          acc[Q][t][0] *= al0;
          acc[Q][t][1] *= al1;
          acc[Q][t][2] *= al2;
          acc[Q][t][3] *= al3;
        }
        l_run[Q] *= alpha;
        z_run[Q] *= alpha;
        m_run[Q] = m_new;
      }
      float pv[2][4];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sp[Q][X][i], c1[Q], -m_run[Q]));
          l_run[Q] += p;
          z_run[Q] = fmaf(p, zv[X][i], z_run[Q]);
          pv[X][i] = p * sv[X][i];
        }
      half8 pA;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) pA[4 * X + i] = static_cast<_Float16>(pv[X][i]);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[Q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pA, vB[t], acc[Q][t], 0, 0, 0);
    }
  }

  // ---- per-wave results to LDS: lane (a, b) owns channels 32a + b and
  //      32a + 16 + b (tiles 2a, 2a+1) for the four heads of each quad.
#pragma unroll
  for (int Q = 0; Q < kNQ; ++Q) {
    const float lsum = rows_sum(l_run[Q]);
    const float zsum = rows_sum(z_run[Q]);  // lane (., grp, jj): sum_s p z_v for (jj, grp)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float zi = __shfl(zsum, 4 * a + i);  // zero part of head i, group a
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if ((t >> 1) == a) s_acc[wave][4 * Q + i][16 * t + col] = acc[Q][t][i] * kTwo24 + zi;
      }
    }
    if (lane < 4) {
      s_m[wave][4 * Q + lane] = m_run[Q];
      s_l[wave][4 * Q + lane] = lsum;
    }
  }
  __syncthreads();

  for (int idx = tid; idx < kNH * kHeadDim; idx += 256) {
    const int jh = idx / kHeadDim;
    const int c = idx % kHeadDim;
    if (jh >= g) continue;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][jh]);
    float av = 0.0f, lv = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = __builtin_amdgcn_exp2f(s_m[w][jh] - M);
      av = fmaf(wt, s_acc[w][jh][c], av);
      lv = fmaf(wt, s_l[w][jh], lv);
    }
    float* dst = part + ((static_cast<size_t>(b) * num_q_heads + h * g + jh) * n_splits + split) * kPartStride;
    dst[c] = av;
    if (c == 0) {
      dst[128] = M;
      dst[129] = lv;
    }
  }
}

// ------------------------------------------------------------- merge kernel
template <int kOut>  // 0 bf16, 1 fp32
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    const int32_t* __restrict__ seq_lens, int max_pages,
                                                    int num_q_heads, int g,
                                                    int pages_per_split, int n_splits, const float* __restrict__ r_v,
                                                    void* __restrict__ out) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ float so[16][kHeadDim];
  const int T = min(seq_lens[b], max_pages * kPage);
  const int n_pages = (T + kPage - 1) / kPage;
  const int nval = min(n_splits, (n_pages + pages_per_split - 1) / pages_per_split);

  for (int idx = tid; idx < g * kHeadDim; idx += 256) {
    const int jh = idx / kHeadDim;
    const int c = idx % kHeadDim;
    const float* src = part + (static_cast<size_t>(b) * num_q_heads + h * g + jh) * n_splits * kPartStride;
    float M = kNegBig;
    for (int s = 0; s < nval; ++s) M = fmaxf(M, src[s * kPartStride + 128]);
    float av = 0.0f, lv = 0.0f;
    for (int s = 0; s < nval; ++s) {
      const float wt = __builtin_amdgcn_exp2f(src[s * kPartStride + 128] - M);
      av = fmaf(wt, src[s * kPartStride + c], av);
      lv = fmaf(wt, src[s * kPartStride + 129], lv);
    }
    so[jh][c] = lv > 0.0f ? av / lv : 0.0f;
  }
  __syncthreads();

  if (tid < kHeadDim) {
    const int i = tid;  // output channel: o[i] = sum_c o_rot[c] * R_V[i][c]
    const float* Rrow = r_v + (static_cast<size_t>(h) * kHeadDim + i) * kHeadDim;
    float o[16];
#pragma unroll
    for (int jh = 0; jh < 16; ++jh) o[jh] = 0.0f;
    for (int c = 0; c < kHeadDim; c += 4) {
      const float4v r4 = *reinterpret_cast<const float4v*>(Rrow + c);
#pragma unroll
      for (int jh = 0; jh < 16; ++jh) {
        if (jh < g) {
          o[jh] = fmaf(so[jh][c + 0], r4[0], o[jh]);
          o[jh] = fmaf(so[jh][c + 1], r4[1], o[jh]);
          o[jh] = fmaf(so[jh][c + 2], r4[2], o[jh]);
          o[jh] = fmaf(so[jh][c + 3], r4[3], o[jh]);
        }
      }
    }
#pragma unroll
    for (int jh = 0; jh < 16; ++jh) {
      if (jh < g) {
        const size_t oi = (static_cast<size_t>(b) * num_q_heads + h * g + jh) * kHeadDim + i;
        if (kOut == 0)
          static_cast<uint16_t*>(out)[oi] = f32_to_bf16_bits(o[jh]);
        else
          static_cast<float*>(out)[oi] = o[jh];
      }
    }
  }
}

// ----------------------------------------------------------------- launcher
template <int kNQ>
static void launch_split(const DecodeArgs& a, const DecodePlan& plan, int g, hipStream_t stream) {
  const dim3 grid(plan.n_splits, a.num_kv_heads, a.batch);
  hipLaunchKernelGGL(split_kernel<kNQ>, grid, dim3(256), 0, stream, a.pool, a.num_kv_heads, a.num_pages, a.qhat,
                     a.page_table,
                     a.max_pages, a.seq_lens, a.num_q_heads, g, plan.pages_per_split, plan.n_splits, a.part);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream, hipEvent_t ev_begin,
                         hipEvent_t ev_end) {
  const int g = a.num_q_heads / a.num_kv_heads;
  (void)hipGetLastError();  // report only this call's launch errors, not stale ones
  const dim3 qgrid(a.batch * a.num_q_heads);
  if (a.q_kind == 0)
    hipLaunchKernelGGL(qrot_kernel<0>, qgrid, dim3(128), 0, stream, a.q, a.r_k, a.num_q_heads, g, a.logit_scale,
                       a.qhat);
  else
    hipLaunchKernelGGL(qrot_kernel<1>, qgrid, dim3(128), 0, stream, a.q, a.r_k, a.num_q_heads, g, a.logit_scale,
                       a.qhat);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (ev_begin != nullptr && (err = hipEventRecord(ev_begin, stream)) != hipSuccess) return err;
  if (g <= 4)
    launch_split<1>(a, plan, g, stream);
  else if (g <= 8)
    launch_split<2>(a, plan, g, stream);
  else
    launch_split<4>(a, plan, g, stream);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev_end != nullptr && (err = hipEventRecord(ev_end, stream)) != hipSuccess) return err;

  const dim3 mgrid(a.num_kv_heads, a.batch);
  if (a.out_kind == 0)
    hipLaunchKernelGGL(merge_kernel<0>, mgrid, dim3(256), 0, stream, a.part, a.seq_lens, a.max_pages, a.num_q_heads, g,
                       plan.pages_per_split, plan.n_splits, a.r_v, a.out);
  else
    hipLaunchKernelGGL(merge_kernel<1>, mgrid, dim3(256), 0, stream, a.part, a.seq_lens, a.max_pages, a.num_q_heads, g,
                       plan.pages_per_split, plan.n_splits, a.r_v, a.out);
  return hipGetLastError();
}

}  // namespace kvq
