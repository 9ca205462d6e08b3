// Decode attention read straight from the packed INT2 cache, in one kernel.
//
// OptR ("Output-Oriented Rotation for INT2 KV-Cache Quantization"), section 3,
// Eq. (1)-(2) and section 3.2, Eq. (5): softmax attention of each query head
// over the effective (dequantized) keys and values of its KV head.  Since the
// cache holds Q2(zR) and R is orthogonal, the query is rotated once
// (q_hat = q R_K), logits are <q_hat, x_hat_s>, the value sum is formed in the
// rotated basis and mapped back once with R_V^T (section 3.1, Eq. (4)).
//
// Work decomposition.  One workgroup of kW waves per (split, KV head h,
// sequence b), sized so that one workgroup fills a compute unit; a split is a
// contiguous range of the sequence's pages.  The workgroups of one KV head are
// consecutive in the flattened grid with h fastest, so on an 8-XCD part the
// workgroups of one KV head share an XCD's L2.
//   prologue   load the split's page ids, the g query rows and R_K together
//              (with the sequence length, from a guess of the split where one
//              exists); start streaming the first page pair; compute
//              q_hat = q R_K * sm_scale * log2(e) (fp32) and a per-head power
//              of two f that brings max|q_hat*f| into [2^13, 2^14); request
//              the next pairs.
//   main loop  wave w takes page pairs w, w+kW, ...: each pair is copied by
//              direct global->LDS loads into a ring of kDepth slots per wave
//              (kDepth - 1 pairs in flight while one is computed); logits and
//              P.V run on the matrix cores, the online softmax in fp32.
//   epilogue   the kW waves merge through LDS into one partial (max, sum,
//              acc[128]) stored to the workspace with agent-scope (cross-XCD
//              coherent) stores; the last workgroup of the (sequence, KV head)
//              (atomic ticket) merges all partials with log-sum-exp weights,
//              divides, applies R_V^T and stores the output.
//
// Logits on the matrix cores (per page, per quad of query heads).  A group's
// dequantized key is z + s*c with codes c in {0..3}, so
//   <q_hat, x_hat> = sum_grp s_grp * <q_hat_grp, c_grp> + z_grp * sum(q_hat_grp).
// The inner products <q_hat_grp, c_grp> come from v_mfma_f32_16x16x32_f16 with
// A = the page's 16 tokens x 32 codes and B = a block-diagonal query operand:
// column n = 4*grp + j holds q_hat_j on group grp's channels and 0 elsewhere,
// so the four chunks of 32 channels fill all 16 columns.  Codes enter as the
// raw fp16 bit patterns c (subnormals c * 2^-24, exact in the MFMA); the
// query enters as an fp16 hi/lo pair of q_hat * f, so the products carry
// about 22 bits.  The per-group scale/zero are applied in fp32 and the 4
// groups summed with two DPP row rotations.
// P.V on the matrix cores (per page pair).  A = p * s_v as fp16 with rows
// n = 4*grp + j and 32 token columns (the 2 x 16 tokens the lane already
// holds), B = value codes (subnormal bit patterns) of 32 tokens x 16 channels;
// rows whose group does not own the tile's channels are discarded.  The
// zero-point part sum_s p_s z_v,s is accumulated in fp32.
// For g = 5..8 one octet layout replaces the two quads: column (row)
// n = 8*h + j is head j on the groups h and h + 2.  The logits take two
// accumulators per page (groups 0-1 and 2-3, half the columns of each
// product live) summed across the column halves by one DPP rotation, and
// P.V one A operand per group half (tiles 0-3 and 4-7): 24 products per
// page pair for eight heads instead of 48.  For g = 9..16 the hexadeca
// layout makes every column a head: four logit accumulators per page (one
// per group, all columns live) and one P.V operand per group, 24 products
// per page pair for sixteen heads instead of 96.

#pragma once

#include <hip/hip_ext.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {

constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima
constexpr float kTwo24 = 16777216.0f;
constexpr float kLazy = 8.0f;  // rescale threshold of the online softmax (log2 units)
// DMA instructions per page pair: K/V codes of page 0, of page 1; metadata of
// page 0, of page 1; with 3- or 4-bit keys (values) also the keys' (values')
// high-bit planes of pages 0 and 1.
template <bool kKW, bool kVW> struct PairDma { static constexpr int n = 4 + 2 * kKW + 2 * kVW; };

// Launch shape by the number of head quads and of ring parts per page pair (3
// for 2-bit codes, one more per high-bit plane): waves per workgroup (a
// quarter of them per SIMD) and the per-wave ring depth (page pairs staged in
// LDS by direct global->LDS loads; depth - 1 pairs are in flight while one is
// computed).  The g <= 4 kernel fits 3 waves per SIMD, so one 12-wave
// workgroup fills a compute unit, while its ring fits the LDS (up to one
// plane); so does g <= 8 with 2-bit codes (the octet layout's 168 registers),
// and with a plane 2 per SIMD; g <= 16 with 2-bit codes runs 2 per SIMD (the
// hexadeca layout), with a plane 1 per SIMD and more pairs in flight per wave.
template <int kNQ, int kParts> struct DecodeShape {
  static constexpr int waves = kParts == 3 ? 8 : 4, depth = kParts == 3 ? 4 : 6;
};
template <int kParts> struct DecodeShape<1, kParts> { static constexpr int waves = kParts <= 4 ? 12 : 8, depth = 3; };
template <int kParts> struct DecodeShape<2, kParts> {
  static constexpr int waves = kParts == 3 ? 12 : 8, depth = kParts == 3 ? 3 : (kParts <= 4 ? 4 : 3);
};
// The narrow shape for batches of g <= 4 with 2-bit codes and no window: three
// 4-wave workgroups per compute unit (the same 3 waves per SIMD and per-wave
// ring).  Three times the splits per KV head cut each sequence's pages more
// finely, so the largest split, which sets the kernel's length when lengths
// differ, sits closer to the mean.
constexpr int kNarrowWaves = 4, kNarrowDepth = 3, kNarrowWgPerCu = 3;

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16 bytes per lane from global memory straight into LDS: lane l reads
// base + voff (base wave-uniform, in SGPRs) and its bytes land at lds + 16*l
// (global_load_lds_dwordx4, LDS base in M0).  Issued as inline asm so the
// compiler adds none of its own (whole-queue) waits for it; every read of a
// ring slot is preceded by an explicit vmcnt wait instead.  The page stream is
// read once per call, so it carries the non-temporal hint (nt): it displaces
// less of what the L2 holds for the call's prologue and merge (R, page table,
// partial rows, code).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, void* lds) {
  const uint32_t lds_addr =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(lds))));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// dma16 with the cache policy of an agent-scope load (sc1): reads what other
// workgroups stored with agent-scope stores, as ld_agent does.
__device__ __forceinline__ void dma16_agent(const uint8_t* base, uint32_t voff, void* lds) {
  const uint32_t lds_addr =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(lds))));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 sc1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kN) : "memory");
}

struct PagePair {
  uint4v rec0, rec1, km0, vm0, km1, vm1;
};

// Sum of v over the workgroup, returned to every thread (s_red: kW ints).
template <int kW>
__device__ __forceinline__ int block_sum(int v, int lane, int wave, int* s_red) {
  v = wave_sum_int(v);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) t += s_red[w];
  __syncthreads();  // s_red is free again
  return t;
}

// Exclusive prefix sum of v in thread order; `total` receives the sum.
template <int kW>
__device__ __forceinline__ int block_excl_scan(int v, int lane, int wave, int* s_red, int& total) {
  // inclusive scan inside each 16-lane row (DPP row shifts; lanes shifted in from outside the row add 0),
  // then the totals of the rows before the lane's, read from lanes 15, 31, 47
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  if (lane == 63) s_red[wave] = x;
  __syncthreads();
  int before = 0, t = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int c = s_red[w];
    before += w < wave ? c : 0;
    t += c;
  }
  __syncthreads();
  total = t;
  return before + x - v;
}

__device__ __forceinline__ int seq_pages(const DecodeParams& p, int b) {
  const int T = min(p.seq_lens[b], p.len_cap);
  return T > 0 ? (T + kPage - 1) / kPage : 0;
}

// Balanced plan: the split of work slot w (of one KV head).  Every sequence b
// takes max(1, ceil(pages_b / pps)) consecutive slots, in sequence order, with
// pps sized from the batch's total pages; a slot past the last split gets b = -1.
struct SplitLoc {
  int b, split, pps, first;  // first = slot of split 0 of sequence b
  int len;                   // batch 1: seq_lens[0] as read (else unset)
};
template <int kW>
__device__ SplitLoc locate_split(const DecodeParams& p, int w, int tid, int lane, int wave, int* s_red, int* s_loc) {
  constexpr int kThreads = 64 * kW;
  auto pps_for = [&](int total_pages) {
    const long long want = (static_cast<long long>(p.num_kv_heads) * total_pages + p.target_wgs - 1) / p.target_wgs;
    return static_cast<int>(min(max(want, static_cast<long long>(p.pps_min)), static_cast<long long>(p.pps_max)));
  };
  SplitLoc r;
  if (p.batch == 1) {  // no scan needed
    r.len = p.seq_lens[0];
    const int T0 = min(r.len, p.len_cap);
    const int pages = T0 > 0 ? (T0 + kPage - 1) / kPage : 0;
    r.pps = step_pages_per_split(pages, pps_for(pages), p.pps_max, (p.k_new != nullptr) + (p.win != nullptr));
    const int n = max(1, (pages + r.pps - 1) / r.pps);
    r.b = w < n ? 0 : -1;
    r.split = w;
    r.first = 0;
    return r;
  }
  const int pages0 = tid < p.batch ? seq_pages(p, tid) : 0;  // first chunk, kept for the later passes
  int tot = pages0;
  for (int c = kThreads; c < p.batch; c += kThreads) tot += c + tid < p.batch ? seq_pages(p, c + tid) : 0;
  r.pps = pps_for(block_sum<kW>(tot, lane, wave, s_red));
  // Each sequence's last split is partial, so the split count can exceed the
  // target; grow pps (proportionally, a few rounds) until every split of the
  // batch has a workgroup slot in the first round of the grid.  The smallest
  // such pps minimises the largest split.
  auto n_splits_at = [&](int pps) {
    int n = tid < p.batch ? max(1, (pages0 + pps - 1) / pps) : 0;
    for (int c = kThreads; c < p.batch; c += kThreads)
      n += c + tid < p.batch ? max(1, (seq_pages(p, c + tid) + pps - 1) / pps) : 0;
    return block_sum<kW>(n, lane, wave, s_red);
  };
  for (int it = 0; it < 8 && r.pps < p.pps_max; ++it) {
    const long long fill = static_cast<long long>(p.num_kv_heads) * n_splits_at(r.pps);
    if (fill <= p.target_wgs) break;
    const long long next = (static_cast<long long>(r.pps) * fill + p.target_wgs - 1) / p.target_wgs;
    r.pps = static_cast<int>(min(max(next, static_cast<long long>(r.pps) + 1), static_cast<long long>(p.pps_max)));
  }
  if (tid == 0) s_loc[0] = -1;  // ordered before the publishing write by the scan's barriers
  int run = 0;
  for (int c = 0; c < p.batch; c += kThreads) {
    const int i = c + tid;
    const int pages = c == 0 ? pages0 : (i < p.batch ? seq_pages(p, i) : 0);
    const int n = i < p.batch ? max(1, (pages + r.pps - 1) / r.pps) : 0;
    int chunk_total;
    const int excl = run + block_excl_scan<kW>(n, lane, wave, s_red, chunk_total);
    if (w >= excl && w < excl + n) {  // exactly one thread of the batch
      s_loc[0] = i;
      s_loc[1] = w - excl;
      s_loc[2] = excl;
    }
    run += chunk_total;
  }
  __syncthreads();
  r.b = s_loc[0];
  r.split = s_loc[1];
  r.first = s_loc[2];
  return r;
}

// Coherent (agent-scope) load of a value another workgroup stored with an agent-scope store.
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kNQ: g <= 4 * kNQ (1: one quad of heads, 2: the octet layout, 4: the
// hexadeca layout); waves per workgroup, ring depth, 3- or 4-bit keys, 3- or
// 4-bit values, Hadamard rotation, workgroups per compute unit
template <int kNQ, int kW, int kDepth, bool kKW, bool kVW, bool kHad, int kWgPerCu = 1>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kW / 4 * kWgPerCu)))
void decode_kernel(const DecodeParams p) {
  constexpr int kDmaPerPair = PairDma<kKW, kVW>::n;
  // ring parts: codes of page 0, of page 1, metadata, then the keys' and the values' high-bit planes
  constexpr int kRingParts = 3 + kKW + kVW;
  constexpr int kKPart = 3, kVPart = 3 + kKW;
  // the block's size and the offsets of its metadata's end and planes follow
  // the cache format (G, and 3- or 4-bit codes: kvq_device.h)
  const int kBlk = block_bytes(p.kbits, p.vbits, p.gsize);
  const int kKPlane = k_hi_plane(p.gsize);
  const int kVPlane = v_hi_plane(p.kbits, p.gsize);
  static_assert(kDepth >= 2 && kDmaPerPair * (kDepth - 1) <= 63, "ring depth within the vmcnt range");
  constexpr int kNH = 4 * kNQ;
  constexpr int kThreads = 64 * kW;
  // q_hat and the new token's rotation: thread (column rc, part rpart) sums
  // rows [kRows * rpart, +kRows) of R; threads past the last part repeat it.
  constexpr int kParts = kThreads >= 4 * kHeadDim ? 4 : kThreads / kHeadDim;
  constexpr int kRows = kHeadDim / kParts;
  static_assert(kParts >= 2, "at least two row parts");
  __shared__ int s_pages[kMaxPagesPerSplit];
  __shared__ __align__(16) float s_q[kNH][kHeadDim];  // q rows -> q_hat -> o_rot
  __shared__ float s_f[kNH];
  __shared__ float s_m[kW][kNH];
  __shared__ float s_l[kW][kNH];
  __shared__ int s_ticket;
  // step form: the new token's centred (then rotated) key and value rows,
  // dequantized levels and per-head logits
  __shared__ float s_nrow[2][kHeadDim];
  __shared__ float s_hat[2][kHeadDim];
  __shared__ float2 s_nrng[4];  // G = 128: the new token's range per wave
  __shared__ float s_nlog[kNH];
  // Page-pair ring [slot][wave][part][lane]: part 0/1 = 64 x 16 B codes of
  // page 0/1, part 2 = 32 x 16 B metadata of page 0 then of page 1; parts 3
  // and on: the high-bit planes of page 0 then of page 1 (keys', values').
  __shared__ uint4v s_ring[kDepth][kW][kRingParts][64];
  // Prologue scratch (q_hat partials [kParts][kNH][128], then the new token's
  // partials [2][4][128]) lives in the last ring slot, which no load targets
  // before the main loop, when it fits there.  After the main loop the whole
  // ring holds the per-wave partials and then the R_V^T partial sums.
  constexpr int kProFloats = (kParts * kNH + 2 * 4) * kHeadDim;
  constexpr bool kProInRing = kProFloats * 4 <= kW * kRingParts * 64 * 16;
  __shared__ float s_pro_sep[kProInRing ? 1 : kProFloats];
  float* const s_pro = kProInRing ? reinterpret_cast<float*>(&s_ring[kDepth - 1][0][0][0]) : s_pro_sep;
  float* const s_npart = s_pro + kParts * kNH * kHeadDim;
  float* const s_post = reinterpret_cast<float*>(&s_ring[0][0][0][0]);
  static_assert(sizeof(s_ring) >= sizeof(float) * kW * kNH * kHeadDim, "per-wave partials fit in the ring");

  const int H = p.num_kv_heads;
  const int g = p.g;
  const int id = blockIdx.x;
  const int h = id % H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: ring addresses stay scalar
  auto ring = [&](int slot) -> uint4v(*)[64] { return s_ring[slot][wave]; };

  // Loads that depend only on the (sequence, first page) are issued before the
  // length is known, from a guess: exact under a fixed plan, the host's split
  // size for a batch of one (right whenever the length is max_seq_len), none
  // for a larger batch under the automatic plan.  A wrong guess reloads.
  int b_g = -1, p0_g = 0;
  if (!p.balanced) {
    b_g = id / (H * p.n_splits);
    p0_g = ((id / H) % p.n_splits) * p.pages_per_split;
  } else if (p.batch == 1) {
    b_g = 0;
    p0_g = (id / H) * p.pages_per_split;
  }
  const bool stepping = p.k_new != nullptr;
  constexpr int kPidPerThread = (kMaxPagesPerSplit + kThreads - 1) / kThreads;
  constexpr int kQPerThread = (kNH * kHeadDim + kThreads - 1) / kThreads;
  const int rc = tid & (kHeadDim - 1);
  const int rpart = min(tid / kHeadDim, kParts - 1);
  int pid[kPidPerThread];   // page ids of the split (index clamped into the table row)
  uint32_t qraw[kQPerThread];  // q as raw dwords: the bf16 element's dword, or the fp32 element
  uint32_t nraw = 0, muraw = 0;  // step form: the new key / value element, mu
  float rv[kRows], rvv[kRows];   // rows [kRows * rpart, +kRows) of column rc of R_K, R_V
  auto load_pages = [&](int bb, int pp0) {
    const int32_t* pt = p.page_table + static_cast<size_t>(bb) * p.max_pages;
#pragma unroll
    for (int u = 0; u < kPidPerThread; ++u) pid[u] = pt[min(pp0 + tid + u * kThreads, p.max_pages - 1)];
  };
  auto load_seq = [&](int bb) {  // q rows and the new token of sequence bb
    const size_t row0 = static_cast<size_t>(bb) * p.num_q_heads + static_cast<size_t>(h) * g;
#pragma unroll
    for (int u = 0; u < kQPerThread; ++u) {
      const int idx = min(tid + u * kThreads, kNH * kHeadDim - 1);
      const size_t qi = (row0 + min(idx / kHeadDim, g - 1)) * kHeadDim + idx % kHeadDim;
      qraw[u] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.q) +
                                                   (p.q_kind == 0 ? (2 * qi) & ~static_cast<size_t>(3) : 4 * qi));
    }
    if (stepping) {
      const size_t ni = (static_cast<size_t>(bb) * H + h) * kHeadDim + rc;
      const uint8_t* src = static_cast<const uint8_t*>(tid < kHeadDim ? p.k_new : p.v_new);
      nraw = *reinterpret_cast<const uint32_t*>(src + (p.kv_kind == 0 ? (2 * ni) & ~static_cast<size_t>(3) : 4 * ni));
    }
  };
  if (b_g >= 0) {
    load_pages(b_g, p0_g);
    load_seq(b_g);
  }
  const bool hadamard = p.rot_kind == 1;  // R = diag(s) H / sqrt(128): r_k, r_v hold the signs s
  const float vmid = 0.5f * static_cast<float>((1 << p.vbits) - 1);  // middle value code
  if (!hadamard) {
    const float* R = p.r_k + (static_cast<size_t>(h) * kHeadDim + kRows * rpart) * kHeadDim + rc;
#pragma unroll
    for (int ii = 0; ii < kRows; ++ii) rv[ii] = R[ii * kHeadDim];
  } else {
#pragma unroll
    for (int ii = 1; ii < kRows; ++ii) rv[ii] = 0.0f;
    rv[0] = p.r_k[h * kHeadDim + rc];
  }
  // the appending workgroup, guessed from max_seq_len (the last split of the guess)
  const int pps_g = max(p.pages_per_split, 1);
  const bool own_g = b_g >= 0 && (p0_g / pps_g) == ((p.len_cap + kPage - 1) / kPage + pps_g - 1) / pps_g - 1;
  auto load_own = [&]() {
    muraw = *reinterpret_cast<const uint32_t*>(p.mu != nullptr ? p.mu + h * kHeadDim + rc : p.r_v);
    if (!hadamard) {
      const float* R = p.r_v + (static_cast<size_t>(h) * kHeadDim + kRows * rpart) * kHeadDim + rc;
#pragma unroll
      for (int ii = 0; ii < kRows; ++ii) rvv[ii] = R[ii * kHeadDim];
    } else {
#pragma unroll
      for (int ii = 1; ii < kRows; ++ii) rvv[ii] = 0.0f;
      rvv[0] = p.r_v[h * kHeadDim + rc];
    }
  };
  if (stepping && own_g) load_own();

  // this workgroup's (sequence, split) and the partial row of the sequence's split 0
  int b, split, pps;
  size_t head_base;
  int T_raw;
  if (p.balanced) {
    __shared__ int s_red[kW], s_loc[3];
    const SplitLoc loc = locate_split<kW>(p, id / H, tid, lane, wave, s_red, s_loc);
    if (loc.b < 0) return;  // past the batch's last split (whole workgroup)
    b = loc.b;
    split = loc.split;
    pps = loc.pps;
    head_base = static_cast<size_t>(h) * p.n_splits + loc.first;
    T_raw = p.batch == 1 ? loc.len : p.seq_lens[b];
  } else {
    split = (id / H) % p.n_splits;
    b = id / (H * p.n_splits);
    pps = p.pages_per_split;
    head_base = (static_cast<size_t>(b) * H + h) * p.n_splits;
    T_raw = p.seq_lens[b];
  }

  // Pages past the table row are never read (a length beyond max_pages*16, or
  // beyond the host's max_seq_len, is cut).
  const int T = min(T_raw, p.len_cap);
  const int n_pages = T > 0 ? (T + kPage - 1) / kPage : 0;
  const size_t out_row0 = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(h) * g;
  if (n_pages == 0) {  // nothing to attend to: zero output, written once
    if (split == 0) {
      for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
        if (p.out_kind == 0)
          static_cast<uint16_t*>(p.out)[out_row0 * kHeadDim + idx] = 0;
        else
          static_cast<float*>(p.out)[out_row0 * kHeadDim + idx] = 0.0f;
      }
    }
    return;
  }
  const int n_valid = (n_pages + pps - 1) / pps;
  const int p0 = split * pps;
  if (p0 >= n_pages) return;  // whole workgroup
  const int np = min(pps, n_pages - p0);
  const int npairs = (np + 1) >> 1;
  // Step form: the last split appends the token at position T - 1 and attends
  // it from its packed levels; the paged read masks that position, whose slot
  // may still hold an older token (and is rewritten during this launch).
  const bool own = stepping && split == n_valid - 1;
  // INT2 positions attended from the paged cache: [int2_lo, int2_hi).  An exact
  // window takes the first win_sinks and the last win_recent positions; in the
  // step form the new token at T - 1 is attended from its packed levels
  // instead (unless the window holds it).
  const bool has_win = p.win != nullptr;
  const bool new_in_win = stepping && has_win && (T - 1 < p.win_sinks || p.win_recent > 0);
  const int int2_lo = has_win ? min(p.win_sinks, T) : 0;
  int int2_hi = has_win ? max(int2_lo, T - p.win_recent) : T;
  if (stepping && !new_in_win) int2_hi = min(int2_hi, T - 1);

  // ---- prologue loads not yet issued (no guess, or a wrong one): this split's
  // page ids, the g query rows and the new token.  Every prologue load lands
  // before the first page-pair load is issued.
  if (b != b_g || p0 != p0_g) load_pages(b, p0);
  if (b != b_g) load_seq(b);
  if (own && !own_g) load_own();
  const size_t ni = (static_cast<size_t>(b) * H + h) * kHeadDim + rc;
#pragma unroll
  for (int u = 0; u < kPidPerThread; ++u) {
    const int i = tid + u * kThreads;
    if (i < np) s_pages[i] = (pid[u] >= 0 && pid[u] < p.num_pages) ? pid[u] : -1;  // outside the pool: masked
  }
#pragma unroll
  for (int u = 0; u < kQPerThread; ++u) {
    const int idx = tid + u * kThreads;
    const size_t qi = (out_row0 + min(idx / kHeadDim, g - 1)) * kHeadDim + idx % kHeadDim;
    const float qv = p.q_kind == 0 ? bf16_bits_to_f32(static_cast<uint16_t>(qraw[u] >> (16 * (qi & 1))))
                                   : __uint_as_float(qraw[u]);
    if (idx < kNH * kHeadDim) s_q[idx / kHeadDim][idx % kHeadDim] = idx / kHeadDim < g ? qv : 0.0f;
  }
  if (own && tid < 2 * kHeadDim) {
    float nv = p.kv_kind == 0 ? bf16_bits_to_f32(static_cast<uint16_t>(nraw >> (16 * (ni & 1)))) : __uint_as_float(nraw);
    if (new_in_win && T_raw == T) {  // the new token's exact row into its window slot (bf16, nearest even)
      const int t = T - 1;
      const int slot = t < p.win_sinks ? t : p.win_sinks + t % p.win_recent;
      p.win[((static_cast<size_t>(b) * H + h) * (p.win_sinks + p.win_recent) + slot) * 2 * kHeadDim +
            (tid / kHeadDim) * kHeadDim + rc] = f32_to_bf16_bits(nv);
    }
    if (tid < kHeadDim && p.mu != nullptr) nv = nv - __uint_as_float(muraw);  // key centering (fp32)
    s_nrow[tid / kHeadDim][rc] = nv;
  }
  // Every prologue load must have landed before the first page-pair load is
  // issued: the compiler's own waits know nothing of those (inline asm) loads,
  // so a later wait for R would also wait for page data.
#pragma unroll
  for (int ii = 0; ii < kRows; ++ii) asm volatile("" ::"v"(rv[ii]));
  if (own) {
#pragma unroll
    for (int ii = 0; ii < kRows; ++ii) asm volatile("" ::"v"(rvv[ii]));
  }
  __syncthreads();
  // the new token's slot: position T - 1 on the split's last page (masked page,
  // or a length that was cut: no append)
  const bool new_ok = own && s_pages[np - 1] >= 0 && T_raw == T;
  const bool new_att = new_ok && !new_in_win;  // attended from its packed levels here

  const int a = lane >> 4;    // row of 16 lanes: token quad (QK) / channel octet
  const int col = lane & 15;  // MFMA column: 4*grp + jj
  const int grp = col >> 2;
  const int jj = col & 3;
  // within a page's metadata: the record of the group of G channels holding 32-channel group grp
  const int meta_off = kMetaRecordBytes * (4 * (grp >> meta_shift(p.gsize)) + a);
  // The octet layout (g = 5..8): every product covers all eight heads.  MFMA
  // column 8 oh + oj is head oj on the groups oh and oh + 2: a logit product
  // puts group oh (one accumulator) or oh + 2 (another) in the columns of its
  // half, and the P.V rows 8 oh + oj carry head oj's weights times the values'
  // scales of group oh (tiles 0-3) or oh + 2 (tiles 4-7).  Half the products
  // of two quads, and half their accumulators.
  constexpr bool kOct = kNQ == 2;
  // The hexadeca layout (g = 9..16): column (and P.V row) n is head n, and each
  // product is one group's: four logit accumulators per page and one P.V
  // operand per group, 24 products per page pair instead of four quads' 96.
  // The units of the P.V operand are then wave-uniform, one per group.
  constexpr bool kHex = kNQ == 4;
  const int oh = col >> 3, oj = col & 7;
  const int meta_lo = kMetaRecordBytes * (4 * (oh >> meta_shift(p.gsize)) + a);
  const int meta_hi = kMetaRecordBytes * (4 * ((oh + 2) >> meta_shift(p.gsize)) + a);
  int meta_g[4];  // hexadeca layout: the records of all four groups
#pragma unroll
  for (int G = 0; G < 4; ++G) meta_g[G] = kMetaRecordBytes * (4 * (G >> meta_shift(p.gsize)) + a);
  // 16-byte chunks per page of the metadata and of the planes (fewer lanes load them when compact)
  const int meta_ch = meta_bytes(p.gsize) / 16;
  const int kplane_ch = plane_bytes(p.kbits) / 16, vplane_ch = plane_bytes(p.vbits) / 16;
  const uint8_t* pool_h = p.pool + static_cast<size_t>(h) * kBlk;
  const size_t page_stride = static_cast<size_t>(H) * kBlk;

  auto issue = [&](int slot, int pair) {
    const int i0 = 2 * pair;
    // page ids are wave-uniform: block addresses live in scalar registers
    const int ph0 = __builtin_amdgcn_readfirstlane(s_pages[i0]);
    const int ph1 = __builtin_amdgcn_readfirstlane(i0 + 1 < np ? s_pages[i0 + 1] : -1);
    // a masked page reads page 0 (in bounds) and contributes no tokens
    const uint8_t* blk0 = pool_h + static_cast<size_t>(ph0 < 0 ? 0 : ph0) * page_stride;
    const uint8_t* blk1 = ph1 < 0 ? blk0 : pool_h + static_cast<size_t>(ph1) * page_stride;
    uint4v(*r)[64] = ring(slot);
    dma16(blk0, 16 * lane, &r[0][0]);
    dma16(blk1, 16 * lane, &r[1][0]);
    // metadata: lanes 0.. take page 0's, lanes 32.. page 1's (512 B apart in
    // the ring whatever their size)
    if (lane < 32) {
      if (lane < meta_ch) dma16(blk0, kCodeBytes + 16 * lane, &r[2][0]);
    } else {
      if (lane - 32 < meta_ch) dma16(blk1, kCodeBytes - 512 + 16 * lane, &r[2][0]);
    }
    if (kKW) {  // the keys' high-bit planes, page 0 then page 1 (512 B apart)
      if (lane < 32) {
        if (lane < kplane_ch) dma16(blk0, kKPlane + 16 * lane, &r[kKPart][0]);
      } else {
        if (lane - 32 < kplane_ch) dma16(blk1, kKPlane - 512 + 16 * lane, &r[kKPart][0]);
      }
    }
    if (kVW) {  // the values' high-bit planes
      if (lane < 32) {
        if (lane < vplane_ch) dma16(blk0, kVPlane + 16 * lane, &r[kVPart][0]);
      } else {
        if (lane - 32 < vplane_ch) dma16(blk1, kVPlane - 512 + 16 * lane, &r[kVPart][0]);
      }
    }
  };

  // Every wave keeps kDepth - 1 page pairs in flight ahead of the one it
  // computes (indices clamped to the last pair, so the wait counts are static;
  // a wave near the end loads the last pair again and never uses it).  The
  // first pair is requested now; the others after q_hat, which would otherwise
  // queue behind the whole grid's first requests.
  issue(0, min(wave, npairs - 1));

  // ---- q_hat for the g query heads of this KV head
  constexpr int kVecPasses = (kNH * kHeadDim + kThreads - 1) / kThreads;  // 128-vectors per thread (Hadamard)
  if (hadamard) {
    // q_hat = WHT(q * s_K) / sqrt(128) * scale, and the new token's centred key and
    // value rows by the transform the append kernel uses (kvq_quant.h: wht128)
#pragma unroll 1
    for (int pass = 0; pass < kVecPasses; ++pass) {
      const int idx = tid + pass * kThreads;
      const bool act = idx < kNH * kHeadDim;
      const int jh = min(idx / kHeadDim, kNH - 1), c = idx & (kHeadDim - 1);
      const float y = wht128(act ? s_q[jh][c] * rv[0] : 0.0f, c, act ? s_pro + jh * kHeadDim : nullptr);
      if (act) s_q[jh][c] = y * kInvSqrt128 * p.logit_scale;
    }
    if (new_ok) {
      const bool act = tid < 2 * kHeadDim;
      const int tensor = min(tid / kHeadDim, 1);
      const float x = act ? s_nrow[tensor][rc] * (tensor == 0 ? rv[0] : rvv[0]) : 0.0f;
      const float y = wht128(x, rc, act ? s_npart + tensor * kHeadDim : nullptr);
      if (act) s_nrow[tensor][rc] = y * kInvSqrt128;  // rotated
    }
  } else {
  if (tid < kParts * kHeadDim) {
    float accq[kNH];
#pragma unroll
    for (int jh = 0; jh < kNH; ++jh) accq[jh] = 0.0f;
#pragma unroll
    for (int ii = 0; ii < kRows; ++ii) {
#pragma unroll
      for (int jh = 0; jh < kNH; ++jh) accq[jh] = fmaf(s_q[jh][kRows * rpart + ii], rv[ii], accq[jh]);
    }
#pragma unroll
    for (int jh = 0; jh < kNH; ++jh) s_pro[(rpart * kNH + jh) * kHeadDim + rc] = accq[jh];
    if (new_ok) {  // rotation partials of the new key and value (shared summation order)
      s_npart[(0 * 4 + rpart) * kHeadDim + rc] = rot_chains<kRows>(&s_nrow[0][kRows * rpart], rv);
      s_npart[(1 * 4 + rpart) * kHeadDim + rc] = rot_chains<kRows>(&s_nrow[1][kRows * rpart], rvv);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kNH * kHeadDim; idx += kThreads) {
    const int jh = idx / kHeadDim;
    const int c = idx % kHeadDim;
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < kParts; ++u) sum += s_pro[(u * kNH + jh) * kHeadDim + c];
    s_q[jh][c] = sum * p.logit_scale;
  }
  if (new_ok && tid < 2 * kHeadDim) {
    const float* np_ = s_npart + tid / kHeadDim * 4 * kHeadDim + rc;
    const float x = kParts == 4 ? (np_[0] + np_[kHeadDim]) + (np_[2 * kHeadDim] + np_[3 * kHeadDim])
                                : np_[0] + np_[kHeadDim];
    s_nrow[tid / kHeadDim][rc] = x;  // rotated
  }
  }  // dense R
  __syncthreads();
  if (new_ok) {  // quantize-append the new token (two waves per tensor); new_ok is uniform here
    float2 rg = float2{0.0f, 0.0f};
    if (tid < 2 * kHeadDim) rg = q2_wave_range(s_nrow[tid / kHeadDim][rc], p.gsize);
    if (p.gsize == 128) {  // a group spans the tensor's two waves
      if (tid < 2 * kHeadDim && lane == 0) s_nrng[wave] = rg;
      __syncthreads();
      if (tid < 2 * kHeadDim) {
        const float2 a = s_nrng[wave & ~1], b = s_nrng[wave | 1];
        rg = float2{fminf(a.x, b.x), fmaxf(a.y, b.y)};
      }
    }
    if (tid < 2 * kHeadDim) {
      const int tensor = tid / kHeadDim;
      const int pos = T - 1;
      uint8_t* blk = p.pool + (static_cast<size_t>(s_pages[np - 1]) * H + h) * kBlk;
      s_hat[tensor][rc] = q2_pack_channel(s_nrow[tensor][rc], rc, tensor, blk, pos & (kPage - 1), p.clip, rg.x, rg.y,
                                          p.kbits, p.vbits, p.gsize);
    }
  }
  for (int jh = wave; jh < kNH; jh += kW) {
    const float am = wave_max_all(fmaxf(fabsf(s_q[jh][lane]), fabsf(s_q[jh][lane + 64])));
    if (lane == 0) {
      int e = 0;
      frexpf(am, &e);  // am in [2^(e-1), 2^e)
      s_f[jh] = am > 0.0f ? ldexpf(1.0f, 14 - e) : 1.0f;
    }
  }
  __syncthreads();
  if (new_att) {  // logits (log2 units) of the new token: one wave per head
    for (int jh = wave; jh < g; jh += kW) {
      const float d = wave_sum_all(fmaf(s_q[jh][lane], s_hat[0][lane], s_q[jh][lane + 64] * s_hat[0][lane + 64]));
      if (lane == 0) s_nlog[jh] = d;
    }
  }

#pragma unroll
  for (int d = 1; d < kDepth - 1; ++d) issue(d, min(wave + kW * d, npairs - 1));

  // ---- block-diagonal query operands (fp16 hi/lo of q_hat * f): per quad Q,
  //      column 4 grp + jj is head 4 Q + jj on group grp; in the octet layout
  //      (one set), column 8 oh + oj is head oj on groups oh and oh + 2
  half8 qhi[kNQ][4], qlo[kNQ][4];
  float qz[kNQ], c1[kNQ];  // octet layout: qz[0], qz[1] for groups oh, oh + 2
  // the hi/lo pair of head jl on 32-channel group gq, and its sum of q_hat over the group
  auto q_part = [&](int jl, int gq, float f, half8& hi, half8& lo) {
    float qsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e meets key register e/2, whose codes carry a factor 4^(e/2)
      const float qv = s_q[jl][32 * gq + 8 * a + e];
      const float sc = qv * f * (1.0f / static_cast<float>(1 << (2 * (e >> 1))));
      const _Float16 hh = static_cast<_Float16>(sc);
      hi[e] = hh;
      lo[e] = static_cast<_Float16>(sc - static_cast<float>(hh));
      qsum += qv;
    }
    return rows_sum(qsum);  // over the group's 32 channels
  };
  const half8 zero = {};
  if constexpr (kHex) {  // column col is head col; qz[G] for group G
    const float f = s_f[col];
    c1[0] = kTwo24 / f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qz[kk] = q_part(col, kk, f, qhi[0][kk], qlo[0][kk]) / c1[0];
  } else if constexpr (kOct) {
    const float f = s_f[oj];
    half8 hl, ll, hh, lh;
    const float qs_lo = q_part(oj, oh, f, hl, ll), qs_hi = q_part(oj, oh + 2, f, hh, lh);
    c1[0] = kTwo24 / f;
    qz[0] = qs_lo / c1[0];
    qz[1] = qs_hi / c1[0];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qhi[0][kk] = kk == oh ? hl : (kk == oh + 2 ? hh : zero);
      qlo[0][kk] = kk == oh ? ll : (kk == oh + 2 ? lh : zero);
    }
  } else {
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      const int jl = 4 * Q + jj;
      const float f = s_f[jl];
      half8 hi, lo;
      const float qsum = q_part(jl, grp, f, hi, lo);
      c1[Q] = kTwo24 / f;
      qz[Q] = qsum / c1[Q];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        qhi[Q][kk] = (grp == kk) ? hi : zero;
        qlo[Q][kk] = (grp == kk) ? lo : zero;
      }
    }
  }

  // Online-softmax state per quad.  m_run: the reference max of the lane's head
  // (log2 units); thr = (m_run + kLazy) / c1, the logit (in MFMA units) above
  // which the reference must move.  The P.V operand p * s_v is kept in units
  // of 2^e_u, e_u per value group (the lane's group grp, shared by the quads):
  // weights are formed as exp2(logit - m_run - e_u), so l_run, z_run and acc
  // hold 2^-e_u times their value.  e_u keeps the page pair's largest value
  // scale s_v of the group within [2^(e_u-3), 2^(e_u+7)); moving it (rarely)
  // rescales the sums.  With weights <= 2^kLazy the fp16 operand then stays
  // below 2^15, for every scale the cache format stores, and the group's
  // largest scale gives operands of at least p * 2^-3 (normal down to
  // p = 2^-11).  m_adj = m_run + e_u is the exp2 argument's offset.
  // The octet layout keeps one state (index 0) for head oj, z_run[0], [1] for
  // its groups oh and oh + 2, and a unit per group: e_u (oh) and e_u2 (oh + 2);
  // the weights are formed in units of 2^e_u and scaled by ratio =
  // 2^(e_u - e_u2) for group oh + 2.
  // The hexadeca layout keeps one state (index 0) for head col, z_run[G] per
  // group, and wave-uniform units eg[G]: its weights are formed without a
  // unit (exp2(logit - m_run) <= 2^kLazy) and scaled by 2^-eg[G] per group.
  float m_run[kNQ], l_run[kNQ], z_run[kNQ], m_adj[kNQ], thr[kNQ];
  float e_u = 0.0f, e_u2 = 0.0f, ratio = 1.0f;
  float eg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ug[4] = {1.0f, 1.0f, 1.0f, 1.0f};  // hexadeca: eg, ug = 2^-eg
  _Float16 uhg[4], ulg[4];  // hexadeca: 2^(eg+7), 2^(eg-3)
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    uhg[G] = static_cast<_Float16>(128.0f);
    ulg[G] = static_cast<_Float16>(0.125f);
  }
  _Float16 u_hi = static_cast<_Float16>(128.0f), u_lo = static_cast<_Float16>(0.125f);  // 2^(e_u+7), 2^(e_u-3)
  _Float16 u_hi2 = u_hi, u_lo2 = u_lo;                                                 // the same for e_u2
  float4v acc[kNQ][8];
#pragma unroll
  for (int Q = 0; Q < kNQ; ++Q) {
    m_run[Q] = kNegBig;
    l_run[Q] = 0.0f;
    z_run[Q] = 0.0f;
    m_adj[Q] = kNegBig;
    thr[Q] = -INFINITY;  // the first pair with a live position sets the reference
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[Q][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto compute = [&](int slot, int pair) {
    wait_vmcnt<kDmaPerPair * (kDepth - 1)>();  // this slot's loads have landed
    PagePair P;
    uint4v(*r)[64] = ring(slot);
    P.rec0 = r[0][lane];
    P.rec1 = r[1][lane];
    const uint8_t* meta = reinterpret_cast<const uint8_t*>(&r[2][0]);
    P.km0 = *reinterpret_cast<const uint4v*>(meta + meta_off);
    P.vm0 = *reinterpret_cast<const uint4v*>(meta + meta_off + 16);
    P.km1 = *reinterpret_cast<const uint4v*>(meta + 512 + meta_off);
    P.vm1 = *reinterpret_cast<const uint4v*>(meta + 512 + meta_off + 16);
    // wide codes: the high bits of record `lane`, per page, at the positions of
    // their low bits in the code words (H0, H1 or VH0, VH1).  4-bit planes hold
    // them so; a 3-bit key plane word holds both K words' bits interleaved (bit
    // j + w), a 3-bit value plane word one byte per slot (bit 8 i + t), spread
    // here to bit 2 t + 16 (i % 2) of word i / 2.
    uint32_t kh[2][2] = {{0u, 0u}, {0u, 0u}}, vh[2][2] = {{0u, 0u}, {0u, 0u}};
    if (kKW) {
      const uint32_t* hp = reinterpret_cast<const uint32_t*>(&r[kKPart][0]);
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        if (p.kbits == 3) {
          const uint32_t w = hp[128 * X + lane];
          kh[X][0] = w & 0x55555555u;
          kh[X][1] = (w >> 1) & 0x55555555u;
        } else {
          kh[X][0] = hp[128 * X + 2 * lane];
          kh[X][1] = hp[128 * X + 2 * lane + 1];
        }
      }
    }
    if (kVW) {
      const uint32_t* hp = reinterpret_cast<const uint32_t*>(&r[kVPart][0]);
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        if (p.vbits == 3) {
          const uint32_t w = hp[128 * X + lane];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint32_t y = ((w >> (16 * q)) & 0xffu) | (((w >> (16 * q + 8)) & 0xffu) << 16);
            y = (y | (y << 4)) & 0x0f0f0f0fu;
            y = (y | (y << 2)) & 0x33333333u;
            vh[X][q] = (y | (y << 1)) & 0x55555555u;
          }
        } else {
          vh[X][0] = hp[128 * X + 2 * lane];
          vh[X][1] = hp[128 * X + 2 * lane + 1];
        }
      }
    }
    const int i0 = 2 * pair;
    // page ids and the pair's validity are wave-uniform (scalar registers)
    const int ph0 = __builtin_amdgcn_readfirstlane(s_pages[i0]);
    const int ph1 = __builtin_amdgcn_readfirstlane(i0 + 1 < np ? s_pages[i0 + 1] : -1);
    const bool ok0 = ph0 >= 0;
    const bool has1 = ph1 >= 0;
    // no position of the pair masked
    const bool full = ok0 && has1 && (p0 + i0) * kPage >= int2_lo && (p0 + i0 + 2) * kPage <= int2_hi;
    // Key operands of page X: a code at bits 2q (+16) of a word is the fp16
    // subnormal code * 4^q * 2^-24, so one AND per register; groups 1 and 3 sit
    // in the upper byte of each half and are shifted down first.  The factor
    // 4^q is divided out of the query operand.  A wide key's high bits, moved
    // two bits up, fill bits 2q + 2 and 2q + 3: low | high is the whole code
    // times 4^q (at most 15 * 64 < 2^10, still a subnormal), one AND-OR more.
    auto key_ops = [&](int X, half8 (&kA)[4]) {
      const uint4v rec = X ? P.rec1 : P.rec0;
      const uint32_t kw[4] = {rec[0], rec[0] >> 8, rec[1], rec[1] >> 8};
      const uint32_t kw2[4] = {kh[X][0] << 2, (kh[X][0] >> 8) << 2, kh[X][1] << 2, (kh[X][1] >> 8) << 2};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint4v rr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t m = 0x00030003u << (2 * q);
          rr[q] = kKW ? ((kw[kk] & m) | (kw2[kk] & (m << 2))) : (kw[kk] & m);
        }
        kA[kk] = __builtin_bit_cast(half8, rr);
      }
    };
    // Value operands: tile t holds channels 16t..16t+15.  Tiles 0-3 sit in the
    // low byte of each half (bits 2t), tiles 4-7 in the high byte; a register
    // of tile t holds the codes times 4^(t%4) (divided out of acc at the end).
    // Wide values: the plane's bits two up, OR-ed in as for the keys.
    auto value_ops = [&](half8 (&vB)[8]) {
      const uint32_t vw[8] = {P.rec0[2], P.rec0[3], P.rec1[2], P.rec1[3],
                              P.rec0[2] >> 8, P.rec0[3] >> 8, P.rec1[2] >> 8, P.rec1[3] >> 8};
      const uint32_t vw2[8] = {vh[0][0] << 2, vh[0][1] << 2, vh[1][0] << 2, vh[1][1] << 2,
                               (vh[0][0] >> 8) << 2, (vh[0][1] >> 8) << 2, (vh[1][0] >> 8) << 2,
                               (vh[1][1] >> 8) << 2};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t m = 0x00030003u << (2 * (t & 3));
        const int hb = 4 * (t >> 2);
        uint4v rr;
#pragma unroll
        for (int i = 0; i < 4; ++i) rr[i] = kVW ? ((vw[hb + i] & m) | (vw2[hb + i] & (m << 2))) : (vw[hb + i] & m);
        vB[t] = __builtin_bit_cast(half8, rr);
      }
    };
    // position i of page X's quad a is attended from the cache
    auto live = [&](int X, int i) {
      return (X == 0 ? ok0 : has1) && (p0 + i0 + X) * kPage + 4 * a + i >= int2_lo &&
             (p0 + i0 + X) * kPage + 4 * a + i < int2_hi;
    };

    if constexpr (kHex) {
      // metadata records of the four groups, tokens 4 a + i of pages 0 and 1
      uint4v kmg[2][4], vmg[2][4];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          kmg[X][G] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_g[G]);
          vmg[X][G] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_g[G] + 16);
        }
      // logits (log2 units, divided by c1) of head col, tokens 4 a + i of page X
      float sx[2][4];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        half8 kA[4];
        key_ops(X, kA);
        float4v C[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          C[kk] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
          C[kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qhi[0][kk], C[kk], 0, 0, 0);
          C[kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qlo[0][kk], C[kk], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = 0.0f;
#pragma unroll
          for (int G = 0; G < 4; ++G) {
            const uint32_t km = kmg[X][G][i];
            s = fmaf(C[G][i], f16_lo(km), fmaf(f16_hi(km), qz[G], s));
          }
          sx[X][i] = s;
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!live(X, i)) {  // weight 0; the value metadata may hold any bits
              sx[X][i] = -INFINITY;
#pragma unroll
              for (int G = 0; G < 4; ++G) vmg[X][G][i] = 0u;
            }
        }
      }
      half8 vB[8];
      value_ops(vB);

      // the P.V unit of each group (wave-uniform): moved when a scale of the
      // pair reaches 2^(eg+7), or when the group's nonzero scales all lie below
      // 2^(eg-3); the sums kept in the old unit are rescaled
      {
        auto s16 = [](uint32_t w) { return __builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)); };
        const _Float16 z16 = static_cast<_Float16>(0.0f);
        _Float16 mg[4];
        bool need = false;
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          mg[G] = s16(vmg[0][G][0]);
#pragma unroll
          for (int X = 0; X < 2; ++X)
#pragma unroll
            for (int i = 0; i < 4; ++i) mg[G] = __builtin_fmaxf16(mg[G], s16(vmg[X][G][i]));
          need = need || __ballot(mg[G] >= uhg[G]) != 0 ||
                 (__ballot(mg[G] > z16) != 0 && __ballot(mg[G] >= ulg[G]) == 0);
        }
        if (need) {  // rare
#pragma unroll
          for (int G = 0; G < 4; ++G) {
            const float gs = wave_max_all(static_cast<float>(mg[G]));
            int ex = 0;
            frexpf(gs, &ex);  // gs in [2^(ex-1), 2^ex)
            const bool move = gs >= static_cast<float>(uhg[G]) || (gs < static_cast<float>(ulg[G]) && gs > 0.0f);
            const float en = move ? static_cast<float>(ex - 7) : eg[G];
            const float fl = ldexpf(1.0f, static_cast<int>(eg[G] - en));  // old unit / new unit
            acc[0][2 * G] *= fl;
            acc[0][2 * G + 1] *= fl;
            z_run[G] *= fl;
            eg[G] = en;
            ug[G] = ldexpf(1.0f, -static_cast<int>(en));
            uhg[G] = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(en) + 7));  // inf past fp16: never reached
            ulg[G] = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(en) - 3));  // 0 below fp16: no lower unit
          }
        }
      }

      // online softmax of head col (lazy reference; weights formed without a unit)
      float smax = sx[0][0];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) smax = fmaxf(smax, sx[X][i]);
      if (__ballot(smax > thr[0]) != 0) {
        const float m_new = fmaxf(m_run[0], rows_max(smax) * c1[0]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[0] - m_new);
        // acc row 4 a + i is head 4 a + i: its factor from lane 4 a + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * a + i);
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[0][t][i] *= al;
        }
        l_run[0] *= alpha;
#pragma unroll
        for (int G = 0; G < 4; ++G) z_run[G] *= alpha;
        m_run[0] = m_new;
        thr[0] = (m_new + kLazy) * (1.0f / c1[0]);
      }
      half8 pG[4];  // row col: head col's weights times the value scales of group G, in units of 2^eg
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sx[X][i], c1[0], -m_run[0]));
          l_run[0] += pr;
#pragma unroll
          for (int G = 0; G < 4; ++G) {
            const uint32_t vm = vmg[X][G][i];
            const float pw = pr * ug[G];
            z_run[G] = fmaf(f16_hi(vm), pw, z_run[G]);
            if (kHad) {
              const float ps = f16_lo(vm) * pw;
              const _Float16 hi = static_cast<_Float16>(ps);
              pG[G][4 * X + i] = hi;
              z_run[G] = fmaf(vmid, ps - static_cast<float>(hi), z_run[G]);
            } else {
              pG[G][4 * X + i] = static_cast<_Float16>(fmaf(f16_lo(vm), pw, 0.0f));
            }
          }
        }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pG[t >> 1], vB[t], acc[0][t], 0, 0, 0);
      return;
    }

    if constexpr (kOct) {
      // metadata records of the lane's groups oh (L) and oh + 2 (H), pages 0 and 1
      uint4v kmL[2], kmH[2], vmL[2], vmH[2];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        kmL[X] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_lo);
        vmL[X] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_lo + 16);
        kmH[X] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_hi);
        vmH[X] = *reinterpret_cast<const uint4v*>(meta + 512 * X + meta_hi + 16);
      }
      // logits (log2 units, divided by c1) of head oj, tokens 4 a + i of page X
      float so[2][4];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        half8 kA[4];
        key_ops(X, kA);
        float4v CL = {0.0f, 0.0f, 0.0f, 0.0f}, CH = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {  // groups 0, 1: column half oh holds group oh
          CL = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qhi[0][kk], CL, 0, 0, 0);
          CL = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qlo[0][kk], CL, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 2; kk < 4; ++kk) {  // groups 2, 3: group oh + 2
          CH = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qhi[0][kk], CH, 0, 0, 0);
          CH = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qlo[0][kk], CH, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the lane's two groups, then the other column half's two (lane col ^ 8)
          const uint32_t kl = kmL[X][i], kh2 = kmH[X][i];
          const float s = fmaf(CL[i], f16_lo(kl), fmaf(f16_hi(kl), qz[0], fmaf(CH[i], f16_lo(kh2), f16_hi(kh2) * qz[1])));
          so[X][i] = s + dpp_f32<kDppRowRor8>(s);
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!live(X, i)) {  // weight 0; the value metadata may hold any bits
              so[X][i] = -INFINITY;
              vmL[X][i] = 0u;
              vmH[X][i] = 0u;
            }
        }
      }
      half8 vB[8];
      value_ops(vB);

      // the P.V units of groups oh and oh + 2, as in the quad layout below
      {
        auto s16 = [](uint32_t w) { return __builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)); };
        _Float16 mL = s16(vmL[0][0]), mH = s16(vmH[0][0]);
#pragma unroll
        for (int X = 0; X < 2; ++X)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mL = __builtin_fmaxf16(mL, s16(vmL[X][i]));
            mH = __builtin_fmaxf16(mH, s16(vmH[X][i]));
          }
        // bit 8 h of fold(b): some lane of column half h (lanes 16 a + 8 h + j) is set
        auto fold = [](uint64_t b) {
          b |= b >> 32;
          b |= b >> 16;
          b |= b >> 1;
          b |= b >> 2;
          b |= b >> 4;
          return b & 0x101ull;
        };
        const _Float16 z16 = static_cast<_Float16>(0.0f);
        const uint64_t need = __ballot(mL >= u_hi) | __ballot(mH >= u_hi2) |
                              (fold(__ballot(mL > z16)) & ~fold(__ballot(mL >= u_lo))) |
                              (fold(__ballot(mH > z16)) & ~fold(__ballot(mH >= u_lo2)));
        if (need != 0) {  // rare
          // a group's largest scale: its column half (8 columns) over the four rows
          auto group_max = [](float x) {
            x = fmaxf(x, dpp_f32<QuadXor1::ctrl>(x));
            x = fmaxf(x, dpp_f32<QuadXor2::ctrl>(x));
            x = fmaxf(x, __shfl_xor(x, 4));
            return rows_max(x);
          };
          auto new_unit = [](float gs, float e_old, _Float16 uh, _Float16 ul) {
            int ex = 0;
            frexpf(gs, &ex);  // gs in [2^(ex-1), 2^ex)
            const bool move = gs >= static_cast<float>(uh) || (gs < static_cast<float>(ul) && gs > 0.0f);
            return move ? static_cast<float>(ex - 7) : e_old;
          };
          const float nL = new_unit(group_max(static_cast<float>(mL)), e_u, u_hi, u_lo);
          const float nH = new_unit(group_max(static_cast<float>(mH)), e_u2, u_hi2, u_lo2);
          const float fL = ldexpf(1.0f, static_cast<int>(e_u - nL));  // old unit / new unit
          const float fH = ldexpf(1.0f, static_cast<int>(e_u2 - nH));
          // acc rows 4 a + i belong to group a / 2 (tiles 0-3) and a / 2 + 2 (tiles 4-7)
          const float faL = __shfl(fL, 8 * (a >> 1)), faH = __shfl(fH, 8 * (a >> 1));
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[0][t] *= t < 4 ? faL : faH;
          l_run[0] *= fL;
          z_run[0] *= fL;
          z_run[1] *= fH;
          e_u = nL;
          e_u2 = nH;
          m_adj[0] = m_run[0] + e_u;
          ratio = ldexpf(1.0f, static_cast<int>(e_u - e_u2));
          u_hi = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u) + 7));  // inf past fp16: never reached
          u_lo = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u) - 3));  // 0 below fp16: no lower unit
          u_hi2 = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u2) + 7));
          u_lo2 = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u2) - 3));
        }
      }

      // online softmax of head oj (lazy reference, as below)
      float smax = so[0][0];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) smax = fmaxf(smax, so[X][i]);
      if (__ballot(smax > thr[0]) != 0) {
        const float m_new = fmaxf(m_run[0], rows_max(smax) * c1[0]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[0] - m_new);
        // acc row 4 a + i is head 4 (a % 2) + i: its factor from lane 4 (a % 2) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * (a & 1) + i);
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[0][t][i] *= al;
        }
        l_run[0] *= alpha;
        z_run[0] *= alpha;
        z_run[1] *= alpha;
        m_run[0] = m_new;
        m_adj[0] = m_new + e_u;
        thr[0] = (m_new + kLazy) * (1.0f / c1[0]);
      }
      half8 pL, pH;  // rows 8 oh + oj: weights times the value scales of group oh / oh + 2
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(so[X][i], c1[0], -m_adj[0]));
          const float prh = pr * ratio;
          l_run[0] += pr;
          z_run[0] = fmaf(f16_hi(vmL[X][i]), pr, z_run[0]);
          z_run[1] = fmaf(f16_hi(vmH[X][i]), prh, z_run[1]);
          if (kHad) {
            const float psl = f16_lo(vmL[X][i]) * pr, psh = f16_lo(vmH[X][i]) * prh;
            const _Float16 hl = static_cast<_Float16>(psl), hh = static_cast<_Float16>(psh);
            pL[4 * X + i] = hl;
            pH[4 * X + i] = hh;
            z_run[0] = fmaf(vmid, psl - static_cast<float>(hl), z_run[0]);
            z_run[1] = fmaf(vmid, psh - static_cast<float>(hh), z_run[1]);
          } else {
            pL[4 * X + i] = static_cast<_Float16>(fmaf(f16_lo(vmL[X][i]), pr, 0.0f));
            pH[4 * X + i] = static_cast<_Float16>(fmaf(f16_lo(vmH[X][i]), prh, 0.0f));
          }
        }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(t < 4 ? pL : pH, vB[t], acc[0][t], 0, 0, 0);
      return;
    }

    // logits (log2 units, divided by c1) for both pages
    float sp[kNQ][2][4];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const uint4v km = X ? P.km1 : P.km0;
      half8 kA[4];
      key_ops(X, kA);
      const int pos0 = (p0 + i0 + X) * kPage + 4 * a;
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
          // s_grp * <codes, q_hat> + z_grp * sum(q_hat), scale/zero read as fp16 operands
          float s = fmaf(C[i], f16_lo(km[i]), fmaf(f16_hi(km[i]), qz[Q], 0.0f));
          sp[Q][X][i] = row_sum_stride4(s);
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!(page_ok && pos0 + i >= int2_lo && pos0 + i < int2_hi)) sp[Q][X][i] = -INFINITY;
        }
      }
      // A masked position (stale slot, absent page, window position) weighs 0;
      // its value metadata may hold any bits, so it is cleared (0 * inf would
      // be NaN in the P.V operand and the zero-point sum).
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(page_ok && pos0 + i >= int2_lo && pos0 + i < int2_hi)) {
            if (X)
              P.vm1[i] = 0u;
            else
              P.vm0[i] = 0u;
          }
      }
    }

    half8 vB[8];
    value_ops(vB);

    // The P.V operand's unit per value group, from the pair's value scales
    // (lane: its group's scales of 8 positions; masked ones are 0): any scale
    // at or above 2^(e_u+7), or a group whose scales are all below 2^(e_u-3)
    // but not all zero, moves that group's unit so that its largest scale
    // lies in [2^6, 2^7) units, and rescales the sums kept in the old unit.
    {
      auto s16 = [](uint32_t w) { return __builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)); };
      _Float16 smx = s16(P.vm0[0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) smx = __builtin_fmaxf16(smx, s16(P.vm0[i]));
#pragma unroll
      for (int i = 0; i < 4; ++i) smx = __builtin_fmaxf16(smx, s16(P.vm1[i]));
      const uint64_t b_hi = __ballot(smx >= u_hi);
      const uint64_t b_lo = __ballot(smx >= u_lo);
      const uint64_t b_nz = __ballot(smx > static_cast<_Float16>(0.0f));
      // bit 4 grp of fold(b): some lane of group grp (lanes 16 a + 4 grp + jj) is set
      auto fold = [](uint64_t b) {
        b |= b >> 32;
        b |= b >> 16;
        b |= b >> 1;
        b |= b >> 2;
        return b & 0x1111ull;
      };
      if ((b_hi | (fold(b_nz) & ~fold(b_lo))) != 0) {  // rare
        float gs = static_cast<float>(smx);           // the group's largest scale
        gs = fmaxf(gs, dpp_f32<QuadXor1::ctrl>(gs));
        gs = fmaxf(gs, dpp_f32<QuadXor2::ctrl>(gs));
        gs = rows_max(gs);
        int ex = 0;
        frexpf(gs, &ex);  // gs in [2^(ex-1), 2^ex)
        const bool move = gs >= static_cast<float>(u_hi) || (gs < static_cast<float>(u_lo) && gs > 0.0f);
        const float e_new = move ? static_cast<float>(ex - 7) : e_u;
        const float fl = ldexpf(1.0f, static_cast<int>(e_u - e_new));  // old unit / new unit, this lane's group
        const float fa = __shfl(fl, 4 * a);                              // the same for acc rows of group a
#pragma unroll
        for (int Q = 0; Q < kNQ; ++Q) {
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[Q][t] *= fa;
          l_run[Q] *= fl;
          z_run[Q] *= fl;
          m_adj[Q] = m_run[Q] + e_new;
        }
        e_u = e_new;
        u_hi = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u) + 7));  // inf past fp16: never reached
        u_lo = static_cast<_Float16>(ldexpf(1.0f, static_cast<int>(e_u) - 3));  // 0 below fp16: no lower unit
      }
    }

    // online softmax and P.V per quad
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      // Lazy rescaling: the reference max moves only when some head's logits
      // exceed it by more than kLazy (log2 units), so the weights
      // exp2(logit - m_run) stay <= 2^kLazy and most pairs skip the rescale.
      // The test is lane-local against thr (c1 is a power of two, so
      // logit * c1 > m_run + kLazy exactly when logit > thr); only a pair that
      // moves the reference reduces its maximum across the rows.
      float smax = sp[Q][0][0];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) smax = fmaxf(smax, sp[Q][X][i]);
      if (__ballot(smax > thr[Q]) != 0) {
        const float m_new = fmaxf(m_run[Q], rows_max(smax) * c1[Q]);
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
        m_adj[Q] = m_new + e_u;
        thr[Q] = (m_new + kLazy) * (1.0f / c1[Q]);
      }
      // A = p * s_v as fp16, in units of 2^e_u.  Its rounding error times the
      // codes would, in the sum over tokens, leave an error common to the 32
      // channels of a group (the code part of the value sum largely cancels
      // against the zero-point part, z_v being about the group's minimum); a
      // Hadamard R_V^T gathers such an error into single output channels, where
      // it came within a few percent of the 2e-3 gate.  With a Hadamard R the
      // rounding error times the middle code goes into the zero-point sum
      // instead, so what is left multiplies (code - middle), which has no
      // common part.  A dense R spreads the error over all channels and needs
      // no correction.
      half8 pA;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sp[Q][X][i], c1[Q], -m_adj[Q]));
          const uint32_t vm = X ? P.vm1[i] : P.vm0[i];
          l_run[Q] += pr;
          z_run[Q] = fmaf(f16_hi(vm), pr, z_run[Q]);
          if (kHad) {
            const float ps = f16_lo(vm) * pr;
            const _Float16 hi = static_cast<_Float16>(ps);
            pA[4 * X + i] = hi;
            z_run[Q] = fmaf(vmid, ps - static_cast<float>(hi), z_run[Q]);
          } else {
            pA[4 * X + i] = static_cast<_Float16>(fmaf(f16_lo(vm), pr, 0.0f));
          }
        }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[Q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pA, vB[t], acc[Q][t], 0, 0, 0);
    }
  };

  // ---- main loop
  for (int pair = wave; pair < npairs;) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      issue((k + kDepth - 1) % kDepth, min(pair + kW * (kDepth - 1), npairs - 1));
      compute(k, pair);
      pair += kW;
      if (pair >= npairs) break;
    }
  }
  wait_vmcnt<0>();  // no load into the ring outlives the loop
  __syncthreads();   // every wave is done with the ring; its LDS is reused below

  // ---- per-wave results to LDS: lane (a, b) owns channels 32a + b and
  //      32a + 16 + b (tiles 2a, 2a+1) for the four heads of each quad.
  // lane values broadcast by readlane (scalar operands), picked by the lane's row a
  auto lane_val = [](float x, int k) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k)); };
  auto pick_a = [&](float x, int k0) {  // x at lane k0 + 4 a
    const float v0 = lane_val(x, k0), v1 = lane_val(x, k0 + 4), v2 = lane_val(x, k0 + 8), v3 = lane_val(x, k0 + 12);
    return a == 0 ? v0 : (a == 1 ? v1 : (a == 2 ? v2 : v3));
  };
  if constexpr (kHex) {
    // lane (a, col) holds acc rows 4 a + i, head 4 a + i, of every tile; the
    // sums of tile t are in units of 2^eg[t / 2]; lanes 0..15 carry head col's
    // weight sum (no unit)
    const float lsum = rows_sum(l_run[0]);
    float zs[4];  // lane (., col): sum_s p z_v for (head col, group G)
#pragma unroll
    for (int G = 0; G < 4; ++G) zs[G] = rows_sum(z_run[G]) * ldexpf(1.0f, static_cast<int>(eg[G]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jh = 4 * a + i;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const float zi = pick_a(zs[G], i);  // lane 4 a + i: head jh, group G
        const float ut = ldexpf(1.0f, static_cast<int>(eg[G]));
#pragma unroll
        for (int t = 2 * G; t < 2 * G + 2; ++t)
          s_post[(wave * kNH + jh) * kHeadDim + 16 * t + col] =
              acc[0][t][i] * ((kTwo24 / static_cast<float>(1 << (2 * (t & 3)))) * ut) + zi;
      }
    }
    if (lane < 16) {
      s_m[wave][lane] = m_run[0];
      s_l[wave][lane] = lsum;
    }
  } else if constexpr (kOct) {
    // sums in units of 2^e_u (group oh) and 2^e_u2 (group oh + 2); lanes 0..7
    // (column half 0) carry head oj's weight sum.  Lane (a, col) holds acc rows
    // 4 a + i: head 4 (a % 2) + i on group a / 2 (tiles 0-3) or a / 2 + 2
    // (tiles 4-7), kept where the tile's channels are that group's.
    const float unit_l = ldexpf(1.0f, static_cast<int>(e_u)), unit_h = ldexpf(1.0f, static_cast<int>(e_u2));
    const float ua_l = (a >> 1) ? lane_val(unit_l, 8) : lane_val(unit_l, 0);
    const float ua_h = (a >> 1) ? lane_val(unit_h, 8) : lane_val(unit_h, 0);
    const float lsum = rows_sum(l_run[0]) * unit_l;
    // lane (., oh, oj): sum_s p z_v for (oj, group oh) and (oj, group oh + 2)
    const float zs_l = rows_sum(z_run[0]) * unit_l, zs_h = rows_sum(z_run[1]) * unit_h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jh = 4 * (a & 1) + i;
      const float zl = pick_a(zs_l, i), zh = pick_a(zs_h, i);  // lane 4 a + i: head jh, group a / 2 (+ 2)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (((t >> 1) & 1) == (a >> 1))
          s_post[(wave * kNH + jh) * kHeadDim + 16 * t + col] =
              acc[0][t][i] * ((kTwo24 / static_cast<float>(1 << (2 * (t & 3)))) * (t < 4 ? ua_l : ua_h)) +
              (t < 4 ? zl : zh);
      }
    }
    if (lane < 8) {
      s_m[wave][lane] = m_run[0];
      s_l[wave][lane] = lsum;
    }
  } else {
#pragma unroll
    for (int Q = 0; Q < kNQ; ++Q) {
      // the sums were kept in units of 2^e_u of the lane's value group: lanes
      // 0..3 (group 0) carry the weight sums, acc rows of group a take group a's unit
      const float unit = ldexpf(1.0f, static_cast<int>(e_u));
      const float unit_a = pick_a(unit, 0);
      const float lsum = rows_sum(l_run[Q]) * unit;
      const float zsum = rows_sum(z_run[Q]) * unit;  // lane (., grp, jj): sum_s p z_v for (jj, grp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zi = pick_a(zsum, i);  // zero part of head i, group a (the rows hold the same sums)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if ((t >> 1) == a)  // undo the tile's code factor 4^(t%4), the 2^-24 code scale and the unit
            s_post[(wave * kNH + 4 * Q + i) * kHeadDim + 16 * t + col] =
                acc[Q][t][i] * ((kTwo24 / static_cast<float>(1 << (2 * (t & 3)))) * unit_a) + zi;
        }
      }
      if (lane < 4) {
        s_m[wave][4 * Q + lane] = m_run[Q];
        s_l[wave][4 * Q + lane] = lsum;
      }
    }
  }
  __syncthreads();

  // ---- workgroup partial -> workspace (agent-scope stores: coherent across
  //      XCDs without an L2 writeback).  Each thread keeps the elements it
  //      stored, for the merge should this workgroup be the last.
  constexpr int kIdx = (kNH * kHeadDim + kThreads - 1) / kThreads;  // output elements per thread
  float own_m[kIdx], own_l[kIdx], own_a[kIdx];
#pragma unroll
  for (int k = 0; k < kIdx; ++k) {
    const int idx = tid + k * kThreads;
    if (idx >= g * kHeadDim) break;
    const int jh = idx / kHeadDim;
    const int c = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, s_m[w][jh]);
    if (new_att) M = fmaxf(M, s_nlog[jh]);
    float av = 0.0f, lv = 0.0f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float wt = __builtin_amdgcn_exp2f(s_m[w][jh] - M);
      av = fmaf(wt, s_post[(w * kNH + jh) * kHeadDim + c], av);
      lv = fmaf(wt, s_l[w][jh], lv);
    }
    if (new_att) {  // the new token, weight exp2(logit - M), level w_hat
      const float wt = __builtin_amdgcn_exp2f(s_nlog[jh] - M);
      av = fmaf(wt, s_hat[1][c], av);
      lv += wt;
    }
    own_m[k] = M;
    own_l[k] = lv;
    own_a[k] = av;
    float* dst = p.part + ((head_base + split) * g + jh) * kPartStride;
    __hip_atomic_store(dst + c, av, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c == 0) {
      __hip_atomic_store(dst + 128, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 129, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Exact window, on the matrix cores (v_mfma_f32_16x16x32_bf16; the window
  // rows are exact bf16), computed by the workgroup of the sequence's last
  // split after its page loop and stored to the workspace before its ticket
  // (the window row of each query head: acc 128 | max | sum, acc unnormalised
  // and in the original basis); the merging workgroup loads it with the split
  // rows.  Rows: n_ws sinks, then positions w_r0 .. T-1, loaded whole into
  // registers, then staged in the upper part of the ring 256 B per row: first
  // the keys (16-byte chunks XOR-swizzled by row % 16) for the logits, then
  // the values in the same place for the value sums; above the merge's
  // max/sum pairs (at most 2 * kNH * (max splits with a window) floats); the
  // R_V^T partials later reuse the rows' space.
  //   logits  C[head][row] = <q_head, k_row> over 16-row tiles: A = q split
  //           into three bf16 parts (truncation; about 21 bits), B = key rows;
  //           <q_head, mu> is taken off in fp32.
  //   values  O[head][ch] = sum_row p[head][row] v_row[ch] over 16-channel tiles
  //           and 32-row blocks: A = p in two bf16 parts, B = values.
  // Both splits are made once into LDS in operand order.  Rows past n_w read
  // row n_w - 1 (finite) and carry weight 0.
  constexpr bool kWinOk = kWgPerCu == 1;  // the narrow shape's ring cannot stage a window
  constexpr int kWinMax = 8 + 128;                    // window rows
  constexpr int kWinLd = kWinOk ? (kWinMax * 32 + kThreads - 1) / kThreads : 1;  // 16-byte chunks per thread
  constexpr int kWinRowsPad = 32 * ((kWinMax + 31) / 32);  // 32-row blocks of the value product
  constexpr int kHeadRow = kWinRowsPad + 8;           // floats per head: logits, then p hi | p lo (bf16)
  constexpr int kQpStride = kHeadDim + 8;             // bf16 per (part, head) row of the q parts
  constexpr int kWinSplits = kNQ == 1 ? kMaxSplits : 128;  // splits per sequence allowed with a window
  constexpr int kRingFloats = static_cast<int>(sizeof(s_ring) / sizeof(float));
  constexpr int kOwOff = kRingFloats - kNH * kHeadDim;  // [kNH][128] window value sums
  constexpr int kWmlOff = kOwOff - 2 * kNH;             // [kNH][2] window max, sum of weights
  constexpr int kRowsOff = kWmlOff - kWinMax * kHeadDim / 2;  // [kWinMax][128] bf16 rows (keys, then values)
  constexpr int kWpOff = kRowsOff - kNH * kHeadRow;     // [kNH][kHeadRow]
  constexpr int kQpOff = kWpOff - 3 * kNH * kQpStride / 2;  // [3][kNH][kQpStride] bf16 q parts
  constexpr int kWmuOff = kQpOff - kHeadDim - kNH;      // [128] mu, then [kNH] <q, mu>
  static_assert(!kWinOk || (kRowsOff % 4 == 0 && kWpOff % 4 == 0 && kQpOff % 4 == 0 && kWmuOff >= 0 &&
                            kWmuOff >= 2 * kNH * kWinSplits && kWmlOff >= kParts * kNH * kHeadDim),
                "window staging fits above the merge scratch");
  const bool win_here = kWinOk && has_win;
  const bool win_wg = win_here && split == n_valid - 1;  // computes the window part
  int n_ws = 0, w_r0 = 0, n_w = 0;
  uint4v wraw[kWinLd];
  uint32_t qwr[kQPerThread];
  float wmu = 0.0f;
  if (win_wg) {
    n_ws = min(p.win_sinks, T);
    w_r0 = max(n_ws, T - p.win_recent);
    n_w = n_ws + (T - w_r0);
    const int n_slots = p.win_sinks + p.win_recent;
    const uint16_t* wb = p.win + (static_cast<size_t>(b) * H + h) * n_slots * 2 * kHeadDim;
    const size_t nrow = (static_cast<size_t>(b) * H + h) * kHeadDim;
    // The step's new token (position T - 1, always the last window row when the
    // window holds it) is read from k_new / v_new: its slot is written by the
    // appending workgroup during this launch.  fp32 input: the row's 8 floats
    // arrive as two 16-byte words (at most one chunk of it per thread) and are
    // rounded to bf16 once all loads have landed.
    const bool new_here = new_in_win && T_raw == T;
    uint4v f32_hi = {0u, 0u, 0u, 0u};
    int u_f32 = -1;
#pragma unroll
    for (int u = 0; u < kWinLd; ++u) {
      const int idx = tid + u * kThreads;  // row wi, chunk j: 8 bf16 of the key (j < 16) or value row
      const int wi = idx >> 5, j = idx & 31;
      wraw[u] = uint4v{0u, 0u, 0u, 0u};
      if (wi < n_w) {
        if (new_here && wi == n_w - 1) {
          const uint8_t* src = static_cast<const uint8_t*>(j < 16 ? p.k_new : p.v_new) +
                               (nrow + 8 * (j & 15)) * (p.kv_kind == 0 ? 2 : 4);
          wraw[u] = *reinterpret_cast<const uint4v*>(src);
          if (p.kv_kind != 0) {
            f32_hi = *reinterpret_cast<const uint4v*>(src + 16);
            u_f32 = u;
          }
        } else {
          const int t = wi < n_ws ? wi : w_r0 + (wi - n_ws);
          const int slot = t < p.win_sinks ? t : p.win_sinks + t % p.win_recent;
          wraw[u] = *reinterpret_cast<const uint4v*>(wb + static_cast<size_t>(slot) * 2 * kHeadDim + 8 * j);
        }
      }
    }
    if (u_f32 >= 0) {
#pragma unroll
      for (int u = 0; u < kWinLd; ++u) {
        if (u == u_f32) {
          const uint4v lo = wraw[u];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            wraw[u][i] = f32_to_bf16_bits(__uint_as_float(lo[2 * i])) |
                         (static_cast<uint32_t>(f32_to_bf16_bits(__uint_as_float(lo[2 * i + 1]))) << 16);
            wraw[u][2 + i] = f32_to_bf16_bits(__uint_as_float(f32_hi[2 * i])) |
                             (static_cast<uint32_t>(f32_to_bf16_bits(__uint_as_float(f32_hi[2 * i + 1]))) << 16);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kQPerThread; ++u) {
      const int idx = min(tid + u * kThreads, kNH * kHeadDim - 1);
      const size_t qi = (out_row0 + min(idx / kHeadDim, g - 1)) * kHeadDim + idx % kHeadDim;
      qwr[u] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.q) +
                                                  (p.q_kind == 0 ? (2 * qi) & ~static_cast<size_t>(3) : 4 * qi));
    }
    if (tid < kHeadDim && p.win_mu != nullptr) wmu = p.win_mu[h * kHeadDim + tid];
  }
  if (win_wg) __syncthreads();  // the per-wave partials were read; the ring takes the window rows
  uint4v* const s_rows = reinterpret_cast<uint4v*>(s_post + kRowsOff);  // 16 chunks per row
  float* const s_wp = s_post + kWpOff;
  uint16_t* const s_qp = reinterpret_cast<uint16_t*>(s_post + kQpOff);
  if (win_wg) {
#pragma unroll
    for (int u = 0; u < kWinLd; ++u) {  // the keys
      const int idx = tid + u * kThreads;
      const int wi = idx >> 5, j = idx & 31;
      if (wi < n_w && j < 16) s_rows[16 * wi + (j ^ (wi & 15))] = wraw[u];
    }
#pragma unroll
    for (int u = 0; u < kQPerThread; ++u) {  // the query rows as given, and their three bf16 parts
      const int idx = tid + u * kThreads;
      const size_t qi = (out_row0 + min(idx / kHeadDim, g - 1)) * kHeadDim + idx % kHeadDim;
      const float qv = p.q_kind == 0 ? bf16_bits_to_f32(static_cast<uint16_t>(qwr[u] >> (16 * (qi & 1))))
                                     : __uint_as_float(qwr[u]);
      if (idx < kNH * kHeadDim) {
        const int jh = idx / kHeadDim, c = idx % kHeadDim;
        float r = jh < g ? qv : 0.0f;
        s_q[jh][c] = r;
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const uint32_t t = __float_as_uint(r) & 0xffff0000u;
          s_qp[(sp * kNH + jh) * kQpStride + c] = static_cast<uint16_t>(t >> 16);
          r -= __uint_as_float(t);
        }
      }
    }
    if (tid < kHeadDim) s_post[kWmuOff + tid] = wmu;
  }
  if (win_wg) __syncthreads();
  if (win_wg) {
    const int hq = lane & 15, kq = lane >> 4;
    // <q_head, mu>, one wave per head
    for (int jh = wave; jh < g; jh += kW) {
      float d = fmaf(s_q[jh][lane], s_post[kWmuOff + lane], s_q[jh][lane + 64] * s_post[kWmuOff + lane + 64]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if (lane == 0) s_post[kWmuOff + kHeadDim + jh] = d;
    }
    // logits <q, k>, 16-row tiles: C lane (a, col) = heads 4a + i, window row 16 tile + col
    for (int tile = wave; 16 * tile < n_w; tile += kW) {
      const int wi = min(16 * tile + hq, n_w - 1);  // B column = window row
      float4v C = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kB = __builtin_bit_cast(bf16x8, s_rows[16 * wi + ((4 * kb + kq) ^ (wi & 15))]);
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const uint4v qa = hq < kNH ? *reinterpret_cast<const uint4v*>(s_qp + (sp * kNH + hq) * kQpStride + 32 * kb +
                                                                        8 * kq)
                                     : uint4v{0u, 0u, 0u, 0u};
          C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa), kB, C, 0, 0, 0);
        }
      }
      const int col = 16 * tile + hq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jh = 4 * kq + i;
        if (jh < g && col < n_w) s_wp[jh * kHeadRow + col] = C[i];
      }
    }
    __syncthreads();
    // the keys were read: the values take their place (the softmax below reads only the logits)
#pragma unroll
    for (int u = 0; u < kWinLd; ++u) {
      const int idx = tid + u * kThreads;
      const int wi = idx >> 5, j = idx & 31;
      if (wi < n_w && j >= 16) s_rows[16 * wi + (j - 16)] = wraw[u];
    }
    // per head (one wave): logits (log2 units) = (<q, k> - <q, mu>) * scale, max, weights
    // exp2(logit - max) split into bf16 hi | lo over the same row (all reads first), their sum
    const int n_wpad = 32 * ((n_w + 31) / 32);
    for (int jh = wave; jh < g; jh += kW) {
      const float qmu = s_post[kWmuOff + kHeadDim + jh];
      float lg[(kWinRowsPad + 63) / 64];
      float m = kNegBig;
#pragma unroll
      for (int r = 0; r < (kWinRowsPad + 63) / 64; ++r) {
        const int wi = lane + 64 * r;
        lg[r] = wi < n_w ? (s_wp[jh * kHeadRow + wi] - qmu) * p.logit_scale : kNegBig;
        m = fmaxf(m, lg[r]);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      float l = 0.0f;
      uint16_t* prow = reinterpret_cast<uint16_t*>(s_wp + jh * kHeadRow);
#pragma unroll
      for (int r = 0; r < (kWinRowsPad + 63) / 64; ++r) {
        const int wi = lane + 64 * r;
        const float e = wi < n_w ? __builtin_amdgcn_exp2f(lg[r] - m) : 0.0f;
        l += e;
        if (wi < n_wpad) {
          const uint32_t t = __float_as_uint(e) & 0xffff0000u;
          prow[wi] = static_cast<uint16_t>(t >> 16);
          prow[kWinRowsPad + 8 + wi] = static_cast<uint16_t>((__float_as_uint(e - __uint_as_float(t))) >> 16);
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
      if (lane == 0) {
        s_post[kWmlOff + 2 * jh] = m;
        s_post[kWmlOff + 2 * jh + 1] = l;
      }
    }
    __syncthreads();
    // value sums: channels 16 cw .. +16 for cw = wave, wave + kW, ..; A = weights (hi, lo), B = values
    for (int cw = wave; cw < kHeadDim / 16; cw += kW) {
      const uint16_t* vrows = reinterpret_cast<const uint16_t*>(s_rows) + 16 * cw + hq;
      const uint16_t* prow = reinterpret_cast<const uint16_t*>(s_wp + (hq < kNH ? hq : 0) * kHeadRow);
      float4v C = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int kb = 0; kb < n_wpad / 32; ++kb) {
        uint4v vv;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int w0 = min(32 * kb + 8 * kq + 2 * e2, n_w - 1), w1 = min(32 * kb + 8 * kq + 2 * e2 + 1, n_w - 1);
          vv[e2] = static_cast<uint32_t>(vrows[w0 * kHeadDim]) | (static_cast<uint32_t>(vrows[w1 * kHeadDim]) << 16);
        }
        const bool live = hq < g;
        const uint4v ph = live ? *reinterpret_cast<const uint4v*>(prow + 32 * kb + 8 * kq) : uint4v{0u, 0u, 0u, 0u};
        const uint4v pl = live ? *reinterpret_cast<const uint4v*>(prow + kWinRowsPad + 8 + 32 * kb + 8 * kq)
                               : uint4v{0u, 0u, 0u, 0u};
        const bf16x8 vB = __builtin_bit_cast(bf16x8, vv);
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph), vB, C, 0, 0, 0);
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl), vB, C, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jh = 4 * kq + i;
        if (jh < g) s_post[kOwOff + jh * kHeadDim + 16 * cw + hq] = C[i];
      }
    }
    __syncthreads();
    // the window rows to the workspace (agent scope, like the split partials)
    for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
      const int jh = idx / kHeadDim, c = idx % kHeadDim;
      float* dst = p.win_part + (out_row0 + jh) * kPartStride;
      __hip_atomic_store(dst + c, s_post[kOwOff + jh * kHeadDim + c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) {
        __hip_atomic_store(dst + 128, s_post[kWmlOff + 2 * jh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 129, s_post[kWmlOff + 2 * jh + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // ---- the last workgroup of (b, h) merges the splits.  The partial stores
  // complete (vmcnt 0) before the ticket is taken; the merging workgroup reads
  // them with agent-scope loads after seeing the last ticket.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_ticket = __hip_atomic_fetch_add(p.counters + b * H + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // R_V rows for the output rotation, requested by every workgroup right after
  // its ticket (the merging one finds them in flight).  Thread (row ri, part
  // rq), rq in the upper lane bits, takes channels [kRows * rq, +kRows) of
  // row ri, in 16-byte chunks rotated by rq so that the kParts lanes sharing a
  // row read different LDS banks of o_rot; the parts are then summed across
  // lanes.  Hadamard: thread oi holds the sign of output channel oi.
  constexpr int kOiW = 64 / kParts;          // output rows per wave
  constexpr int kChunks = kRows / 4;         // 16-byte chunks per part
  constexpr int kChunkRot = 8 / kParts;      // chunk rotation per part
  const bool rot_lane = tid < kParts * kHeadDim;  // whole waves
  const int ri = (tid >> 6) * kOiW + (lane % kOiW);
  const int rq = lane / kOiW;
  const int oi = tid & (kHeadDim - 1);
  float4v rr[kChunks];
  float sgv = 0.0f;
  if (!hadamard) {
    if (rot_lane) {
      const float* Rrow = p.r_v + (static_cast<size_t>(h) * kHeadDim + ri) * kHeadDim + kRows * rq;
#pragma unroll
      for (int u = 0; u < kChunks; ++u)
        rr[u] = *reinterpret_cast<const float4v*>(Rrow + 4 * ((u + kChunkRot * rq) % kChunks));
    }
  } else {
    sgv = p.r_v[h * kHeadDim + oi];
  }
  __syncthreads();
  if (s_ticket != n_valid - 1) return;

  // Merge, in one load round.  When they fit, the split partial rows
  // (contiguous in the workspace) are copied whole into the ring, which is free
  // now, by 16-byte coherent DMA (1 KB per wave instruction).  Otherwise every
  // (split, head) max/sum pair is loaded by one thread and shared through LDS,
  // while thread (head jh, channel c) loads acc[c] of the first kAB splits;
  // this workgroup's own split comes from registers.  With a window, each
  // thread also loads its channel of the head's window row.
  constexpr int kAB = kNQ == 1 ? 32 : 8;  // splits per acc load round
  static_assert(sizeof(s_ring) >= sizeof(float) * 2 * kMaxSplits * kNH, "max/sum pairs fit in the ring");
  const float* pb = p.part + head_base * g * kPartStride;
  float* s_ml = s_post;  // [split][head][2]: max, sum
  const int n_ml = n_valid * g;
  const int n_img = n_ml * kPartStride;  // floats of the partial rows
  // staged rows stay below the window's value sums (kOwOff) when there is a window
  const bool img = n_img + 64 * 4 <= (win_here ? kOwOff : kRingFloats);
  float av[kIdx][kAB];
  auto load_acc = [&](int k, int s0) {
    const int idx = min(tid + k * kThreads, g * kHeadDim - 1);
    const int jh = idx / kHeadDim, c = idx % kHeadDim;
#pragma unroll
    for (int u = 0; u < kAB; ++u) av[k][u] = ld_agent(pb + (min(s0 + u, n_valid - 1) * g + jh) * kPartStride + c);
  };
  float ml0 = 0.0f, ml1 = 0.0f;
  if (img) {
    // chunk ch of 16 B lands at s_post + 4 ch; the last instruction's spare
    // lanes repeat the last chunk into the 1 KB of slack after the rows
    static_assert(kPartStride % 4 == 0, "partial rows are whole 16-byte chunks");
    const int n_ch = n_img / 4;
    for (int c0 = 64 * wave; c0 < n_ch; c0 += 64 * kW)
      dma16_agent(reinterpret_cast<const uint8_t*>(pb), 16 * min(c0 + lane, n_ch - 1), s_post + 4 * c0);
  } else {
    if (tid < n_ml) {
      ml0 = ld_agent(pb + static_cast<size_t>(tid) * kPartStride + 128);  // split tid / g, head tid % g
      ml1 = ld_agent(pb + static_cast<size_t>(tid) * kPartStride + 129);
    }
#pragma unroll
    for (int k = 0; k < kIdx; ++k) load_acc(k, 0);
  }
  // the window row of thread (head, channel): acc, max, sum
  float w_acc[kIdx], w_m[kIdx], w_l[kIdx];
  if (win_here) {
#pragma unroll
    for (int k = 0; k < kIdx; ++k) {
      const int idx = min(tid + k * kThreads, g * kHeadDim - 1);
      const float* wr = p.win_part + (out_row0 + idx / kHeadDim) * kPartStride;
      w_acc[k] = ld_agent(wr + idx % kHeadDim);
      w_m[k] = ld_agent(wr + 128);
      w_l[k] = ld_agent(wr + 129);
    }
  }

  for (int q = tid; q < (img ? 0 : n_ml); q += kThreads) {
    if (q != tid) {  // beyond the first pair per thread
      ml0 = ld_agent(pb + static_cast<size_t>(q) * kPartStride + 128);
      ml1 = ld_agent(pb + static_cast<size_t>(q) * kPartStride + 129);
    }
    s_ml[2 * q] = ml0;
    s_ml[2 * q + 1] = ml1;
  }
  if (img) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial-row copies have landed
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kIdx; ++k) {
    const int idx = tid + k * kThreads;
    if (idx >= g * kHeadDim) break;
    const int jh = idx / kHeadDim;
    const int c = idx % kHeadDim;
    float M = kNegBig, l = 0.0f;
    if (img) {
      // Whole rows in the ring ([split][head][acc 128 | max | sum | pad]).  The
      // 64 lanes of a wave are 64 channels of one head (idx's head is uniform
      // per wave): lane l forms the weight exp2(max_split - M) of splits l,
      // l + 64, ... in registers, and each weight reaches the channel sums as a
      // scalar operand (readlane), with no barrier and no LDS round trip.
      const float* rows = s_post + jh * kPartStride;
      float m = kNegBig;
      for (int sp = lane; sp < n_valid; sp += 64) m = fmaxf(m, rows[sp * g * kPartStride + 128]);
      m = wave_max_all(m);
      float o = 0.0f;
      for (int s0 = 0; s0 < n_valid; s0 += 64) {
        const int sl = min(s0 + lane, n_valid - 1);
        const float w = s0 + lane < n_valid ? __builtin_amdgcn_exp2f(rows[sl * g * kPartStride + 128] - m) : 0.0f;
        l = fmaf(w, rows[sl * g * kPartStride + 129], l);
        // 16 splits per batch: their loads are issued together, then the FMAs
        // in split order (w = 0 past the last split, whose rows read a valid one)
        const int n = min(64, n_valid - s0);
        const float* col = rows + s0 * g * kPartStride + c;
        for (int u0 = 0; u0 < n; u0 += 16) {
          float x[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] = col[min(u0 + e, n - 1) * g * kPartStride];
#pragma unroll
          for (int e = 0; e < 16; ++e)
            o = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u0 + e)), x[e], o);
        }
      }
      l = wave_sum_all(l);
      if (win_here) {  // the window's part: its weight against the splits' max, value sum added after R_V^T
        const float mx = fmaxf(m, w_m[k]);
        const float a = __builtin_amdgcn_exp2f(m - mx), ww = __builtin_amdgcn_exp2f(w_m[k] - mx);
        l = fmaf(a, l, ww * w_l[k]);
        o *= a;
        s_post[kOwOff + jh * kHeadDim + c] = l > 0.0f ? ww * w_acc[k] / l : 0.0f;
      }
      s_q[jh][c] = l > 0.0f ? o / l : 0.0f;  // o_rot
      continue;
    }
    for (int sp = 0; sp < n_valid; ++sp) M = fmaxf(M, s_ml[2 * (sp * g + jh)]);
    const float wm = win_here ? w_m[k] : kNegBig;
    M = fmaxf(M, wm);
    for (int sp = 0; sp < n_valid; ++sp)
      l = fmaf(__builtin_amdgcn_exp2f(s_ml[2 * (sp * g + jh)] - M), s_ml[2 * (sp * g + jh) + 1], l);
    const float ww = __builtin_amdgcn_exp2f(wm - M);  // weight of the window's part
    if (win_here) l = fmaf(ww, w_l[k], l);
    float o = 0.0f;
    for (int s0 = 0; s0 < n_valid; s0 += kAB) {
      if (s0 > 0) load_acc(k, s0);
#pragma unroll
      for (int u = 0; u < kAB; ++u) {
        const int sp = s0 + u;
        if (sp < n_valid)
          o = fmaf(__builtin_amdgcn_exp2f(s_ml[2 * (sp * g + jh)] - M), sp == split ? own_a[k] : av[k][u], o);
      }
    }
    s_q[jh][c] = l > 0.0f ? o / l : 0.0f;  // o_rot
    if (win_here)  // the window's value sum (original basis), added after R_V^T
      s_post[kOwOff + jh * kHeadDim + c] = l > 0.0f ? ww * w_acc[k] / l : 0.0f;
  }
  __syncthreads();

  auto store_out = [&](int jh, int i, float o) {
    if (win_here) o += s_post[kOwOff + jh * kHeadDim + i];
    const size_t oidx = (out_row0 + jh) * kHeadDim + i;
    if (p.out_kind == 0)
      static_cast<uint16_t*>(p.out)[oidx] = f32_to_bf16_bits(o);
    else
      static_cast<float*>(p.out)[oidx] = o;
  };
  if (hadamard) {
    // o = o_rot R_V^T = s_V * WHT(o_rot) / sqrt(128), one vector per (2 waves, pass)
#pragma unroll 1
    for (int pass = 0; pass < kVecPasses; ++pass) {
      const int idx = tid + pass * kThreads;
      const bool act = idx < kNH * kHeadDim;
      const int jh = min(idx / kHeadDim, kNH - 1), i = idx & (kHeadDim - 1);
      const float y = wht128(act ? s_q[jh][i] : 0.0f, i, act ? s_post + jh * kHeadDim : nullptr);
      if (act && jh < g) store_out(jh, i, y * kInvSqrt128 * sgv);
    }
  } else {
  // o = o_rot R_V^T: o[i] = sum_c o_rot[c] R_V[i][c]; thread (ri, rq) sums
  // kRows channels, the kParts lanes of row ri add their sums, and lane part
  // rq stores heads rq, rq + kParts, ...
  static_assert(kParts == 2 || kParts == 4, "the parts of a row sit in lane bit 5, or bits 4..5");
  if (rot_lane) {
    float o[kNH];
#pragma unroll
    for (int jh = 0; jh < kNH; ++jh) o[jh] = 0.0f;
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c0 = kRows * rq + 4 * ((u + kChunkRot * rq) % kChunks);
#pragma unroll
      for (int jh = 0; jh < kNH; ++jh) {
        const float4v qv = *reinterpret_cast<const float4v*>(&s_q[jh][c0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[jh] = fmaf(qv[e], rr[u][e], o[jh]);
      }
    }
#pragma unroll
    for (int jh = 0; jh < kNH; ++jh) {
      float x, y;
      if (kParts == 4) {
        o[jh] = rows_sum(o[jh]);
      } else {
        swap32(o[jh], x, y);
        o[jh] = x + y;
      }
    }
#pragma unroll
    for (int jh = 0; jh < kNH; ++jh)
      if (jh % kParts == rq && jh < g) store_out(jh, ri, o[jh]);
  }
  }  // dense R
  if (tid == 0) __hip_atomic_store(p.counters + b * H + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- launcher
// hipExtLaunchKernel stamps the events with the dispatch's own start and end
// times, so an event pair measures the kernel alone.
template <int kNQ, bool kKW, bool kVW>
static hipError_t launch_one(const DecodeParams& prm, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  constexpr int kW = DecodeShape<kNQ, 3 + kKW + kVW>::waves;
  constexpr int kD = DecodeShape<kNQ, 3 + kKW + kVW>::depth;
  DecodeParams arg = prm;
  void* args[] = {&arg};
  const void* kern = prm.rot_kind == 1 ? reinterpret_cast<const void*>(&decode_kernel<kNQ, kW, kD, kKW, kVW, true>)
                                       : reinterpret_cast<const void*>(&decode_kernel<kNQ, kW, kD, kKW, kVW, false>);
  return hipExtLaunchKernel(kern,
                            dim3((prm.balanced ? 1 : prm.batch) * prm.num_kv_heads * prm.n_splits), dim3(64 * kW),
                            args, 0, stream,
                            ev_begin, ev_end, 0);
}
template <int kNQ>  // instantiated for kNQ = 1 only
static hipError_t launch_narrow(const DecodeParams& prm, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  constexpr int kW = kNarrowWaves, kD = kNarrowDepth, kC = kNarrowWgPerCu;
  DecodeParams arg = prm;
  void* args[] = {&arg};
  const void* kern = prm.rot_kind == 1 ? reinterpret_cast<const void*>(&decode_kernel<1, kW, kD, false, false, true, kC>)
                                       : reinterpret_cast<const void*>(&decode_kernel<1, kW, kD, false, false, false, kC>);
  return hipExtLaunchKernel(kern, dim3(prm.num_kv_heads * prm.n_splits), dim3(64 * kW), args, 0, stream, ev_begin,
                            ev_end, 0);
}

// The decode kernels for g <= 4 kNQ query heads per KV head, for every key
// and value code width and rotation kind; 3- and 4-bit codes of a tensor share
// one kernel (the plane's unused bit is 0).  Each kNQ is instantiated in a
// translation unit of its own (kvq_decode.hip, kvq_decode_g8.hip,
// kvq_decode_g16.hip), so the three compile in parallel.
template <int kNQ>
hipError_t launch_decode_quads(const DecodeParams& prm, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if constexpr (kNQ == 1) {
    if (prm.narrow) return launch_narrow<kNQ>(prm, stream, ev_begin, ev_end);
  }
  const bool kw = prm.kbits > 2, vw = prm.vbits > 2;
  if (kw)
    return vw ? launch_one<kNQ, true, true>(prm, stream, ev_begin, ev_end)
              : launch_one<kNQ, true, false>(prm, stream, ev_begin, ev_end);
  return vw ? launch_one<kNQ, false, true>(prm, stream, ev_begin, ev_end)
            : launch_one<kNQ, false, false>(prm, stream, ev_begin, ev_end);
}
extern template hipError_t launch_decode_quads<1>(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_quads<2>(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_quads<4>(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace kvq
