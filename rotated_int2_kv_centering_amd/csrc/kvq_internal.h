// Kernel launchers used by the C ABI (internal to libkvq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

hipError_t launch_append(uint8_t* pool, int num_pages, int num_kv_heads, const void* k, const void* v, int in_kind,
                         int n_tokens, const int32_t* slots, const float* mu, const float* r_k, const float* r_v,
                         float* rot_out, float clip, int rot_kind, int gsize, float* sq_err, int kbits, int vbits,
                         hipStream_t stream);

// Split plan of one decode call.  Fixed plan (an explicit split count): every
// sequence is cut into n_splits splits of pages_per_split pages.  Balanced
// plan (automatic): the kernel sizes the splits from the batch's actual total
// length (pages per split = clamp(ceil(H * total pages / target_wgs), pps_min,
// pps_max)), so that short sequences take fewer workgroups; n_splits is then
// the number of split slots per KV head, an upper bound on the batch's total.
// Exact window fill: bf16 buf [batch][num_kv_heads][sinks + recent][2][128].
hipError_t launch_window_fill(uint16_t* buf, int batch, int num_kv_heads, int sinks, int recent, const void* k,
                              const void* v, int in_kind, int n_tokens, const int32_t* seq_ids,
                              const int32_t* positions, const int32_t* seq_lens, hipStream_t stream);

// Batch of one: the workgroup of the last split also does the step's append
// (rotating, quantizing and packing the new token before its page loop) and
// the exact window's part (after it), each about as long as this many pages of
// the loop take, so that split is planned up to this many pages per extra task
// (at most half a split) shorter than the others.
constexpr int kStepSplitDeficit = 48;

// Pages per split of a batch of one under the automatic plan, from the pages
// p of the sequence and the split size pps0 the balanced plan gives: the same
// split count, with the last split up to extra * kStepSplitDeficit pages
// shorter (extra: 1 for an append, 1 for a window).  Host and kernel both use
// it (the host to guess the page ids of a split before the length is read).
__host__ __device__ inline int step_pages_per_split(int pages, int pps0, int pps_max, int extra) {
  const int n = pages > 0 ? (pages + pps0 - 1) / pps0 : 1;
  if (extra <= 0 || n < 2) return pps0;
  const int want = extra * kStepSplitDeficit;
  const int d = pps0 / 2 < want ? pps0 / 2 : want;
  const int pps = (pages + d + n - 1) / n;  // n * pps >= pages + d, and still n splits
  return pps <= pps_max ? pps : pps0;
}

struct DecodePlan {
  int n_pages_max;      // ceil(max_seq_len / 16)
  bool balanced;
  int pages_per_split;  // fixed plan: pages handled by one workgroup, <= kMaxPagesPerSplit;
                        // balanced: the split size for one sequence of max_seq_len (a guess)
  int n_splits;         // fixed plan: splits per (sequence, KV head); balanced: slots per KV head
  int pps_min, pps_max, target_wgs;  // balanced plan
  bool narrow;          // the narrow decode shape (three 4-wave workgroups per compute unit)
};

// Kernel arguments of the fused decode (passed by value).
struct DecodeParams {
  uint8_t* pool;  // written only by the step form (the new token's slot)
  int num_kv_heads;
  int num_pages;
  const void* q;
  int q_kind;  // 0 bf16, 1 fp32
  int batch;
  int num_q_heads;
  int g;  // query heads per KV head
  const int32_t* page_table;
  int max_pages;
  const int32_t* seq_lens;
  const float* r_k;
  const float* r_v;
  float logit_scale;  // sm_scale * log2(e)
  void* out;
  int out_kind;        // 0 bf16, 1 fp32
  // Split partials, rows of kPartStride floats: fixed plan
  // [batch][num_kv_heads][n_splits][g]; balanced plan [num_kv_heads][n_splits][g],
  // where the splits of sequence b take the slots after those of sequences < b.
  float* part;
  int32_t* counters;   // [batch][num_kv_heads], zero between calls
  int len_cap;         // lengths are cut at min(max_seq_len, max_pages * 16)
  int balanced;        // DecodePlan fields
  int pages_per_split;
  int n_splits;
  int pps_min, pps_max, target_wgs;
  int narrow;  // 1: the narrow shape (three 4-wave workgroups per compute unit; balanced plan, g <= 4)
  // Exact window (win null = none): bf16 [batch'][num_kv_heads][win_sinks +
  // win_recent][2][128]; positions t < win_sinks and t >= T - win_recent are
  // attended from it (logit <q, k - win_mu>), the rest from the pool.  The
  // step form also stores the new token into its slot.
  uint16_t* win;
  int win_sinks, win_recent;
  const float* win_mu;
  float* win_part;  // the window's part per output row [batch * num_q_heads][kPartStride]: acc 128, max, sum
  // Step form: when k_new is non-null, the token at position seq_lens[b] - 1 of
  // every sequence is first quantize-appended from k_new/v_new [batch][H_kv][128]
  // (kv_kind 0 bf16, 1 fp32; mu [H_kv][128] or null) by the workgroup whose
  // split holds that position, and attended from its packed levels.
  const void* k_new;
  const void* v_new;
  int kv_kind;
  const float* mu;
  float clip;  // Q2's clip ratio for the appended token
  int gsize;   // Q2's group size G (32, 64 or 128) for the appended token
  int kbits;   // bits per key code: 2, or 3 / 4 (a high-bit plane after the metadata)
  int vbits;   // bits per value code: 2, or 3 / 4 (a high-bit plane after the keys' one, if any)
  int rot_kind;  // 0: r_k, r_v are dense [H][128][128]; 1: Hadamard, r_k, r_v are signs [H][128]
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);

// The static decode workspace of kvq_decode_attn_noalloc (kvq_noalloc.hip):
// kStaticScratchBytes per GPU, the merge tickets in its first
// kStaticTicketBytes.  static_scratch returns the current device's copy,
// setting it up (address lookup, tickets cleared on `stream`) on first use.
constexpr size_t kStaticScratchBytes = static_cast<size_t>(8) << 20;
constexpr size_t kStaticTicketBytes = static_cast<size_t>(64) << 10;
hipError_t static_scratch(void** out, hipStream_t stream);

// Output-error evaluator (OptR section 3.2, Eq. (6)-(10)).
constexpr int kEvPartStride = 392;   // split partial row: A, B, C [128 each], m_a, l_a, m_q, l_q, e_rec (head 0)
constexpr int kMaxEvalBatch = 64;
constexpr int kMaxEvalSplits = 256;
constexpr int kProjRows = 256;       // rows of W_O per projection workgroup (one per thread)
constexpr int kEvHeads = 8;          // query heads per evaluator workgroup (g = 16 takes two chunks)

struct EvalParams {
  const uint8_t* pool;
  int num_kv_heads, num_pages;
  const void* q;
  int q_kind;  // 0 bf16, 1 fp32
  int batch, num_q_heads, g;
  const int32_t* page_table;
  int max_pages;
  const int32_t* seq_lens;
  int len_cap;
  const void* k;  // exact rows [row][H_kv][128]; sequence b's position s is row row0[b] + s
  const void* v;
  int kv_kind;    // 0 bf16, 1 fp32
  const int64_t* row0;
  const float* sq_err;  // [row][H_kv][2][2] from the append, or null (e_rec = 0)
  const float* r_k;
  const float* r_v;
  int rot_kind;   // 0 dense [H][128][128], 1 Hadamard signs [H][128]
  int gsize;      // Q2's group size G (32, 64 or 128): one metadata pair per G channels
  int kbits;      // bits per key code (3 and 4: a high-bit plane after the metadata)
  int vbits;      // bits per value code (3 and 4: a high-bit plane after the keys' one, if any)
  float sm_scale;
  int n_splits, pages_per_split;
  float* part;             // [B][H_kv][head chunk][n_splits][kEvHeads][kEvPartStride]
  int32_t* counters;       // [B][H_kv][head chunk], zero between calls
  float* dobuf;            // [B][H_q][2][128]: dO_K, dO_V
  float* e_rec;            // [B][H_kv]
  const void* w_o;         // [d_model][H_q * 128]
  int w_kind;              // 0 bf16, 1 fp32
  int d_model, n_chunks;
  float* dy_k;             // [B][H_q][d_model]
  float* dy_v;
  float* e_out;            // [B][H_q]
  float* e_chunk;          // [H_q][n_chunks][kMaxEvalBatch]
  int32_t* proj_counters;  // [H_q], zero between calls
};

hipError_t launch_eval(const EvalParams& p, hipStream_t stream);

}  // namespace kvq
