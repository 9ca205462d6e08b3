// Host side of the C ABI declared in include/kvq.h: argument validation,
// split planning, kernel launches and the host page-table helper.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"
#include "kvq_layout.h"

namespace {

thread_local std::string g_error = "no error";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kHeadDim = 128;
constexpr int kGroupMetadata = 32;  // the block keeps one (scale, zero) pair per 32 channels
constexpr int kPage = 16;
constexpr int kRowStride = 132;  // floats per split partial (acc[128], max, sum, pad)
constexpr int kMaxGroup = 16;
constexpr int kMinPagesPerSplit = 8;
constexpr int kMaxPagesPerSplit = 2048;  // page ids of one split staged in LDS
constexpr int kMaxSplits = 512;         // merge weights of one (sequence, KV head) staged in LDS
constexpr long long kMaxContext = static_cast<long long>(kMaxPagesPerSplit) * kMaxSplits * kPage;

kvq_status check_cache(const kvq_cache* c) {
  if (c == nullptr) return fail(KVQ_EINVAL, "cache is NULL");
  if (c->head_dim != kHeadDim || c->page_size != kPage ||
      (c->group_size != kGroupMetadata && c->group_size != 2 * kGroupMetadata && c->group_size != kHeadDim))
    return fail(KVQ_EUNSUPPORTED,
                "unsupported geometry head_dim=%d group_size=%d page_size=%d (need 128, 32/64/128, 16)", c->head_dim,
                c->group_size, c->page_size);
  if (c->num_kv_heads < 1) return fail(KVQ_EINVAL, "num_kv_heads=%d must be >= 1", c->num_kv_heads);
  if (c->num_pages < 0) return fail(KVQ_EINVAL, "num_pages=%d must be >= 0", c->num_pages);
  if (static_cast<long long>(c->num_pages) * kPage > 0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "num_pages=%d exceeds the int32 slot range", c->num_pages);
  if (c->pool == nullptr && c->num_pages > 0) return fail(KVQ_EINVAL, "cache pool is NULL");
  if (reinterpret_cast<uintptr_t>(c->pool) % 16 != 0) return fail(KVQ_EINVAL, "cache pool must be 16-byte aligned");
  if (c->key_bits != 0 && c->key_bits != 2 && c->key_bits != 3 && c->key_bits != 4)
    return fail(KVQ_EUNSUPPORTED, "key_bits=%d must be 2, 3 or 4 (0 selects 2)", c->key_bits);
  if (c->val_bits != 0 && c->val_bits != 2 && c->val_bits != 3 && c->val_bits != 4)
    return fail(KVQ_EUNSUPPORTED, "val_bits=%d must be 2, 3 or 4 (0 selects 2)", c->val_bits);
  if (c->rotation != KVQ_ROT_DENSE && c->rotation != KVQ_ROT_HADAMARD)
    return fail(KVQ_EINVAL, "rotation=%d must be KVQ_ROT_DENSE or KVQ_ROT_HADAMARD", c->rotation);
  if (!(c->clip_ratio >= 0.0f && c->clip_ratio <= 1.0f))
    return fail(KVQ_EINVAL, "clip_ratio=%g must be in [0, 1] (0 selects 1)", static_cast<double>(c->clip_ratio));
  return KVQ_OK;
}

// Q2's clip ratio of a cache (0 selects 1).
float clip_of(const kvq_cache* c) { return c->clip_ratio == 0.0f ? 1.0f : c->clip_ratio; }
// Bits per key and per value code (0 selects 2).
int kbits_of(const kvq_cache* c) { return c->key_bits > 2 ? c->key_bits : 2; }
int vbits_of(const kvq_cache* c) { return c->val_bits > 2 ? c->val_bits : 2; }
// Bytes of one (page, KV head) block: codes, one metadata pair per group of G
// channels, one high-bit plane per tensor wider than 2 bits (kvq_layout.h).
size_t block_bytes_of(const kvq_cache* c) {
  return static_cast<size_t>(kvq::block_bytes(kbits_of(c), vbits_of(c), c->group_size));
}

// Compute units of the current device, cached per device id (256 when no
// device can be queried, e.g. on a host without a GPU).
int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0) return 256;
  if (static_cast<size_t>(dev) >= cache.size()) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

// Decode workgroups per compute unit: one, with as many waves as a compute unit
// holds for its group size (12 for g <= 4, 8 for g <= 8, else 4); three 4-wave
// workgroups in the narrow shape, taken by batches of g <= 4 with 2-bit codes
// and no window under the balanced plan (finer splits when lengths differ).
bool narrow_shape(int batch, int g, int kbits, int vbits, bool win) {
  return batch > 1 && g <= 4 && kbits == 2 && vbits == 2 && !win;
}

// Splits of one (sequence, KV head) the merging workgroup can stage in LDS
// next to an exact window (kvq_decode.hip lays the window out in the same
// LDS; without a window the limit is kMaxSplits).
int max_splits_with_window(int g) { return g <= 4 ? kMaxSplits : 128; }

bool make_plan(int batch, int num_kv_heads, int max_seq_len, int num_splits, kvq::DecodePlan* plan,
               int max_splits = kMaxSplits, int extra = 0, bool narrow = false) {
  if (batch < 0 || num_kv_heads < 1 || max_seq_len < 0 || num_splits < 0) return false;
  if (max_seq_len > kMaxContext) return false;
  const int n_pages = (max_seq_len + kPage - 1) / kPage;
  const long long n1 = std::max(n_pages, 1);
  plan->n_pages_max = n_pages;
  // no sequence is cut into more than max_splits splits
  const long long pps_floor = (n_pages + max_splits - 1) / max_splits;
  plan->balanced = num_splits == 0 && static_cast<long long>(batch) * n1 <= 0x7fffffffLL;
  plan->narrow = plan->balanced && narrow;
  const long long target = static_cast<long long>(plan->narrow ? 3 : 1) * device_cu_count();
  if (plan->balanced) {
    // The kernel picks pps in [pps_min, pps_max] from the batch's total pages P:
    // pps >= H P / target, or pps = pps_max.  Sequence b takes max(1, ceil(p_b / pps))
    // splits; that sum is below P / pps + B when some sequence is non-empty (and B
    // otherwise), so at most max(ceil(target / H), ceil(B n / pps_max)) + B - 1 slots
    // per KV head are used, and never more than B ceil(n / pps_min).
    const long long pps_min = std::max<long long>(kMinPagesPerSplit, pps_floor);
    const long long pps_max = kMaxPagesPerSplit;
    const long long bound = std::max((target + num_kv_heads - 1) / num_kv_heads,
                                     (static_cast<long long>(batch) * n1 + pps_max - 1) / pps_max) +
                            std::max(batch, 1) - 1;
    const long long per_seq = (n1 + pps_min - 1) / pps_min;
    const long long slots = std::min(bound, static_cast<long long>(std::max(batch, 1)) * per_seq);
    if (slots > 0x7fffffffLL) return false;
    plan->pps_min = static_cast<int>(pps_min);
    plan->pps_max = static_cast<int>(pps_max);
    plan->target_wgs = static_cast<int>(target);
    // the kernel's pps for one sequence of length max_seq_len: its guess of the
    // split size under a batch of one, so page ids load before the length does
    const long long want = (static_cast<long long>(num_kv_heads) * n_pages + target - 1) / target;
    plan->pages_per_split = static_cast<int>(std::min(std::max(want, pps_min), pps_max));
    if (batch == 1)  // the kernel's split size with an append or a window (a shorter last split)
      plan->pages_per_split =
          kvq::step_pages_per_split(n_pages, plan->pages_per_split, static_cast<int>(pps_max), extra);
    plan->n_splits = static_cast<int>(std::max<long long>(slots, 1));
    return true;
  }
  long long pps;
  if (num_splits > 0) {
    pps = (n1 + num_splits - 1) / num_splits;
  } else {
    // fixed plan sized for the longest sequence (only for batches whose page
    // total overflows 32 bits)
    const long long work = static_cast<long long>(std::max(batch, 1)) * num_kv_heads * n1;
    pps = std::max<long long>((work + target - 1) / target, kMinPagesPerSplit);
  }
  pps = std::max<long long>(pps, pps_floor);
  pps = std::min<long long>(pps, kMaxPagesPerSplit);
  pps = std::max<long long>(1, std::min<long long>(pps, n1));
  plan->pages_per_split = static_cast<int>(pps);
  plan->n_splits = std::max(1, (n_pages + plan->pages_per_split - 1) / plan->pages_per_split);
  plan->pps_min = plan->pps_max = plan->target_wgs = 0;
  return true;
}

// The merge tickets take a fixed prefix of the workspace, sized for up to
// kCounterSlots (sequence, KV head) pairs whatever the call's batch, so a
// workspace reused for another shape finds them where every completed call
// leaves them: at zero (a layout that moved with the batch would put one
// call's split partials where a later call reads its tickets).
constexpr size_t kCounterSlots = 4096;
size_t counters_bytes(int batch, int num_kv_heads) {
  const size_t n = std::max(static_cast<size_t>(batch) * num_kv_heads, kCounterSlots);
  return (n * sizeof(int32_t) + 255) / 256 * 256;
}

// Workspace: merge counters, split partial rows, then one window row per output
// row (used when a window is given).
size_t split_rows_bytes(int batch, int num_q_heads, const kvq::DecodePlan& plan) {
  return sizeof(float) * static_cast<size_t>(plan.balanced ? 1 : batch) * num_q_heads * plan.n_splits * kRowStride;
}

size_t workspace_bytes(int batch, int num_q_heads, int num_kv_heads, const kvq::DecodePlan& plan) {
  return counters_bytes(batch, num_kv_heads) + split_rows_bytes(batch, num_q_heads, plan) +
         sizeof(float) * static_cast<size_t>(batch) * num_q_heads * kRowStride;
}

constexpr int kMaxWindowSinks = 8;
constexpr int kMaxWindowRecent = 128;

// A window with no positions is the same as none.
bool window_active(const kvq_window* w) { return w != nullptr && (w->sinks != 0 || w->recent != 0); }

kvq_status check_window(const kvq_window* w) {
  if (w->sinks < 0 || w->sinks > kMaxWindowSinks)
    return fail(KVQ_EINVAL, "window sinks=%d must be in [0, %d]", w->sinks, kMaxWindowSinks);
  if (w->recent < 0 || w->recent > kMaxWindowRecent)
    return fail(KVQ_EINVAL, "window recent=%d must be in [0, %d]", w->recent, kMaxWindowRecent);
  if (w->batch < 0) return fail(KVQ_EINVAL, "window batch=%d must be >= 0", w->batch);
  if (w->buf == nullptr) return fail(KVQ_EINVAL, "window buffer is NULL");
  if (reinterpret_cast<uintptr_t>(w->buf) % 16 != 0) return fail(KVQ_EINVAL, "window buffer must be 16-byte aligned");
  return KVQ_OK;
}

// splitmix64 (Steele, Lea, Flood 2014) as the page allocator's random stream.
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
  }
  uint64_t below(uint64_t n) { return next() % n; }  // n > 0; bias is irrelevant here
};

void shuffle(std::vector<int32_t>& v, SplitMix64& rng) {
  for (size_t i = v.size(); i > 1; --i) std::swap(v[i - 1], v[rng.below(i)]);
}

// Shared body of the decode entry points; k_new == nullptr is plain decode.
kvq_status decode_common(const kvq_cache* cache, const void* k_new, const void* v_new, kvq_dtype kv_dtype,
                         const float* mu, const void* q, kvq_dtype q_dtype, int32_t batch, int32_t num_q_heads,
                         const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                         const float* r_k, const float* r_v, float sm_scale, void* out, kvq_dtype out_dtype,
                         void* workspace, size_t workspace_bytes_, int32_t num_splits, const kvq_window* window,
                         void* stream, void* ev_begin, void* ev_end, size_t ticket_bytes = 0) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (batch < 0) return fail(KVQ_EINVAL, "batch=%d must be >= 0", batch);
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(KVQ_EINVAL, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d", num_q_heads,
                cache->num_kv_heads);
  const int g = num_q_heads / cache->num_kv_heads;
  if (g > kMaxGroup) return fail(KVQ_EUNSUPPORTED, "query heads per KV head g=%d exceeds %d", g, kMaxGroup);
  if (q_dtype != KVQ_BF16 && q_dtype != KVQ_F32) return fail(KVQ_EUNSUPPORTED, "q dtype must be bf16 or fp32");
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32) return fail(KVQ_EUNSUPPORTED, "out dtype must be bf16 or fp32");
  const bool stepping = k_new != nullptr || v_new != nullptr;
  if (stepping && (k_new == nullptr || v_new == nullptr))
    return fail(KVQ_EINVAL, "k_new and v_new must both be non-NULL");
  if (stepping && kv_dtype != KVQ_BF16 && kv_dtype != KVQ_F32)
    return fail(KVQ_EUNSUPPORTED, "new-token dtype must be bf16 or fp32");
  if (max_seq_len < 0) return fail(KVQ_EINVAL, "max_seq_len=%d must be >= 0", max_seq_len);
  if (num_splits < 0) return fail(KVQ_EINVAL, "num_splits=%d must be >= 0", num_splits);
  if (max_pages < (max_seq_len + kPage - 1) / kPage)
    return fail(KVQ_EINVAL, "max_pages=%d cannot hold max_seq_len=%d", max_pages, max_seq_len);
  if (batch > 0 && max_seq_len > 0 && cache->num_pages == 0) return fail(KVQ_ENOSPACE, "cache has no pages");
  if (std::isnan(sm_scale) || std::isinf(sm_scale) || sm_scale < 0.0f)
    return fail(KVQ_EINVAL, "sm_scale must be finite and >= 0");
  if (batch == 0) return KVQ_OK;
  if (q == nullptr || page_table == nullptr || seq_lens == nullptr || r_k == nullptr || r_v == nullptr ||
      out == nullptr || workspace == nullptr)
    return fail(KVQ_EINVAL, "q, page_table, seq_lens, r_k, r_v, out and workspace must be non-NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(KVQ_EINVAL, "workspace must be 16-byte aligned");
  if (static_cast<long long>(batch) * num_q_heads > 0x7fffffffLL / kRowStride)
    return fail(KVQ_EUNSUPPORTED, "batch * num_q_heads too large");

  if (max_seq_len > kMaxContext)
    return fail(KVQ_EUNSUPPORTED, "max_seq_len=%d exceeds the supported %lld", max_seq_len, kMaxContext);
  const bool win = window_active(window);
  if (win) {
    st = check_window(window);
    if (st != KVQ_OK) return st;
    if (window->batch < batch)
      return fail(KVQ_EINVAL, "window holds %d sequences, the call has %d", window->batch, batch);
  }
  kvq::DecodePlan plan;
  if (!make_plan(batch, cache->num_kv_heads, max_seq_len, num_splits, &plan,
                 win ? max_splits_with_window(g) : kMaxSplits, static_cast<int>(stepping) + static_cast<int>(win),
                 narrow_shape(batch, g, kbits_of(cache), vbits_of(cache), win)))
    return fail(KVQ_EINVAL, "cannot plan the decode split");
  // the tickets' prefix: the caller workspace's, or a fixed one (static workspace)
  const size_t tickets = ticket_bytes != 0 ? ticket_bytes : counters_bytes(batch, cache->num_kv_heads);
  if (static_cast<size_t>(batch) * cache->num_kv_heads * sizeof(int32_t) > tickets)
    return fail(KVQ_ENOSPACE, "batch * num_kv_heads = %lld exceeds the %zu tickets of the workspace",
                static_cast<long long>(batch) * cache->num_kv_heads, tickets / sizeof(int32_t));
  const size_t need = workspace_bytes(batch, num_q_heads, cache->num_kv_heads, plan) -
                      counters_bytes(batch, cache->num_kv_heads) + tickets;
  if (workspace_bytes_ < need)
    return fail(KVQ_ENOSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes_, need);
  if (static_cast<long long>(plan.balanced ? 1 : batch) * cache->num_kv_heads * plan.n_splits > 0x7fffffffLL)
    return fail(KVQ_EUNSUPPORTED, "grid too large");

  const float scale = sm_scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(kHeadDim)) : sm_scale;
  kvq::DecodeParams a;
  a.pool = static_cast<uint8_t*>(cache->pool);
  a.num_kv_heads = cache->num_kv_heads;
  a.num_pages = cache->num_pages;
  a.q = q;
  a.q_kind = q_dtype == KVQ_BF16 ? 0 : 1;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.g = g;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.r_k = r_k;
  a.r_v = r_v;
  a.logit_scale = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);  // log2(e)
  a.out = out;
  a.out_kind = out_dtype == KVQ_BF16 ? 0 : 1;
  a.counters = static_cast<int32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + tickets);
  a.len_cap = static_cast<int>(std::min<long long>(max_seq_len, static_cast<long long>(max_pages) * kPage));
  a.balanced = plan.balanced ? 1 : 0;
  a.pages_per_split = plan.pages_per_split;
  a.n_splits = plan.n_splits;
  a.pps_min = plan.pps_min;
  a.pps_max = plan.pps_max;
  a.target_wgs = plan.target_wgs;
  a.narrow = plan.narrow ? 1 : 0;
  a.win = win ? static_cast<uint16_t*>(window->buf) : nullptr;
  a.win_sinks = win ? window->sinks : 0;
  a.win_recent = win ? window->recent : 0;
  a.win_mu = win ? window->mu : nullptr;
  a.win_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + tickets +
                                        split_rows_bytes(batch, num_q_heads, plan));
  a.k_new = stepping ? k_new : nullptr;
  a.v_new = stepping ? v_new : nullptr;
  a.kv_kind = kv_dtype == KVQ_BF16 ? 0 : 1;
  a.clip = clip_of(cache);
  a.gsize = cache->group_size;
  a.kbits = kbits_of(cache);
  a.vbits = vbits_of(cache);
  a.rot_kind = cache->rotation;
  a.mu = mu;
  hipError_t e = kvq::launch_decode(a, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_begin),
                                    static_cast<hipEvent_t>(ev_end));
  if (e != hipSuccess) return hip_fail(e, stepping ? "decode step launch" : "decode launch");
  return KVQ_OK;
}

// Output-error evaluator: split plan and workspace layout.
struct EvalPlan {
  int n_splits, pages_per_split, n_hc, n_chunks;
  size_t counters_off, proj_counters_off, part_off, dobuf_off, echunk_off, total;
};

bool make_eval_plan(int batch, int num_q_heads, int num_kv_heads, int max_seq_len, int d_model, EvalPlan* e) {
  if (batch < 0 || batch > kvq::kMaxEvalBatch || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || max_seq_len < 0 || d_model < 1)
    return false;
  const int g = num_q_heads / num_kv_heads;
  if (g > kMaxGroup) return false;
  const int n_pages = (max_seq_len + kPage - 1) / kPage;
  // about two workgroups per compute unit in all (two fit one CU's LDS for g <= 4)
  const int want = std::max(1, (512 + batch * num_kv_heads - 1) / std::max(1, batch * num_kv_heads));
  int n_splits = std::max(1, std::min({want, std::max(n_pages, 1), kvq::kMaxEvalSplits}));
  e->pages_per_split = std::max(1, (n_pages + n_splits - 1) / n_splits);
  e->n_splits = std::max(1, (n_pages + e->pages_per_split - 1) / e->pages_per_split);
  e->n_hc = (g + kvq::kEvHeads - 1) / kvq::kEvHeads;
  e->n_chunks = (d_model + kvq::kProjRows - 1) / kvq::kProjRows;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t slots = static_cast<size_t>(batch) * num_kv_heads * e->n_hc;
  // both ticket arrays in fixed prefixes (as for decode): up to 4096 workgroup
  // tickets and 1024 projection tickets keep one layout across shapes
  e->counters_off = 0;
  e->proj_counters_off = up(std::max<size_t>(slots, 4096) * 4);
  e->part_off = e->proj_counters_off + up(std::max<size_t>(num_q_heads, 1024) * 4);
  e->dobuf_off = e->part_off + up(slots * e->n_splits * kvq::kEvHeads * kvq::kEvPartStride * 4);
  e->echunk_off = e->dobuf_off + up(static_cast<size_t>(batch) * num_q_heads * 2 * kHeadDim * 4);
  e->total = e->echunk_off + up(static_cast<size_t>(num_q_heads) * e->n_chunks * kvq::kMaxEvalBatch * 4);
  return true;
}

}  // namespace

extern "C" {

size_t kvq_pool_bytes(const kvq_cache* cache) {
  if (cache == nullptr || cache->num_kv_heads <= 0 || cache->num_pages <= 0) return 0;
  const int g = cache->group_size, kb = cache->key_bits, vb = cache->val_bits;
  if (g != 32 && g != 64 && g != 128) return 0;
  if (kb != 0 && (kb < 2 || kb > 4)) return 0;
  if (vb != 0 && (vb < 2 || vb > 4)) return 0;
  return static_cast<size_t>(cache->num_pages) * static_cast<size_t>(cache->num_kv_heads) * block_bytes_of(cache);
}

kvq_status kvq_quant_append(const kvq_cache* cache, const void* k, const void* v, kvq_dtype in_dtype,
                            int32_t n_tokens, const int32_t* slots, const float* mu, const float* r_k,
                            const float* r_v, float* rot_out, void* stream) {
  return kvq_quant_append_err(cache, k, v, in_dtype, n_tokens, slots, mu, r_k, r_v, rot_out, nullptr, stream);
}

kvq_status kvq_quant_append_err(const kvq_cache* cache, const void* k, const void* v, kvq_dtype in_dtype,
                                int32_t n_tokens, const int32_t* slots, const float* mu, const float* r_k,
                                const float* r_v, float* rot_out, float* sq_err, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0) return fail(KVQ_EINVAL, "n_tokens=%d must be >= 0", n_tokens);
  if (in_dtype != KVQ_BF16 && in_dtype != KVQ_F32 && in_dtype != KVQ_F32_ROTATED)
    return fail(KVQ_EUNSUPPORTED, "unsupported input dtype %d", static_cast<int>(in_dtype));
  if (n_tokens == 0) return KVQ_OK;
  if (cache->num_pages == 0) return fail(KVQ_ENOSPACE, "cache has no pages");
  if (k == nullptr || v == nullptr || slots == nullptr) return fail(KVQ_EINVAL, "k, v and slots must be non-NULL");
  if (in_dtype != KVQ_F32_ROTATED && (r_k == nullptr || r_v == nullptr))
    return fail(KVQ_EINVAL, "r_k and r_v must be non-NULL unless the input is pre-rotated");
  const int kind = in_dtype == KVQ_BF16 ? 0 : (in_dtype == KVQ_F32 ? 1 : 2);
  hipError_t e = kvq::launch_append(static_cast<uint8_t*>(cache->pool), cache->num_pages, cache->num_kv_heads, k, v,
                                    kind, n_tokens, slots, mu, r_k, r_v, rot_out, clip_of(cache), cache->rotation,
                                    cache->group_size, sq_err, kbits_of(cache), vbits_of(cache),
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quant_append launch");
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t num_splits) {
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0) return 0;
  // the larger of the two shapes' needs (the call's shape depends on the cache and window)
  kvq::DecodePlan plan, narrow;
  if (!make_plan(batch, num_kv_heads, max_seq_len, num_splits, &plan)) return 0;
  size_t bytes = workspace_bytes(batch, num_q_heads, num_kv_heads, plan);
  if (narrow_shape(batch, num_q_heads / num_kv_heads, 2, 2, false)) {
    if (!make_plan(batch, num_kv_heads, max_seq_len, num_splits, &narrow, kMaxSplits, 0, true)) return 0;
    bytes = std::max(bytes, workspace_bytes(batch, num_q_heads, num_kv_heads, narrow));
  }
  return bytes;
}

kvq_status kvq_decode_attn(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                           int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                           float sm_scale, void* out, kvq_dtype out_dtype, void* workspace, size_t workspace_bytes_,
                           int32_t num_splits, const kvq_window* window, void* stream) {
  return decode_common(cache, nullptr, nullptr, KVQ_BF16, nullptr, q, q_dtype, batch, num_q_heads, page_table,
                       max_pages, seq_lens, max_seq_len, r_k, r_v, sm_scale, out, out_dtype, workspace,
                       workspace_bytes_, num_splits, window, stream, nullptr, nullptr);
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                                   int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                                   float sm_scale, void* out, kvq_dtype out_dtype, int32_t num_splits,
                                   const kvq_window* window, void* stream) {
  // the shape is checked against the static workspace before the device is touched
  if (cache != nullptr && batch > 0 && cache->num_kv_heads > 0 && num_q_heads > 0 &&
      num_q_heads % cache->num_kv_heads == 0) {
    kvq::DecodePlan plan;
    const int g = num_q_heads / cache->num_kv_heads;
    const bool win = window_active(window);
    if (make_plan(batch, cache->num_kv_heads, max_seq_len, num_splits, &plan,
                  win ? max_splits_with_window(g) : kMaxSplits, win ? 1 : 0,
                  narrow_shape(batch, g, kbits_of(cache), vbits_of(cache), win))) {
      const size_t need = kvq::kStaticTicketBytes + split_rows_bytes(batch, num_q_heads, plan) +
                          sizeof(float) * static_cast<size_t>(batch) * num_q_heads * kRowStride;
      if (need > kvq::kStaticScratchBytes)
        return fail(KVQ_ENOSPACE, "the call needs %zu bytes of workspace, above the static workspace's %zu", need,
                    kvq::kStaticScratchBytes);
      if (static_cast<size_t>(batch) * cache->num_kv_heads * sizeof(int32_t) > kvq::kStaticTicketBytes)
        return fail(KVQ_ENOSPACE, "batch * num_kv_heads = %lld exceeds the static workspace's %zu tickets",
                    static_cast<long long>(batch) * cache->num_kv_heads, kvq::kStaticTicketBytes / sizeof(int32_t));
    }
  }
  void* ws = nullptr;
  if (batch > 0) {
    const hipError_t e = kvq::static_scratch(&ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "static workspace set-up");
  }
  return decode_common(cache, nullptr, nullptr, KVQ_BF16, nullptr, q, q_dtype, batch, num_q_heads, page_table,
                       max_pages, seq_lens, max_seq_len, r_k, r_v, sm_scale, out, out_dtype, ws,
                       kvq::kStaticScratchBytes, num_splits, window, stream, nullptr, nullptr,
                       kvq::kStaticTicketBytes);
}

kvq_status kvq_decode_attn_traced(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                                  int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                                  float sm_scale, void* out, kvq_dtype out_dtype, void* workspace,
                                  size_t workspace_bytes_, int32_t num_splits, const kvq_window* window,
                                  void* stream, void* ev_begin, void* ev_end) {
  return decode_common(cache, nullptr, nullptr, KVQ_BF16, nullptr, q, q_dtype, batch, num_q_heads, page_table,
                       max_pages, seq_lens, max_seq_len, r_k, r_v, sm_scale, out, out_dtype, workspace,
                       workspace_bytes_, num_splits, window, stream, ev_begin, ev_end);
}

kvq_status kvq_decode_step(const kvq_cache* cache, const void* k_new, const void* v_new, kvq_dtype kv_dtype,
                           const float* mu, const void* q, kvq_dtype q_dtype, int32_t batch, int32_t num_q_heads,
                           const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                           int32_t max_seq_len, const float* r_k, const float* r_v, float sm_scale, void* out,
                           kvq_dtype out_dtype, void* workspace, size_t workspace_bytes_, int32_t num_splits,
                           const kvq_window* window, void* stream, void* ev_begin, void* ev_end) {
  if (k_new == nullptr || v_new == nullptr) return fail(KVQ_EINVAL, "k_new and v_new must be non-NULL");
  return decode_common(cache, k_new, v_new, kv_dtype, mu, q, q_dtype, batch, num_q_heads, page_table, max_pages,
                       seq_lens, max_seq_len, r_k, r_v, sm_scale, out, out_dtype, workspace, workspace_bytes_,
                       num_splits, window, stream, ev_begin, ev_end);
}

size_t kvq_output_error_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t max_seq_len, int32_t d_model) {
  EvalPlan e;
  if (!make_eval_plan(batch, num_q_heads, num_kv_heads, max_seq_len, d_model, &e)) return 0;
  return e.total;
}

kvq_status kvq_output_error(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                            int32_t num_q_heads, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                            int32_t max_seq_len, const void* k, const void* v, kvq_dtype kv_dtype,
                            const int64_t* row_offsets, const float* sq_err, const float* r_k, const float* r_v,
                            float sm_scale, const void* w_o, kvq_dtype w_dtype, int32_t d_model, float* dy_k,
                            float* dy_v, float* e_out, float* e_rec, void* workspace, size_t workspace_bytes_,
                            void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (batch < 0) return fail(KVQ_EINVAL, "batch=%d must be >= 0", batch);
  if (batch > kvq::kMaxEvalBatch)
    return fail(KVQ_EUNSUPPORTED, "batch=%d exceeds the evaluator's %d", batch, kvq::kMaxEvalBatch);
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(KVQ_EINVAL, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d", num_q_heads,
                cache->num_kv_heads);
  const int g = num_q_heads / cache->num_kv_heads;
  if (g > kMaxGroup) return fail(KVQ_EUNSUPPORTED, "query heads per KV head g=%d exceeds %d", g, kMaxGroup);
  if (q_dtype != KVQ_BF16 && q_dtype != KVQ_F32) return fail(KVQ_EUNSUPPORTED, "q dtype must be bf16 or fp32");
  if (kv_dtype != KVQ_BF16 && kv_dtype != KVQ_F32) return fail(KVQ_EUNSUPPORTED, "k/v dtype must be bf16 or fp32");
  if (w_dtype != KVQ_BF16 && w_dtype != KVQ_F32) return fail(KVQ_EUNSUPPORTED, "w_o dtype must be bf16 or fp32");
  if (d_model < 1) return fail(KVQ_EINVAL, "d_model=%d must be >= 1", d_model);
  if (max_seq_len < 0) return fail(KVQ_EINVAL, "max_seq_len=%d must be >= 0", max_seq_len);
  if (max_seq_len > kMaxContext)
    return fail(KVQ_EUNSUPPORTED, "max_seq_len=%d exceeds the supported %lld", max_seq_len, kMaxContext);
  if (max_pages < (max_seq_len + kPage - 1) / kPage)
    return fail(KVQ_EINVAL, "max_pages=%d cannot hold max_seq_len=%d", max_pages, max_seq_len);
  if (std::isnan(sm_scale) || std::isinf(sm_scale) || sm_scale < 0.0f)
    return fail(KVQ_EINVAL, "sm_scale must be finite and >= 0");
  if (batch == 0) return KVQ_OK;
  if (batch > 0 && max_seq_len > 0 && cache->num_pages == 0) return fail(KVQ_ENOSPACE, "cache has no pages");
  if (q == nullptr || page_table == nullptr || seq_lens == nullptr || k == nullptr || v == nullptr ||
      row_offsets == nullptr || r_k == nullptr || r_v == nullptr || w_o == nullptr || dy_k == nullptr ||
      dy_v == nullptr || e_out == nullptr || e_rec == nullptr || workspace == nullptr)
    return fail(KVQ_EINVAL, "q, page_table, seq_lens, k, v, row_offsets, r_k, r_v, w_o, dy_k, dy_v, e_out, e_rec "
                            "and workspace must be non-NULL (only sq_err may be NULL)");
  for (const void* a : {static_cast<const void*>(k), static_cast<const void*>(v), static_cast<const void*>(sq_err),
                        static_cast<const void*>(w_o), static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(a) % 16 != 0)
      return fail(KVQ_EINVAL, "k, v, sq_err, w_o and workspace must be 16-byte aligned");
  EvalPlan plan;
  if (!make_eval_plan(batch, num_q_heads, cache->num_kv_heads, max_seq_len, d_model, &plan))
    return fail(KVQ_EUNSUPPORTED, "unsupported evaluator shape");
  if (workspace_bytes_ < plan.total)
    return fail(KVQ_ENOSPACE, "workspace of %zu bytes is below the %zu needed", workspace_bytes_, plan.total);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kvq::EvalParams a{};
  a.pool = static_cast<const uint8_t*>(cache->pool);
  a.num_kv_heads = cache->num_kv_heads;
  a.num_pages = cache->num_pages;
  a.q = q;
  a.q_kind = q_dtype == KVQ_BF16 ? 0 : 1;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.g = g;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.len_cap = std::min<long long>(max_seq_len, static_cast<long long>(max_pages) * kPage);
  a.k = k;
  a.v = v;
  a.kv_kind = kv_dtype == KVQ_BF16 ? 0 : 1;
  a.row0 = row_offsets;
  a.sq_err = sq_err;
  a.r_k = r_k;
  a.r_v = r_v;
  a.rot_kind = cache->rotation;
  a.gsize = cache->group_size;
  a.kbits = kbits_of(cache);
  a.vbits = vbits_of(cache);
  a.sm_scale = sm_scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(kHeadDim)) : sm_scale;
  a.n_splits = plan.n_splits;
  a.pages_per_split = plan.pages_per_split;
  a.part = reinterpret_cast<float*>(ws + plan.part_off);
  a.counters = reinterpret_cast<int32_t*>(ws + plan.counters_off);
  a.dobuf = reinterpret_cast<float*>(ws + plan.dobuf_off);
  a.e_rec = e_rec;
  a.w_o = w_o;
  a.w_kind = w_dtype == KVQ_BF16 ? 0 : 1;
  a.d_model = d_model;
  a.n_chunks = plan.n_chunks;
  a.dy_k = dy_k;
  a.dy_v = dy_v;
  a.e_out = e_out;
  a.e_chunk = reinterpret_cast<float*>(ws + plan.echunk_off);
  a.proj_counters = reinterpret_cast<int32_t*>(ws + plan.proj_counters_off);
  hipError_t e = kvq::launch_eval(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "output_error launch");
  return KVQ_OK;
}

size_t kvq_window_bytes(const kvq_window* window, int32_t num_kv_heads) {
  if (window == nullptr || num_kv_heads < 1 || window->batch < 0 || window->sinks < 0 ||
      window->sinks > kMaxWindowSinks || window->recent < 0 || window->recent > kMaxWindowRecent)
    return 0;
  return static_cast<size_t>(window->batch) * num_kv_heads * (window->sinks + window->recent) * 2 * kHeadDim *
         sizeof(uint16_t);
}

kvq_status kvq_window_fill(const kvq_window* window, int32_t num_kv_heads, const void* k, const void* v,
                           kvq_dtype in_dtype, int32_t n_tokens, const int32_t* seq_ids, const int32_t* positions,
                           const int32_t* seq_lens, void* stream) {
  if (window == nullptr) return fail(KVQ_EINVAL, "window is NULL");
  if (num_kv_heads < 1) return fail(KVQ_EINVAL, "num_kv_heads=%d must be >= 1", num_kv_heads);
  if (n_tokens < 0) return fail(KVQ_EINVAL, "n_tokens=%d must be >= 0", n_tokens);
  if (in_dtype != KVQ_BF16 && in_dtype != KVQ_F32)
    return fail(KVQ_EUNSUPPORTED, "window input dtype must be bf16 or fp32");
  if (!window_active(window)) return KVQ_OK;  // no positions to keep
  kvq_status st = check_window(window);
  if (st != KVQ_OK) return st;
  if (n_tokens == 0 || window->batch == 0) return KVQ_OK;
  if (k == nullptr || v == nullptr || seq_ids == nullptr || positions == nullptr || seq_lens == nullptr)
    return fail(KVQ_EINVAL, "k, v, seq_ids, positions and seq_lens must be non-NULL");
  hipError_t e = kvq::launch_window_fill(static_cast<uint16_t*>(window->buf), window->batch, num_kv_heads,
                                         window->sinks, window->recent, k, v, in_dtype == KVQ_BF16 ? 0 : 1, n_tokens,
                                         seq_ids, positions, seq_lens, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "window_fill launch");
  return KVQ_OK;
}

kvq_status kvq_page_table(int32_t policy, uint64_t seed, const int32_t* seq_lens, int32_t batch, int32_t page_size,
                          int32_t num_pages, int32_t max_pages, int32_t* table, int32_t* slots_out) {
  if (batch < 0 || num_pages < 0 || max_pages < 0) return fail(KVQ_EINVAL, "negative size");
  if (page_size != kPage) return fail(KVQ_EUNSUPPORTED, "page_size must be 16");
  if (batch > 0 && (seq_lens == nullptr || table == nullptr)) return fail(KVQ_EINVAL, "seq_lens and table required");
  if (policy < KVQ_PT_CONTIGUOUS || policy > KVQ_PT_VALIDATE) return fail(KVQ_EINVAL, "unknown policy %d", policy);
  std::vector<int32_t> need(batch);
  long long total = 0;
  int most = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0) return fail(KVQ_EINVAL, "seq_lens[%d]=%d is negative", b, seq_lens[b]);
    need[b] = (seq_lens[b] + kPage - 1) / kPage;
    total += need[b];
    most = std::max(most, need[b]);
  }
  if (most > max_pages) return fail(KVQ_ENOSPACE, "a sequence needs %d pages but max_pages=%d", most, max_pages);
  if (total > num_pages) return fail(KVQ_ENOSPACE, "sequences need %lld pages but the pool has %d", total, num_pages);

  if (policy == KVQ_PT_VALIDATE) {
    std::vector<uint8_t> used(num_pages, 0);
    for (int b = 0; b < batch; ++b)
      for (int i = 0; i < need[b]; ++i) {
        const int32_t p = table[static_cast<size_t>(b) * max_pages + i];
        if (p < 0 || p >= num_pages)
          return fail(KVQ_EINVAL, "table[%d][%d]=%d outside [0, %d)", b, i, p, num_pages);
        if (used[p]) return fail(KVQ_EINVAL, "page %d is used twice (table[%d][%d])", p, b, i);
        used[p] = 1;
      }
  } else {
    std::vector<int32_t> order(num_pages);
    for (int i = 0; i < num_pages; ++i) order[i] = i;
    SplitMix64 rng{seed};
    if (policy != KVQ_PT_CONTIGUOUS) shuffle(order, rng);
    for (size_t i = 0; i < static_cast<size_t>(batch) * max_pages; ++i) table[i] = -1;
    size_t next = 0;
    if (policy == KVQ_PT_INTERLEAVED) {
      std::vector<int32_t> seqs(batch);
      for (int i = 0; i < most; ++i) {
        for (int b = 0; b < batch; ++b) seqs[b] = b;
        shuffle(seqs, rng);
        for (int b : seqs)
          if (i < need[b]) table[static_cast<size_t>(b) * max_pages + i] = order[next++];
      }
    } else {
      for (int b = 0; b < batch; ++b)
        for (int i = 0; i < need[b]; ++i) table[static_cast<size_t>(b) * max_pages + i] = order[next++];
    }
  }
  if (slots_out != nullptr)
    for (int b = 0; b < batch; ++b) {
      const int32_t t = seq_lens[b] - 1;
      slots_out[b] = t < 0 ? -1 : table[static_cast<size_t>(b) * max_pages + t / kPage] * kPage + t % kPage;
    }
  return KVQ_OK;
}

const char* kvq_last_error(void) { return g_error.c_str(); }

}  // extern "C"
