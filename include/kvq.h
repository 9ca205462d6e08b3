/*
 * kvq.h - C ABI of the rotated INT2 KV-cache library (libkvq.so), gfx950.
 *
 * What it computes.  The method is OptR, "Output-Oriented Rotation for INT2
 * KV-Cache Quantization" (arXiv 2608.02691):
 *   - write path (section 1 and section 3.1, Eq. (4)): a new key is centred by a
 *     fixed per-channel mean mu (an attention-equivalent reparameterisation:
 *     every logit of one query moves by the same constant, so softmax is
 *     unchanged), rotated by a fixed orthogonal matrix R_K, and quantized to
 *     INT2 with Q2(.; c, G); a new value is rotated by R_V and quantized;
 *   - read path (section 3, Eq. (1)-(2); section 3.2, Eq. (5)): softmax
 *     attention of every query head of a GQA group against the quantized
 *     cache.  Because R is orthogonal, <q, x_hat R^T> = <q R, x_hat> and
 *     sum_s p_s (w_hat_s R^T) = (sum_s p_s w_hat_s) R^T, so the kernels rotate
 *     the query once, attend in the rotated basis straight from the packed
 *     codes, and rotate the output back once.
 * Q2 here is asymmetric over G = 32 consecutive rotated channels of one token,
 * with the cache's clip ratio c (1 unless set): mn = c*min and mx = c*max in
 * fp32, scale = (mx - mn)/3 and zero = mn, both stored as fp16 (round to
 * nearest even); code = clamp(rint((x - zero)/scale), 0, 3) computed in IEEE
 * fp32 from the stored fp16 scale and zero; a group whose stored scale is 0
 * gets all-zero codes.  The page names Q2(.; c, G) without defining c; both
 * range ends scaled by c is this library's reading.
 *
 * Geometry supported: head_dim 128, group G = 32, 64 or 128, page 16 tokens,
 * query heads per KV head g = num_q_heads / num_kv_heads with 1 <= g <= 16.
 *
 * Cache layout.  One device buffer ("pool") of num_pages * num_kv_heads blocks
 * of B bytes (B below); block (page p, KV head h) starts at
 * (p*num_kv_heads + h)*B and holds the 16 token slots of that page.  Inside a
 * block:
 *   [0, 1024)    64 records of 16 bytes, record r = 16a + b (a < 4, b < 16)
 *                = little-endian uint32 words K0, K1, V0, V1.
 *                K code of slot s, channel c (kk = c/32, a = (c%32)/8, e = c%8):
 *                  record 16a + s, word K[kk/2], bits 2*(4*(kk%2) + e/2) + 16*(e%2) (+1).
 *                V code of slot s, channel c (t = c/16, b = c%16, a = s/4, i = s%4):
 *                  record 16a + b, word V[i/2], bits 2*t + 16*(i%2) (+1).
 *   [1024, 1024 + M), M = 128*(128/G) (512, 256, 128 bytes for G = 32, 64,
 *                128): 4*128/G records of 32 bytes, record m = 4*grp + a:
 *                for slots s = 4a + i, at +4i the K (fp16 scale, fp16 zero)
 *                pair of channel group grp (channels G*grp .. G*grp + G-1),
 *                at +16+4i the V pair.
 * A slot index is page*16 + offset.  96, 80 or 72 bytes per token per KV head.
 * Caches with 3- or 4-bit keys or values (kvq_cache.key_bits, val_bits)
 * append a high-bit plane per widened tensor, the keys' first (at
 * P_K = 1024 + M), then the values' (at P_V = P_K + the keys' plane size):
 *   4 bits: 512 bytes, record r at P + 8r = words H0, H1 (keys) or VH0, VH1
 *           (values); a code's high two bits sit at the record, word index
 *           and bit of its low two bits.
 *   3 bits: 256 bytes, one word W per record at P + 4r.  Keys: the code at
 *           bit j of word K[w] has its high bit at bit j + w of W; values:
 *           the code of slot 4a + i, channel 16t + b has it at bit 8i + t.
 * So B = 1024 + M + the planes: K2V2 1536 / 1280 / 1152 (G = 32 / 64 / 128),
 * K3V2 1792, K3V3 2048, K4V2 2048, K4V4 2560 (G = 32).
 *
 * Conventions for every call.
 *   - Pointers marked "device" are HIP device (or managed) memory; "host" are
 *     CPU memory.  The library never allocates, frees or keeps caller memory.
 *   - Calls validate their arguments on the host and return KVQ_OK or an error
 *     code without launching anything; kvq_last_error() then describes it.
 *     Kernels run asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the device.  A launch failure returns
 *     KVQ_EHIP (an error left pending by an earlier, unrelated HIP call is
 *     cleared first and not reported).
 *   - The library never exits or aborts.  It holds no mutable global state
 *     besides per-thread error text and a cached compute-unit count.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,       /* null pointer, negative size, inconsistent sizes    */
  KVQ_EUNSUPPORTED = 2, /* geometry other than d=128, G in {32,64,128}, page 16, g<=16 */
  KVQ_ENOSPACE = 3,     /* page pool too small / workspace too small          */
  KVQ_EHIP = 4          /* a HIP runtime call or kernel launch failed         */
} kvq_status;

typedef enum {
  KVQ_BF16 = 0,        /* bfloat16                                              */
  KVQ_F32 = 1,         /* float32                                               */
  KVQ_F32_ROTATED = 2  /* append only: k, v are already centred and rotated fp32
                          rows x = (k - mu) R_K and w = v R_V; only Q2 + packing
                          run (mu, r_k, r_v are ignored and may be NULL)        */
} kvq_dtype;

/* How the rotations r_k, r_v passed to every call are given.
 *   KVQ_ROT_DENSE     fp32 [H_kv][128][128], row-major, any orthogonal R.
 *   KVQ_ROT_HADAMARD  fp32 [H_kv][128] signs s (each +1 or -1) of the
 *                     randomized Hadamard rotation R = diag(s) H / sqrt(128),
 *                     H[i][j] = (-1)^popcount(i & j) (Sylvester), the rotation
 *                     family of QuaRot, one of the two base rotations
 *                     OptR corrects (OptR section 1 and section 2).  The
 *                     kernels apply it as a fast Walsh-Hadamard transform
 *                     (x R = WHT(x * s) / sqrt(128)) instead of a 128 x 128
 *                     product; the bulk matrix-core append is not used. */
typedef enum { KVQ_ROT_DENSE = 0, KVQ_ROT_HADAMARD = 1 } kvq_rotation;

/* Geometry of one layer's packed cache. */
typedef struct {
  int32_t num_kv_heads; /* H_kv >= 1                                          */
  int32_t head_dim;     /* must be 128                                        */
  int32_t group_size;   /* Q2's group size G: 32, 64 or 128 consecutive rotated
                           channels, one (scale, zero) pair per group and
                           tensor (the metadata shrinks with G)               */
  int32_t page_size;    /* must be 16                                         */
  int32_t num_pages;    /* pages in the pool                                  */
  void* pool;           /* device, kvq_pool_bytes(cache) bytes, 16-byte aligned */
  float clip_ratio;     /* Q2's clip ratio c in (0, 1]; 0 selects 1 (no clip)  */
  int32_t rotation;     /* kvq_rotation: how r_k and r_v describe R           */
  int32_t key_bits;     /* bits per key code: 2 (or 0, the default), 3 (K3V2)
                           or 4 (K4V2): the code words hold the low two bits,
                           the keys' plane (256 bytes for 3, 512 for 4) the
                           rest, as the layout above states                  */
  int32_t val_bits;     /* bits per value code: 2 (or 0, the default), 3 (K3V3
                           with 3-bit keys) or 4: the low two bits in the code
                           words, the rest in the values' plane              */
} kvq_cache;

/*
 * Optional exact window next to the INT2 history (OptR section 3.1, the text
 * after Eq. (4): the long history is stored in INT2 while a small BF16 window
 * is kept, and attention uses the keys and values left after the rotated INT2
 * quantization and the BF16 window restore; the page leaves the window's size
 * open).  With a window, positions s < sinks and s >= T - recent of a sequence
 * of length T are attended from their exact bf16 key and value kept in `buf`;
 * every other position from the INT2 cache.  Every token is still quantized
 * into the cache as usual (Q2 acts on each token alone, so the INT2 bytes are
 * the same as if a token were quantized when it leaves the window).
 * A window key's logit is <q, k - mu> * sm_scale: the same offset mu the keys
 * were centred with at append, so that exact and INT2 logits share one
 * constant shift.
 *
 *   sinks   0..8: leading positions kept exact.
 *   recent  0..128: trailing positions kept exact.
 *   batch   sequences the buffer holds (>= the batch of every call using it).
 *   buf     device bf16 [batch][num_kv_heads][sinks + recent][2][128]: slot
 *           t of a position t < sinks, else slot sinks + t % recent; in a slot
 *           the key row, then the value row.  16-byte aligned.
 *   mu      device fp32 [num_kv_heads][128] key offsets, or NULL (zero).
 * A window with sinks == recent == 0 is the same as none.
 */
typedef struct {
  int32_t sinks;
  int32_t recent;
  int32_t batch;
  void* buf;
  const float* mu;
} kvq_window;

/* Bytes of the pool: num_pages * num_kv_heads * B, B the block size of the
 * cache's group size and code widths (1024 + 128*(128/G), plus 256 per 3-bit
 * and 512 per 4-bit plane).  0 if `cache` is NULL, has non-positive sizes or
 * an unsupported group size or width. */
size_t kvq_pool_bytes(const kvq_cache* cache);

/*
 * kvq_quant_append - quantize-append n_tokens new tokens into the cache.
 * OptR section 1 (key centering) and section 3.1, Eq. (4) (z -> Q2(zR)).
 *
 *   k, v      device [n_tokens][H_kv][128] of in_dtype (bf16 or fp32), or the
 *             rotated fp32 rows when in_dtype == KVQ_F32_ROTATED.
 *   slots     device int32 [n_tokens]: page*16 + offset of each token; all
 *             distinct, each in [0, num_pages*16).  Out-of-range slots are
 *             skipped by the kernel (never written).
 *   mu        device fp32 [H_kv][128], the key centre; NULL means 0.
 *   r_k, r_v  device fp32 [H_kv][128][128], row-major, x_rot[j] = sum_i x[i] R[i][j]
 *             (must be orthogonal, not checked); under KVQ_ROT_HADAMARD the
 *             signs [H_kv][128] instead (cache->rotation).
 *   rot_out   optional device fp32 [n_tokens][H_kv][2][128]: receives the
 *             fp32 quantizer inputs (index 0: centred rotated key, 1: rotated
 *             value) exactly as the kernel quantized them.  NULL = not written;
 *             rows of tokens whose slot is skipped are not written either.
 * Writes the K/V codes and fp16 scale/zero of every (token, KV head) into its
 * slot.  Other slots of the same page keep their contents.
 * Input range: every rotated value (k - mu) R_K and v R_V must be finite with
 * |x| <= 65504, and every Q2 group's (max - min) / 3 (times c) at most 65504,
 * so that the fp16 scale and zero are finite; outside that the stored bytes
 * are unspecified.  Inside it every path takes any finite input: fewer than 64
 * raw tokens are rotated with fp32 fused multiply-adds, 64 or more on the
 * matrix cores, each row scaled by its own power of two before it is split
 * into fp16 parts (so no magnitude overflows the split, and the rotation stays
 * within the fp32 rounding bound of a 128-term dot product).
 * Errors: KVQ_EINVAL (NULL cache/pool/k/v/slots, NULL r_k or r_v unless
 * pre-rotated, n_tokens < 0, clip_ratio outside [0, 1], unknown rotation), KVQ_EUNSUPPORTED
 * (geometry), KVQ_EHIP.
 * n_tokens == 0 is a no-op.
 */
kvq_status kvq_quant_append(const kvq_cache* cache, const void* k, const void* v, kvq_dtype in_dtype,
                            int32_t n_tokens, const int32_t* slots, const float* mu, const float* r_k,
                            const float* r_v, float* rot_out, void* stream);

/*
 * kvq_quant_append_err - kvq_quant_append that also reports each token's
 * squared quantization error, the per-token terms of E_rec (OptR section 3.2,
 * Eq. (9)).
 *
 *   sq_err    device fp32 [n_tokens][H_kv][2][2], 16-byte aligned, or NULL:
 *             entry [n][h][t][i] = sum over channels c in [64 i, 64 i + 64) of
 *             (x_c - level_c)^2, the rotated quantizer input of tensor t (0 key,
 *             1 value) minus its INT2 level.  R is orthogonal, so the two halves
 *             add up to ||k - k~||^2 (or ||v - v~||^2) of the effective rows.
 *             Tokens whose slot is skipped are not written.
 * Every other argument, the bytes written to the cache and the errors are those
 * of kvq_quant_append.
 */
kvq_status kvq_quant_append_err(const kvq_cache* cache, const void* k, const void* v, kvq_dtype in_dtype,
                                int32_t n_tokens, const int32_t* slots, const float* mu, const float* r_k,
                                const float* r_v, float* rot_out, float* sq_err, void* stream);

/*
 * kvq_decode_workspace_bytes - device workspace needed by kvq_decode_attn for
 * the same (batch, num_q_heads, num_kv_heads, max_seq_len, num_splits).
 * num_splits 0 selects the automatic split plan (the size covers either
 * launch shape the call may take).  Returns 0 on invalid input.
 * The workspace holds per-(sequence, KV head) ticket counters, the split
 * partials and one row per output row for an exact window's part (used when a
 * window is given).  It must be zero-filled before its first use; every completed
 * call leaves the counters at zero again.  The counters take a fixed prefix of
 * 16 KiB for any call with batch * num_kv_heads <= 4096, so a workspace is
 * reusable without clearing by every such call, whatever its shape; a call
 * with more (sequence, KV head) pairs uses a longer prefix, and a workspace
 * whose calls change that length must be zero-filled again in between.  Calls
 * that share one workspace must not overlap in time (same stream, or ordered
 * by events).
 */
size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t num_splits);

/*
 * kvq_decode_attn - one decode step of GQA attention over the packed cache.
 * OptR section 3, Eq. (1)-(2) and section 3.2, Eq. (5): for query head j of
 * sequence b, with KV head h = j / g and T = seq_lens[b],
 *   o_j = ( sum_{s<T} softmax_s( <q_j R_K,h, x_hat_s> * sm_scale ) w_hat_s ) R_V,h^T
 * where x_hat_s, w_hat_s are the dequantized rotated key/value of position s
 * (the cached keys were centred; the dropped <q_j, mu> moves all logits of j
 * equally).  T == 0 gives a zero output.
 *
 *   q           device [batch][num_q_heads][128] of q_dtype (KVQ_BF16 or KVQ_F32).
 *   page_table  device int32 [batch][max_pages]; entry i of row b is the page
 *               holding positions 16i..16i+15; entries for i < ceil(T/16) must
 *               be in [0, num_pages).  The kernel never reads outside the pool:
 *               a page id outside [0, num_pages) contributes no tokens, and a
 *               length beyond max_pages*16 is cut there.
 *   seq_lens    device int32 [batch], each in [0, max_seq_len] (a longer one
 *               is cut to max_seq_len; kvq_decode_step then appends nothing
 *               for that sequence).
 *   max_seq_len host bound on seq_lens; must satisfy ceil(max_seq_len/16) <= max_pages.
 *   r_k, r_v    device fp32, dense or Hadamard signs as in kvq_quant_append.
 *   sm_scale    logit scale; 0 selects 1/sqrt(128).
 *   out         device [batch][num_q_heads][128] of out_dtype (KVQ_BF16 or
 *               KVQ_F32).  The bf16 output is the fp32 result rounded to
 *               nearest even.
 *   workspace   device, >= kvq_decode_workspace_bytes(...) bytes, 16-byte
 *               aligned, zero-filled before first use (see above).
 *   num_splits  0 = automatic: the kernel reads the batch's lengths and cuts
 *               every sequence into splits of one common size, the smallest
 *               (found in a few refinement rounds) for which all splits of all
 *               (sequence, KV head) pairs fit in one round of workgroups (one
 *               per compute unit; three for a batch of more than one sequence
 *               with g <= 4, 2-bit codes and no window), so short sequences
 *               take few workgroups and long ones many.  Otherwise the requested number of splits per
 *               (sequence, KV head), each sized for max_seq_len.  Either way
 *               a split holds at most 2048 pages and a sequence at most 512
 *               splits, so the count used can differ from the request;
 *               kvq_decode_workspace_bytes follows the same plan.  Lengths
 *               above max_seq_len are cut to max_seq_len.
 *   window      NULL, or an exact window (kvq_window): its positions are
 *               attended from the window buffer (read only here), the others
 *               from the cache.  The buffer's slots of every window position
 *               must hold that position's key and value (kvq_window_fill,
 *               kvq_decode_step).  Any g (up to 16, as without a window).
 * Value range: every scale and zero the cache format stores (any finite fp16).
 * The P.V product runs on the matrix cores with the fp16 operand p * s_v (p a
 * softmax weight, s_v a value group's scale); the kernel keeps that operand in
 * a power-of-two unit per value group, chosen from the largest scale of each
 * run of 32 positions, so it never overflows and, for the positions with that
 * scale, stays normal.  Precision limit: when, within 32 consecutive positions
 * (one page pair) of one value group, the scales span more than about 2^20
 * and the positions with the largest scales weigh less than about 2^-20 of
 * the others, those others' share of the value sum loses precision (an fp16
 * subnormal operand).  Stale slots past a sequence's end and absent pages may
 * hold any bytes: they weigh nothing.
 * Work decomposition: one kernel launch; one workgroup per compute unit
 * (with 2-bit codes 12 waves for g <= 8 and 8 for g <= 16; with a high-bit
 * plane 12 or 8 waves for g <= 4, 8 for g <= 8, else 4; for a batch of g <= 4
 * with 2-bit codes and no window, three 4-wave workgroups per compute unit,
 * which cut the sequences into three times as many splits) streams a split's
 * pages, and
 * the last workgroup of each (sequence, KV head) merges the split partials
 * (log-sum-exp), adds the window's part, and applies R_V^T.
 * Limits: max_seq_len <= 16777216 (512 splits x 2048 pages x 16 tokens).
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ENOSPACE (workspace too small),
 * KVQ_EHIP.  batch == 0 is a no-op.
 */
kvq_status kvq_decode_attn(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                           int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                           float sm_scale, void* out, kvq_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, const kvq_window* window, void* stream);

/*
 * kvq_decode_attn_noalloc - kvq_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under stream capture,
 * serving loops or harnesses that forbid allocation).  It allocates nothing:
 * its workspace is a static device array of 8 MiB per GPU, held by the library
 * until the process ends, whose first 64 KiB hold the merge tickets.  The
 * first call on a device sets the array up (its device address, and the
 * tickets cleared by a kernel on `stream`); every completed call leaves the
 * tickets at zero.  Every call on one GPU shares that array, so calls that
 * overlap in time on one GPU (different streams, or threads) race; keep them
 * ordered.
 * Arguments, results and the other errors are those of kvq_decode_attn (same
 * kernels, same split plan, bit-identical outputs).  KVQ_ENOSPACE when the
 * call needs more than the array holds: batch * num_kv_heads above 16384, or
 * split and window rows above 8 MiB - 64 KiB (for example, 32 query heads of
 * a 128K sequence need about 0.55 MiB).
 */
kvq_status kvq_decode_attn_noalloc(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                                   int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                                   float sm_scale, void* out, kvq_dtype out_dtype, int32_t num_splits,
                                   const kvq_window* window, void* stream);

/*
 * kvq_decode_attn_traced - kvq_decode_attn plus timing events for measurement.
 * Identical arguments, results and errors; in addition, when non-NULL,
 * `ev_begin` and `ev_end` (hipEvent_t created by the caller, with timing)
 * take the start and end timestamps of the attention kernel's own dispatch
 * (the call launches exactly one kernel), so hipEventElapsedTime gives the
 * kernel's duration without launch gaps.  Meant for eager launches; they give
 * no timing inside a stream capture.
 */
kvq_status kvq_decode_attn_traced(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                                  int32_t num_q_heads, const int32_t* page_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t max_seq_len, const float* r_k, const float* r_v,
                                  float sm_scale, void* out, kvq_dtype out_dtype, void* workspace,
                                  size_t workspace_bytes, int32_t num_splits, const kvq_window* window,
                                  void* stream, void* ev_begin, void* ev_end);

/*
 * kvq_decode_step - one decode step in one kernel: quantize-append the newest
 * token of every sequence, then decode attention over the whole context.
 *
 * OptR section 1 (key centering) and section 3.1, Eq. (4) for the append;
 * section 3, Eq. (1)-(2) and section 3.2, Eq. (5) for the attention.  The
 * results are those of kvq_quant_append of the tokens k_new[b], v_new[b] at
 * position seq_lens[b] - 1 of each sequence b (slot page_table[b][t / 16] * 16
 * + t % 16 with t = seq_lens[b] - 1), followed by kvq_decode_attn with the
 * same arguments: the cache bytes written are identical to kvq_quant_append's,
 * and the new token is attended from its packed INT2 levels.  With a window
 * whose positions include seq_lens[b] - 1, the new token is attended exactly
 * instead and also stored into its window slot (bf16; fp32 input rounded to
 * nearest even); it is still quantized into the cache.
 *
 * Arguments: those of kvq_decode_attn_traced, plus
 *   k_new, v_new  device [batch][num_kv_heads][128], dtype kv_dtype (KVQ_BF16
 *                 or KVQ_F32): the newest key and value of each sequence.
 *   mu            device fp32 [num_kv_heads][128] key centre, or NULL (zero).
 * seq_lens[b] counts the new token.  A sequence of length 0 appends nothing
 * and outputs zeros.  If the page holding position seq_lens[b] - 1 is outside
 * [0, num_pages), the token is neither written nor attended (as in
 * kvq_quant_append and kvq_decode_attn), unless a window holds that position:
 * then it is still stored into the window and attended from there.  The slot at that position is
 * overwritten; its previous content is never read.  ev_begin / ev_end are
 * optional timing events as in kvq_decode_attn_traced (NULL for none).
 * Errors: those of kvq_decode_attn; KVQ_EINVAL if k_new or v_new is NULL;
 * KVQ_EUNSUPPORTED for another kv_dtype.
 */
kvq_status kvq_decode_step(const kvq_cache* cache, const void* k_new, const void* v_new, kvq_dtype kv_dtype,
                           const float* mu, const void* q, kvq_dtype q_dtype, int32_t batch, int32_t num_q_heads,
                           const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                           int32_t max_seq_len, const float* r_k, const float* r_v, float sm_scale, void* out,
                           kvq_dtype out_dtype, void* workspace, size_t workspace_bytes, int32_t num_splits,
                           const kvq_window* window, void* stream, void* ev_begin, void* ev_end);

/*
 * kvq_output_error_workspace_bytes - device workspace needed by
 * kvq_output_error for the same (batch, num_q_heads, num_kv_heads,
 * max_seq_len, d_model); 0 on invalid input (batch above 64 included).  It
 * holds ticket counters, split partials and the readout differences; zero-fill
 * it before its first use (completed calls leave the counters at zero, in
 * fixed prefixes for up to 4096 workgroup tickets (batch * num_kv_heads *
 * ceil(g / 8)) and 1024 query heads, so such calls of any shape can reuse it).
 */
size_t kvq_output_error_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t max_seq_len, int32_t d_model);

/*
 * kvq_output_error - OptR section 3.2, Eq. (6)-(10): the output-space error the
 * INT2 cache causes at the decode position of each sequence, split into its
 * key-induced and value-induced terms (Eq. (8)).  For query head j of sequence
 * b (KV head h = j / g), over the positions s < T_b on present pages:
 *   p  = softmax_s(sm_scale <q_j, k_s>)            (exact keys, Eq. (1))
 *   p~ = softmax_s(sm_scale <q_j, k~_s>)           (effective keys, Eq. (5))
 *   dy_k[b][j] = (sum_s (p~_s - p_s) v_s) W_O,j^T   (key-induced)
 *   dy_v[b][j] = (sum_s p~_s (v~_s - v_s)) W_O,j^T  (value-induced)
 *   e_out[b][j] = ||dy_k + dy_v||^2                 (Eq. (10))
 *   e_rec[b][h] = sum_s (||k_s - k~_s||^2 + ||v_s - v~_s||^2)  (Eq. (9))
 * with k~ = x_hat R_K^T + mu and v~ = w_hat R_V^T read from the cache.
 *
 *   cache, q, q_dtype, batch (<= 64), num_q_heads, page_table, max_pages,
 *   seq_lens, max_seq_len, r_k, r_v, sm_scale: as in kvq_decode_attn.
 *   k, v         device [rows][H_kv][128] of kv_dtype (bf16 or fp32), 16-byte
 *                aligned: the exact keys and values; position s of sequence b
 *                is row row_offsets[b] + s.
 *   row_offsets  device int64 [batch].
 *   sq_err       device fp32 [rows][H_kv][2][2] from kvq_quant_append_err
 *                (same row order), or NULL: e_rec is then written as 0.
 *   w_o          device [d_model][H_q * 128] of w_dtype (bf16 or fp32), 16-byte
 *                aligned: the layer's output projection, W_O,j = columns
 *                [128 j, 128 j + 128).
 *   dy_k, dy_v   device fp32 [batch][H_q][d_model].
 *   e_out        device fp32 [batch][H_q].   e_rec  device fp32 [batch][H_kv].
 *   workspace    device, kvq_output_error_workspace_bytes(...) bytes, 16-byte
 *                aligned, zero before first use.
 * Two kernels on `stream`, no allocation, no synchronization.  mu is not
 * needed: <q_j, mu> shifts all effective logits of head j equally.
 * Errors: KVQ_EINVAL (NULL arguments, misalignment, bad shapes), KVQ_EUNSUPPORTED
 * (dtype, g > 16, batch > 64), KVQ_ENOSPACE (workspace too small), KVQ_EHIP.
 */
kvq_status kvq_output_error(const kvq_cache* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                            int32_t num_q_heads, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                            int32_t max_seq_len, const void* k, const void* v, kvq_dtype kv_dtype,
                            const int64_t* row_offsets, const float* sq_err, const float* r_k, const float* r_v,
                            float sm_scale, const void* w_o, kvq_dtype w_dtype, int32_t d_model, float* dy_k,
                            float* dy_v, float* e_out, float* e_rec, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * kvq_window_bytes - bytes of the window buffer of `window` for num_kv_heads
 * KV heads: batch * num_kv_heads * (sinks + recent) * 512.  0 on invalid input
 * (NULL, sinks outside 0..8, recent outside 0..128, batch < 0, num_kv_heads < 1).
 */
size_t kvq_window_bytes(const kvq_window* window, int32_t num_kv_heads);

/*
 * kvq_window_fill - store the exact keys and values of window positions.
 * The window of kvq_window (OptR section 3.1, the BF16 window kept next to
 * the INT2 history).  Token i (sequence seq_ids[i], position positions[i])
 * is stored iff its position is a window position of a sequence of length
 * seq_lens[seq_ids[i]] (t < sinks, or T - recent <= t < T); other tokens are
 * skipped.  Positions must be distinct within a sequence.
 *   k, v        device [n_tokens][num_kv_heads][128], in_dtype KVQ_BF16 (copied
 *               bit for bit) or KVQ_F32 (rounded to bf16, nearest even).
 *   seq_ids, positions  device int32 [n_tokens]; a sequence id outside
 *               [0, window->batch) or a negative position skips the token.
 *   seq_lens    device int32 [window->batch]: the lengths the window is for.
 * Errors: KVQ_EINVAL (NULL arguments, bad window), KVQ_EUNSUPPORTED (dtype),
 * KVQ_EHIP.  n_tokens == 0 is a no-op.
 */
kvq_status kvq_window_fill(const kvq_window* window, int32_t num_kv_heads, const void* k, const void* v,
                           kvq_dtype in_dtype, int32_t n_tokens, const int32_t* seq_ids, const int32_t* positions,
                           const int32_t* seq_lens, void* stream);

/* Page-table policies for kvq_page_table. */
typedef enum {
  KVQ_PT_CONTIGUOUS = 0,  /* sequence b gets the next ceil(T_b/16) pages in order       */
  KVQ_PT_PERMUTED = 1,    /* as contiguous, over a seeded random permutation of the pool */
  KVQ_PT_INTERLEAVED = 2, /* free list = seeded permutation; for page index i = 0,1,...
                             visit the sequences in a fresh seeded order and give one
                             page to each sequence that needs page i                    */
  KVQ_PT_VALIDATE = 3     /* do not write `table`: check it (entries of live pages in
                             [0, num_pages), no page used twice)                       */
} kvq_pt_policy;

/*
 * kvq_page_table - host-only helper that builds (or validates) a page table.
 * The paged, regular cache layout is what rotation keeps compatible with
 * paged serving systems (OptR section 1).
 *
 *   seq_lens   host int32 [batch], each >= 0.
 *   table      host int32 [batch][max_pages]; written (unused entries = -1)
 *              unless policy is KVQ_PT_VALIDATE, where it is only read.
 *   slots_out  optional host int32 [batch]: slot of position seq_lens[b]-1
 *              (-1 when seq_lens[b] == 0).
 * The random stream is splitmix64 seeded with `seed`.
 * Errors: KVQ_EINVAL (bad arguments, or an invalid table under
 * KVQ_PT_VALIDATE), KVQ_ENOSPACE (pool or max_pages too small).
 */
kvq_status kvq_page_table(int32_t policy, uint64_t seed, const int32_t* seq_lens, int32_t batch,
                          int32_t page_size, int32_t num_pages, int32_t max_pages, int32_t* table,
                          int32_t* slots_out);

/* Text describing the last non-OK status returned on the calling thread. */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
