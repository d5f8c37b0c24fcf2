/*
 * jl_bifocal.h -- C ABI of the MI355X (gfx950) bifocal-attention library.
 *
 * The operation is the attention of Jet-Long's Dynamic Bifocal RoPE
 * (arXiv 2607.07740), as described by:
 *   - ResearchPod summary (researchpod.app), 2nd paragraph: nearby keys are scored
 *     with the base RoPE; distant positions are folded onto a coarser grid whose
 *     step g is the least integer that holds every folded position inside the
 *     positions seen in training; three FlashAttention-style passes are combined
 *     by inclusion-exclusion in one fused kernel.
 *   - ResearchPod transcript, exchange on the cache: the cache holds every key at
 *     the position it was written at, and the folding is applied when the key is
 *     read.
 *   - ResearchPod transcript, exchange on prefill: the merged result is built from
 *     the near keys at base positions, all keys at folded positions, and the near
 *     keys at folded positions (subtracted).
 *   - Abstract (engineersofai.com paper page): at short inputs the base model is
 *     recovered exactly; the merge and the rotation that moves cached vectors to
 *     their folded positions are computed inside the attention kernel.
 *   - seventnews.com, "How bifocal attention sidesteps the fixed-scaling trap":
 *     the long-range factor follows the length s of the sequence at hand.
 *
 * Definitions used by every entry point (head size D = 128):
 *   s      = n_kv, the number of keys in context (cache index == position).
 *   p_i    = n_kv - n_q + i, position of query row i (the newest n_q tokens),
 *            or q_pos[i] where an entry point takes explicit positions.
 *   theta_d= rope_base^(-2d/D), rotate-half pairs (d, d + D/2).
 *   g      = jl_group_factor(s, L) = smallest integer >= 1 with
 *            floor((s-1)/g) <= L-1  (== max(1, ceil(s/L))).
 *   c(p)   = floor(p/g) - p (the correction rotation moves a vector cached at
 *            position p to its aliased position floor(p/g)).
 *   local  : 0 <= p_i - j <= W-1 (W keys including the query itself);
 *   remote : j <= p_i - W.
 *   Pass A = local keys, scores tau * q_i.k_j (base RoPE, as cached).
 *   Pass B = all causal keys, scores tau * rot(q_i, c(p_i)th).rot(k_j, c(j)th).
 *   Pass C = local keys, the scores of pass B.
 *   out    = (w_A O_A + w_B O_B - w_C O_C) / (w_A + w_B - w_C), w_X = exp(lse_X - M).
 *   tau    = softmax_scale, or 1/sqrt(D) when softmax_scale <= 0.
 *
 * Layout: every tensor is dense, row-major, "BSHD": q/out [B, n_q, Hq, D],
 * k/v [B, n_kv, Hkv, D], element type bfloat16; lse is fp32 [B, Hq, n_q]
 * (natural log).  Query head h reads KV head h / (Hq / Hkv).  Device pointers
 * must be 16-byte aligned.
 *
 * Ownership and synchronisation: the caller owns every buffer.  The library
 * never allocates or frees device memory and never synchronises the host;
 * all work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 * default stream) and buffers must stay valid until the stream has finished.
 * Device contents are not inspected on the host.
 *
 * Errors: every jl_status-returning call validates its host-visible arguments
 * before touching the device.  On error nothing is enqueued, the status is
 * returned and jl_last_error() holds a message (thread-local, valid until the
 * next call on the same thread).  No call aborts or throws.
 */
#ifndef JL_BIFOCAL_H
#define JL_BIFOCAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t jl_status;

#define JL_OK              0
#define JL_ERR_INVALID_ARG 1 /* null/misaligned pointer, size < 1, n_q > n_kv, Hq % Hkv != 0,
                                L < 1, W < 1, W > L, rope_base <= 1 or not finite            */
#define JL_ERR_UNSUPPORTED 2 /* head_dim != 128, n_kv_heads > 65536, or sizes whose element offsets overflow int64 */
#define JL_ERR_WORKSPACE   3 /* workspace smaller than the matching *_workspace_size result    */
#define JL_ERR_DEVICE      4 /* no HIP device, or a HIP error reported at launch              */

/* Message for the last non-OK status on this thread ("" if none). */
const char* jl_last_error(void);

/* g(s): smallest integer g >= 1 with floor((s-1)/g) <= L-1, i.e. every aliased
 * position floor(p/g), p < s, falls inside the pretrained positions 0..L-1
 * (ResearchPod summary, 2nd paragraph: the factor is the least integer that
 * keeps the folded positions inside the trained range).
 * Pure integer host function.  Returns 0 if seq_len < 1 or pretrained_window < 1. */
int64_t jl_group_factor(int64_t seq_len, int64_t pretrained_window);

/* Bifocal prefill (or a chunk of queries against a longer context), in one
 * kernel launch.
 *   q     : bf16 [B, n_q, Hq, D], rotated at positions p_i (as the model produced them)
 *   k, v  : bf16 [B, n_kv, Hkv, D], k rotated at its original positions 0..n_kv-1
 *   out   : bf16 [B, n_q, Hq, D] (written)
 *   lse   : fp32 [B, Hq, n_q] natural-log normaliser of the merged softmax, or NULL
 *   q_pos : NULL: row i sits at p_i = n_kv - n_q + i (the newest n_q tokens).
 *           Otherwise a device int32 [n_q], 4-byte aligned, nondecreasing, each
 *           in [0, n_kv), shared by every sequence of the batch: row i sits at
 *           q_pos[i] (ResearchPod transcript, cache exchange: keys keep their
 *           original positions, so any query position can be scored against
 *           them).  Not read on the host: entries outside the contract give an
 *           unspecified result, never an access out of range (positions are
 *           clamped into [0, n_kv)).
 * g = jl_group_factor(n_kv, L).  When g == 1 every remote rotation is the
 * original one and the call runs jl_plain_prefill (bitwise identical results:
 * the base model, Abstract: exact recovery at short inputs).  Otherwise the
 * kernel rotates q and each staged key tile by the correction c(p) on the fly
 * (the corrected keys never leave LDS) and evaluates the three-pass merge above.
 * Requires 1 <= W <= L.  Errors: as listed above, plus JL_ERR_INVALID_ARG for a
 * misaligned q_pos. */
jl_status jl_bifocal_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                             int64_t pretrained_window, int64_t local_window, double rope_base,
                             float softmax_scale, void* stream);

/* Bytes of device workspace jl_bifocal_prefill_ws needs: one corrected copy of
 * the keys, bf16 [B, n_kv, Hkv, D].  0 for invalid sizes. */
size_t jl_bifocal_prefill_workspace_size(int32_t batch, int32_t n_kv, int32_t n_kv_heads, int32_t head_dim);

/* Same result as jl_bifocal_prefill (same arguments, layouts and rounding of the
 * corrected keys) computed in two launches: an elementwise pass first writes
 * k^g_j = rot(k_j, c(j) theta) for every cached key to `workspace` (bf16,
 * layout of k), then the attention kernel stages those corrected keys like
 * plain keys instead of rotating every key tile once per query block.  The
 * cache itself is not modified.  This departs from the method as described,
 * which corrects the keys inside the one attention kernel (jl_bifocal_prefill);
 * it keeps a corrected copy of the keys for the duration of the call and
 * trades that workspace for speed.  Always uses the newest-rows positions.
 *   workspace       : device memory, 16-byte aligned, owned by the caller; it
 *                     may be NULL when g(n_kv) == 1 (the plain path needs none),
 *                     otherwise NULL or misaligned is JL_ERR_INVALID_ARG
 *   workspace_bytes : >= jl_bifocal_prefill_workspace_size(...), else
 *                     JL_ERR_WORKSPACE
 * The workspace contents are scratch: overwritten by every call. */
jl_status jl_bifocal_prefill_ws(const void* q, const void* k, const void* v, void* out, float* lse,
                                int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                int64_t local_window, double rope_base, float softmax_scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Plain causal RoPE attention built with the same kernel skeleton (the base
 * model; denominator of the "overhead vs plain" and "vs plain causal"
 * comparisons).  Same layouts and q_pos contract as jl_bifocal_prefill. */
jl_status jl_plain_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           float softmax_scale, void* stream);

/* Sliding-window attention: query row i attends to the keys j with
 * 0 <= p_i - j <= W-1 on the cached vectors (base RoPE), one softmax per row.
 * It serves the sliding-window layers of hybrid models, which keep such layers
 * next to the global ones (seventnews.com, "Generalization to hybrid attention
 * architectures"): a window W <= L never leaves the pretrained positions, so
 * those layers need no correction -- it is the local view (pass A) on its own.
 * Same layouts as jl_bifocal_prefill; local_window >= 1 (a window of at least
 * n_kv keys is plain causal attention).  Tiles wholly outside every row's
 * window are not read. */
jl_status jl_sliding_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                             int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int64_t local_window,
                             float softmax_scale, void* stream);

/* Per-pass results of the three FlashAttention-style passes of the merge
 * (ResearchPod transcript, prefill exchange: A, the near keys at base positions;
 * B, all keys at folded positions; C, the near keys at folded positions), each
 * normalised on its own key set:
 *   out_abc : fp32 [3, B, n_q, Hq, D]   (pass A, then B, then C)
 *   lse_abc : fp32 [3, B, Hq, n_q]      natural log; -inf for an empty key set
 * For checking and debugging; slower than jl_bifocal_prefill.  Runs the three
 * passes for every g, including g == 1. */
jl_status jl_bifocal_prefill_passes(const void* q, const void* k, const void* v, float* out_abc,
                                    float* lse_abc, int32_t batch, int32_t n_q, int32_t n_kv,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t pretrained_window, int64_t local_window,
                                    double rope_base, float softmax_scale, void* stream);

/* The merge in its literal form: the same three passes in one kernel sweep over
 * shared LDS tiles, each with its own running maximum and normaliser, combined
 * in the epilogue by their log-sum-exp weights with C subtracted (Abstract and
 * ResearchPod summary, 2nd paragraph: the views are joined without counting the
 * near keys twice):  Z = e_A + e_B - e_C,  O = (e_A O_A + e_B O_B - e_C O_C) / Z,
 * e_X = exp(lse_X - max lse),  lse = max lse + ln Z.
 * Same arguments, layouts and errors as jl_bifocal_prefill without q_pos (rows
 * sit at n_kv - n_q + i):  out bf16 [B, n_q, Hq, D];  lse fp32 [B, Hq, n_q] or
 * NULL.  It equals jl_bifocal_prefill up to rounding (that kernel folds the
 * three passes into one softmax with a shared maximum); it runs the three
 * passes for every g, including g == 1, and is slower.  Subtracting C cancels:
 * where the near keys' grouped weight exceeds everything else by ~1e7, the
 * literal form loses the difference to fp32 rounding, which the shared-maximum
 * form never computes.  For checking. */
jl_status jl_bifocal_prefill_three_pass(const void* q, const void* k, const void* v, void* out,
                                        float* lse, int32_t batch, int32_t n_q, int32_t n_kv,
                                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                        int64_t pretrained_window, int64_t local_window,
                                        double rope_base, float softmax_scale, void* stream);

/* Bytes of device workspace jl_bifocal_decode / jl_plain_decode need for this
 * shape (an upper bound over every L and W).  0 for invalid sizes. */
size_t jl_bifocal_decode_workspace_size(int32_t batch, int32_t n_kv, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim);

/* Bifocal decode: one new token per sequence against a cache that already holds
 * its own key/value at position n_kv-1 (ResearchPod transcript, cache exchange:
 * the cache keeps original positions; the correction is applied at lookup).
 *   q              : bf16 [B, 1, Hq, D], rotated at position n_kv-1
 *   k_cache/v_cache: bf16 [B, n_kv, Hkv, D], original positions, never modified
 *   out            : bf16 [B, 1, Hq, D];  lse: fp32 [B, Hq, 1] or NULL
 *   workspace      : device memory of at least jl_bifocal_decode_workspace_size bytes
 *                    (16-byte aligned; contents on entry are ignored)
 * g = jl_group_factor(n_kv, L).  The cache is split along its length into
 * chunks that are wholly remote (grouped scores) or wholly local (base
 * scores), reduced by a second kernel.  g == 1 runs jl_plain_decode. */
jl_status jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                            float* lse, int32_t batch, int32_t n_kv, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                            int64_t local_window, double rope_base, float softmax_scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* jl_bifocal_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The chunk partials go to a device array of
 * 32 MiB that the library holds on each GPU until the process ends (no
 * hipMalloc, hipFree or other allocating call is made).  Arguments, layouts,
 * results (bitwise those of jl_bifocal_decode on the same inputs) and errors as
 * jl_bifocal_decode, plus JL_ERR_UNSUPPORTED when the shape needs more than 32
 * MiB of workspace (jl_bifocal_decode_workspace_size: batch 8 with 32 query and
 * 8 KV heads at 128K positions fits, batch 16 does not).  Every call on a GPU uses that GPU's one array:
 * calls that overlap in time on one GPU (other streams, other host threads) race
 * and give undefined results; calls in stream order are safe. */
jl_status jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out,
                                    float* lse, int32_t batch, int32_t n_kv, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                    int64_t local_window, double rope_base, float softmax_scale,
                                    void* stream);

/* Plain decode with the same split-K kernels (no correction, no band). */
jl_status jl_plain_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                          float* lse, int32_t batch, int32_t n_kv, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Sliding-window decode: the new token at n_kv-1 attends to the newest
 * min(W, n_kv) cached keys (base RoPE), read by the split-K kernels; keys older
 * than the window are never read.  Layouts and workspace as jl_bifocal_decode
 * (jl_bifocal_decode_workspace_size bytes); local_window >= 1. */
jl_status jl_sliding_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                            float* lse, int32_t batch, int32_t n_kv, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int64_t local_window,
                            float softmax_scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bifocal decode of a batch of sequences of different lengths: one new token
 * per sequence, each against its own cache prefix, with g taken per sequence
 * (seventnews.com, "How bifocal attention sidesteps the fixed-scaling trap": the
 * long-range factor follows the current length; ResearchPod transcript, cache
 * exchange: the cache keeps original positions, so g can change as it grows).
 *   seq_lens       : device int32 [B], 4-byte aligned, not NULL; sequence b holds
 *                    s_b = seq_lens[b] keys, 1 <= s_b <= max_seq_len (device contents are not
 *                    checked on the host; a length outside the range gives an unspecified
 *                    result but no access outside the cache)
 *   q              : bf16 [B, 1, Hq, D]; row b rotated at position s_b - 1
 *   k_cache/v_cache: bf16 [B, max_seq_len, Hkv, D]; sequence b's keys are rows 0 .. s_b-1
 *                    at their original positions; rows past s_b are never read
 *   out, lse       : as jl_bifocal_decode
 *   workspace      : >= jl_bifocal_decode_workspace_size(B, max_seq_len, Hq, Hkv, D) bytes
 * Sequence b gets what jl_bifocal_decode returns for it alone with n_kv = s_b (a
 * sequence with g(s_b) == 1 is the plain decode), up to rounding order: the cache
 * is cut into chunks sized from B, max_seq_len and Hkv.  With every s_b equal to
 * max_seq_len the result is bitwise that of jl_bifocal_decode on the same batch. */
jl_status jl_bifocal_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* out,
                                   float* lse, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int64_t pretrained_window, int64_t local_window,
                                   double rope_base, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Plain decode of a batch of sequences of different lengths (same layouts and
 * kernels as jl_bifocal_decode_varlen, no correction). */
jl_status jl_plain_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* out,
                                 float* lse, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---- Long-range schedules -------------------------------------------------
 * The long-range branch rescales positions by a factor that follows the current
 * length, and the method is reported to be robust across rescaling schedules
 * (seventnews.com, "How bifocal attention sidesteps the fixed-scaling trap";
 * news.transform-ai.online, "How Jet-Long works": the far window's frequencies
 * are scaled from the current sequence length).  Three schedules, selected by
 * `schedule`; the local branch keeps original positions in all of them, and a
 * remote query at p and key at j are scored at positions a_q(p), a_k(j):
 *   JL_SCHED_GROUPED    (0) a_q(p) = floor(p/g), a_k(j) = floor(j/g), g = jl_group_factor:
 *                           what every other entry point computes.
 *   JL_SCHED_SEAM       (1) a_q(p) = floor(p/g) + W - floor(W/g), a_k(j) = floor(j/g): the
 *                           shift makes remote distances continue the local ones at the
 *                           seam (distance W or W+1 at p - j = W); g is the smallest
 *                           integer that keeps every shifted distance <= L-1.  Needs W < L.
 *   JL_SCHED_FRACTIONAL (2) a_q(p) = p/l, a_k(j) = j/l with the real l = max(1, (s-1)/(L-1)):
 *                           the remote branch is RoPE with theta/l.  Needs L >= 2 and
 *                           s < 2^30.
 * Every schedule is the base model when s <= L. */
#define JL_SCHED_GROUPED    0
#define JL_SCHED_SEAM       1
#define JL_SCHED_FRACTIONAL 2

/* The schedule's factor for a sequence of s keys: g for the two integer
 * schedules, l for the fractional one; 0.0 for invalid arguments (s < 1,
 * s > 2^31-1, L < 1, W < 1, W > L, or the schedule's own conditions above). */
double jl_schedule_factor(int64_t seq_len, int64_t pretrained_window, int64_t local_window,
                          int32_t schedule);

/* Bifocal prefill under a long-range schedule.  Arguments, layouts and errors as
 * jl_bifocal_prefill_ws, plus `schedule`; s = n_kv.  With a workspace (non-NULL,
 * >= jl_bifocal_prefill_workspace_size bytes) the corrected keys are written
 * there first and the attention kernel stages them (the two-launch form of
 * jl_bifocal_prefill_ws); with workspace == NULL and workspace_bytes == 0 the
 * keys are corrected tile by tile inside the attention kernel (the single-kernel
 * form of jl_bifocal_prefill).  JL_SCHED_GROUPED gives bitwise the result of
 * those two entry points. */
jl_status jl_bifocal_prefill_sched(const void* q, const void* k, const void* v, void* out,
                                   float* lse, int32_t batch, int32_t n_q, int32_t n_kv,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                   int64_t pretrained_window, int64_t local_window,
                                   double rope_base, int32_t schedule, float softmax_scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Bifocal decode under a long-range schedule.  seq_lens == NULL: every sequence
 * holds n_kv keys (arguments as jl_bifocal_decode); otherwise sequence b holds
 * seq_lens[b] keys of a cache of n_kv = max_seq_len positions (arguments as
 * jl_bifocal_decode_varlen), the factor, the seam shift and the rate taken per
 * sequence.  JL_SCHED_GROUPED gives bitwise the result of jl_bifocal_decode
 * (seq_lens NULL) or jl_bifocal_decode_varlen. */
jl_status jl_bifocal_decode_sched(const void* q, const void* k_cache, const void* v_cache,
                                  void* out, float* lse, const int32_t* seq_lens, int32_t batch,
                                  int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int64_t pretrained_window, int64_t local_window,
                                  double rope_base, int32_t schedule, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- Variable-length prefill batches ---------------------------------------
 * A batch of sequences, each with its own chunk of new queries against its own
 * cache: sequence b owns the packed query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * (n_b of them) at positions s_b - n_b + i, where s_b = seq_lens[b] keys sit in rows
 * 0 .. s_b-1 of its cache, the new tokens' own keys included.  The cache keeps
 * original positions and the factor follows each sequence's current length
 * (ResearchPod transcript, cache exchange; seventnews.com, "How bifocal attention
 * sidesteps the fixed-scaling trap"): g, the seam shift and the fractional rate
 * are taken per sequence from s_b.
 *   q, out        : bf16 [total_q, Hq, D], packed rows
 *   k/v_cache     : bf16 [B, max_seq_len, Hkv, D]; rows past s_b are never read
 *   lse           : fp32 [Hq, total_q] (natural log) or NULL
 *   cu_seqlens_q  : device int32 [B+1], 4-byte aligned, non-decreasing from 0 to total_q
 *   seq_lens      : device int32 [B], 4-byte aligned, n_b <= s_b <= max_seq_len
 *   max_q         : host int, >= every n_b (sizes the grid), <= max_seq_len
 *   workspace     : NULL with workspace_bytes == 0: the keys are corrected inside the
 *                   attention kernel (one launch, the form of jl_bifocal_prefill).
 *                   Otherwise >= jl_bifocal_prefill_workspace_size(B, max_seq_len, Hkv, D)
 *                   bytes for the corrected keys of every sequence, written by a first
 *                   pass (the two-launch form; contents ignored on entry)
 * The device arrays are not read on the host: values outside the contract give an
 * unspecified result but no access outside q, out, lse or the caches.  A sequence
 * with n_b = 0 writes nothing.  Each sequence gets what jl_bifocal_prefill_sched
 * (in the same form) returns for it alone, with n_q = n_b and n_kv = s_b.  With
 * every n_b and s_b equal it is bitwise that call on the padded batch (same
 * corrected keys, same sweep, same rounding; jl_plain_prefill_varlen is bitwise
 * jl_plain_prefill).  The bifocal kernel runs for every sequence, so one with
 * g = 1 is the base model up to rounding order.  Errors as
 * jl_bifocal_prefill_sched, plus JL_ERR_INVALID_ARG for NULL or misaligned length
 * arrays, total_q < 1 or max_q > max_seq_len. */
jl_status jl_bifocal_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                                    void* out, float* lse, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens, int32_t batch, int32_t total_q,
                                    int32_t max_q, int32_t max_seq_len, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                    int64_t local_window, double rope_base, int32_t schedule,
                                    float softmax_scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Plain causal prefill of a variable-length batch (same layouts, no correction,
 * no workspace). */
jl_status jl_plain_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                                  void* out, float* lse, const int32_t* cu_seqlens_q,
                                  const int32_t* seq_lens, int32_t batch, int32_t total_q,
                                  int32_t max_q, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                                  void* stream);

/* ---- Paged caches ------------------------------------------------------------
 * Decode over a paged cache: the keys and values of all sequences live in pools of
 * fixed-size pages, and a table maps each sequence's logical pages to pool pages.
 * The cache still keeps every key at its original position (ResearchPod
 * transcript, cache exchange), and g, the seam shift and the fractional rate follow
 * each sequence's own length (seventnews.com, "How bifocal attention sidesteps the
 * fixed-scaling trap").
 *   k_pages/v_pages: bf16 [n_pages, page_size, Hkv, D]; row r of page p holds one
 *                    position's keys (values) of every KV head
 *   block_table    : device int32 [B, pages_per_seq], 4-byte aligned: position j of
 *                    sequence b sits in row j % page_size of page
 *                    block_table[b * pages_per_seq + j / page_size]
 *   seq_lens       : device int32 [B]; sequence b holds positions 0 .. s_b-1, 1 <= s_b <=
 *                    pages_per_seq * page_size, its query at s_b - 1
 *   page_size      : a power of two in [32, 2^20]
 *   q, out, lse    : as jl_bifocal_decode_varlen
 *   workspace      : >= jl_bifocal_decode_workspace_size(B, pages_per_seq * page_size,
 *                    Hq, Hkv, D) bytes
 * Device contents are not read on the host: table entries are clamped into the pool
 * and lengths into range, so values outside the contract give an unspecified result,
 * never an access outside the pools.  Each sequence gets what jl_bifocal_decode_sched
 * returns for its contiguous cache, up to rounding order (chunks start at multiples
 * of the chunk size here, and the chunk holding both remote and local keys turns
 * its local keys by a zero angle).  Errors as jl_bifocal_decode_varlen, plus
 * JL_ERR_INVALID_ARG for a NULL or misaligned table or a page_size that is not a
 * power of two in range. */
jl_status jl_bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                  void* out, float* lse, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t batch, int32_t n_pages,
                                  int32_t page_size, int32_t pages_per_seq, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                  int64_t local_window, double rope_base, int32_t schedule,
                                  float softmax_scale, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Plain decode over a paged cache (same layouts, no correction). */
jl_status jl_plain_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* out,
                                float* lse, const int32_t* block_table, const int32_t* seq_lens,
                                int32_t batch, int32_t n_pages, int32_t page_size,
                                int32_t pages_per_seq, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, float softmax_scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---- Explicit query positions ----------------------------------------------
 * The query rows of a call need not be the newest tokens: row i sits at position
 * q_pos[i] of the n_kv-key context (ResearchPod transcript, cache exchange: the
 * cache keeps original positions, so any query can be scored against it), with g
 * from s = n_kv.  This serves, for instance, several candidate continuations or
 * rows recomputed in place.
 *   q_pos : device int32 [n_q], 4-byte aligned, nondecreasing, each in [0, n_kv),
 *           shared by every sequence of the batch; not read on the host: values
 *           outside the contract give an unspecified result, never an access out
 *           of range (positions are clamped into [0, n_kv))
 * Everything else as jl_bifocal_prefill_sched: with a workspace the corrected
 * keys are written there first (two launches), with workspace == NULL and
 * workspace_bytes == 0 they are corrected inside the attention kernel (one
 * launch, as jl_bifocal_prefill with q_pos).  Row i gets what the whole prefill
 * of n_kv queries gives at position q_pos[i], up to rounding order.  Errors as
 * those calls, plus JL_ERR_INVALID_ARG for a NULL or misaligned q_pos. */
jl_status jl_bifocal_prefill_positions(const void* q, const void* k, const void* v, void* out,
                                       float* lse, const int32_t* q_pos, int32_t batch, int32_t n_q,
                                       int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, int64_t pretrained_window,
                                       int64_t local_window, double rope_base, int32_t schedule,
                                       float softmax_scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

jl_status jl_plain_prefill_positions(const void* q, const void* k, const void* v, void* out,
                                     float* lse, const int32_t* q_pos, int32_t batch, int32_t n_q,
                                     int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, float softmax_scale, void* stream);

/* ---- A Qwen3-shaped attention layer ---------------------------------------
 * The method runs inside three Qwen3 sizes (1.7B, 4B, 8B) at up to 128K
 * tokens (seventnews.com, "Empirical results that challenge the status quo").
 * One attention layer of such a model, with the attention step bifocal or plain,
 * so that the attention's share of a layer can be measured:
 *   1. qkv = x w_qkv^T (rocBLAS, bf16, fp32 accumulation), no bias;
 *   2. per head: q = RMSNorm(q) * q_norm_weight, k = RMSNorm(k) * k_norm_weight
 *      (RMSNorm(y) = y / sqrt(mean(y^2) + rms_eps), in fp32), both rotated by RoPE
 *      at the tokens' positions p = n_kv - n_new + i; keys and values are written
 *      to rows p of the caches (the cache keeps original positions: ResearchPod
 *      transcript, cache exchange);
 *   3. attention of the n_new queries over the n_kv cached keys: JL_LAYER_BIFOCAL
 *      is jl_bifocal_prefill_sched in its single-kernel form (n_new > 1) or
 *      jl_bifocal_decode_sched (n_new == 1) under `schedule`; JL_LAYER_PLAIN is
 *      plain causal attention (jl_plain_prefill / jl_plain_decode); scale 1/sqrt(128);
 *   4. out = attn w_o^T (rocBLAS), no bias.
 *   x             : bf16 [B, n_new, hidden]
 *   w_qkv         : bf16 [(Hq + 2 Hkv) * 128, hidden]: the query heads' rows, then the
 *                   key heads', then the value heads' (PyTorch Linear layout)
 *   q/k_norm_weight: bf16 [128]
 *   w_o           : bf16 [hidden, Hq * 128]
 *   out           : bf16 [B, n_new, hidden]
 *   k/v_cache     : bf16 [B, n_kv, Hkv, 128]; rows 0 .. n_kv-n_new-1 hold the earlier
 *                   tokens (keys rotated at their positions) and are only read; rows
 *                   n_kv-n_new .. n_kv-1 are written
 *   workspace     : >= jl_qwen3_layer_workspace_size(...) bytes of device memory,
 *                   16-byte aligned, contents ignored on entry
 * All pointers are device pointers, 16-byte aligned, owned by the caller; the
 * layer runs in stream order on `stream`.  Device memory: the library allocates
 * none.  Projections of more than 8 rows run on rocBLAS through one handle per
 * calling thread and device (created on first use, destroyed when the thread
 * exits), whose GEMM scratch is a 32 MiB part of `workspace`; creating a handle
 * is rocBLAS's own work and may allocate inside rocBLAS.  Windows and
 * schedule are checked as in jl_bifocal_prefill_sched when attention ==
 * JL_LAYER_BIFOCAL and ignored otherwise (rope_base is always checked).
 * Errors: JL_ERR_INVALID_ARG for bad pointers, sizes (n_new > n_kv, hidden < 1),
 * rms_eps < 0 or an unknown attention kind; JL_ERR_UNSUPPORTED for head_dim != 128
 * or sizes beyond 32-bit GEMM dimensions; JL_ERR_WORKSPACE; JL_ERR_DEVICE for
 * launch or rocBLAS errors. */
#define JL_LAYER_PLAIN   0
#define JL_LAYER_BIFOCAL 1

size_t jl_qwen3_layer_workspace_size(int32_t batch, int32_t n_new, int32_t n_kv, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim);

jl_status jl_qwen3_attention_layer(const void* x, const void* w_qkv, const void* q_norm_weight,
                                   const void* k_norm_weight, const void* w_o, void* out,
                                   void* k_cache, void* v_cache, int32_t batch, int32_t n_new,
                                   int32_t n_kv, int32_t hidden, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, float rms_eps,
                                   int32_t attention, int64_t pretrained_window,
                                   int64_t local_window, double rope_base, int32_t schedule,
                                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JL_BIFOCAL_H */
