/*
 * dqk.h -- C ABI of libdqk: decode attention over a 2-bit (INT2) KV cache
 * with dynamic query-channel pruning, and its quantize-append step, for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow "Dual-QK: Sharp Queries and Flat Keys for Prunable
 * 2-bit KV Caches" (Whang, Oh, Kim, Seo):
 *   - a fixed transform pair per KV head, q' = q T_Q and k' = k T_K with
 *     T_Q = T_K^{-T}, so q'.k' = q.k before compression (§3.1, Eq. 1);
 *   - per decode step, a channel mask shared by the query heads of a KV head,
 *     chosen from the pooled query energy e_j (§3.2, Eq. 4); scores use only
 *     the kept channels and keep the 1/sqrt(d) normalisation;
 *   - keys stored channel-major in 128-token pages, one channel per 32-byte
 *     row, channel 0 in bf16 outside the INT2 range; values token-major with
 *     separate metadata buffers (§3.3);
 *   - one softmax over the whole context (§3.4).
 *
 * Conventions
 *   Row vectors; T[i][j] with i the input and j the output channel.
 *   head_dim d = DQK_HEAD_DIM = 128, page = DQK_PAGE = 128 tokens.
 *   Query head h uses KV head h / (Hq / Hkv).
 *   Every pointer argument is a DEVICE pointer unless marked "host".  Scalar
 *   arguments are host values.  All device buffers are caller-allocated and
 *   16-byte aligned.  The library never allocates, frees or synchronizes:
 *   work is enqueued on `stream` and the call returns.  Calls are stateless
 *   and may run concurrently on different streams over disjoint outputs.
 *
 * Errors
 *   Every entry point validates its arguments on the host before enqueueing
 *   anything; on error nothing is enqueued.  Contents of device arrays
 *   (lengths, page tables, prefix sums) are preconditions and are not read
 *   by the host; violating them is undefined behaviour.  Kernel faults
 *   surface at the caller's next synchronization.
 */
#ifndef DQK_H
#define DQK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DQK_HEAD_DIM 128
#define DQK_PAGE 128

enum {
    DQK_OK = 0,
    DQK_ERR_NULL = -1,        /* a required pointer is null                         */
    DQK_ERR_SHAPE = -2,       /* Hq % Hkv != 0, n_keep out of range, bad sizes       */
    DQK_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned             */
    DQK_ERR_UNSUPPORTED = -4, /* request outside what the kernels implement          */
    DQK_ERR_WORKSPACE = -5,   /* workspace too small                                 */
    DQK_ERR_HIP = -6          /* a HIP launch failed; see dqk_last_hip_error()       */
};

/*
 * The paged INT2 cache (§3.3).  Plain struct filled by the caller (host
 * memory); the five buffers are device memory.  num_pages is a multiple of 8:
 * the pool is made of aligned blocks of eight pages, and the key rows and key
 * metadata of a channel sit side by side for the block's eight pages (page p
 * is slot p & 7 of block p >> 3), so a selected channel of a whole block is
 * one contiguous 256-byte run.  All little-endian:
 *   k_codes u8   [num_pages/8][Hkv][128 ch][8 slot][32]
 *                                   channel j's 2-bit codes of one page's 128
 *                                   tokens; token t at byte t>>2, bits 2*(t&3).
 *                                   Rows of channel 0 are unused (zero).
 *   k_meta  f16  [num_pages/8][Hkv][128 ch][8 slot][2]
 *                                   (scale, zero) of channel j over the page's
 *                                   valid tokens; channel 0 entries unused (zero).
 * and per physical page p, KV head g:
 *   k_ch0   bf16 [num_pages][Hkv][128 tok]      channel 0 of k', kept in bf16.
 *   v_codes u8   [num_pages][Hkv][128 tok][32]  token t's codes; channel c at
 *                                              byte c>>2, bits 2*(c&3).
 *   v_meta  f16  [num_pages][Hkv][2][4][128]    [0][q][t] scale, [1][q][t] zero
 *                                              of token t, channels 32q..32q+31.
 * The value a code stands for is fma(code, scale, zero) in fp32 (the
 * definition the decode approximates; its arithmetic is stated at
 * dqk_decode_attn).  Grid of a group with
 * minimum mn and maximum mx: zero = mn rounded down to binary16, scale =
 * fp32((mx - zero) / 3) rounded up to binary16; code = number of thresholds
 * fma(c + 0.5, scale, zero), c = 0, 1, 2, that the value reaches.
 */
typedef struct dqk_cache {
    int32_t num_kv_heads;
    int32_t num_pages;
    uint8_t *k_codes;
    uint16_t *k_meta;
    uint16_t *k_ch0;
    uint8_t *v_codes;
    uint16_t *v_meta;
} dqk_cache;

/*
 * Quantize-append: transform keys with T_K and pack keys and values into
 * pages (§3.4: a key enters the cache only after the key transform; layout
 * §3.3).
 *   c           host pointer to the cache description.
 *   k_bf16      bf16 [total_tokens][Hkv][128] raw keys (post-RoPE).
 *   v_bf16      bf16 [total_tokens][Hkv][128] raw values.
 *   t_k_bf16    bf16 [Hkv][128][128] key transform T_K.
 *   n_seqs      number of sequences (>= 1).
 *   cu_tokens   int32 [n_seqs + 1] prefix sums of sequence lengths; sequence i
 *               owns tokens cu_tokens[i] .. cu_tokens[i+1]-1 (at most
 *               max_pages*128 of them) and is written from logical position 0.
 *   page_table  int32 [n_seqs][max_pages]: logical page -> physical page.
 *   kprime_dbg  fp32 [total_tokens][Hkv][128] or NULL: receives k' = k T_K
 *               (the fp32 MFMA accumulator that is quantized).
 * k' = k T_K runs on MFMA (bf16 x bf16 -> fp32).  Key groups are (page, KV
 * head, channel 1..127) over the page's valid tokens; value groups are
 * (token, KV head, 32 consecutive channels).  Slots past a sequence's end are
 * written as code 0, ch0 0 and metadata 0.  Pages are written whole: appending
 * into a partly filled page is not supported.
 */
int dqk_quantize_append(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                        int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens, const int32_t *page_table,
                        int32_t max_pages, float *kprime_dbg, hipStream_t stream);

/*
 * Query transform and dynamic channel selection (§3.2, Eq. 4).
 *   q_bf16   bf16 [batch][hq][128] current queries (post-RoPE).
 *   t_q      fp32 [hkv][128][128] query transform T_Q.
 *   q_prime  fp32 [batch][hq][128] out: q' = q T_Q, each element an fp32 fma
 *            chain over ascending input channel.
 *   sel_idx  int32 [batch][hkv][n_keep] out: the n_keep channels with the
 *            largest pooled energy S_j = sum over the KV head's query heads of
 *            q'_j^2 (fp32 fma chain, ascending head), ties to the lower
 *            channel, listed in ascending channel order.  (e_j = sqrt(S_j) is
 *            monotone in S_j.)
 * Requires 1 <= n_keep <= 128, hq % hkv == 0.
 */
int dqk_select_channels(const void *q_bf16, const float *t_q, int32_t batch, int32_t hq, int32_t hkv,
                        int32_t n_keep, float *q_prime, int32_t *sel_idx, hipStream_t stream);

/* Bytes of workspace dqk_decode_attn / dqk_decode_attn_bf16 need for the
 * split partials (num_splits = 0 means the automatic choice). */
size_t dqk_decode_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t max_pages, int32_t num_splits);

/*
 * Decode attention over the paged INT2 cache (§3.2-§3.4).  For each query
 * head h of sequence b: logit_t = sm_scale * sum_{j in M} q'_{h,j} k^_{t,j}
 * over the KV head's selected set M (channel 0 read from k_ch0, others
 * dequantized), one softmax over tokens t < seq_lens[b], and
 * out_{h,:} = sum_t p_t v^_t.  Split-K over pages with a log-sum-exp merge.
 *   q_prime     fp32 [batch][hq][128] from dqk_select_channels.
 *   sel_idx     int32 [batch][hkv][n_keep] from dqk_select_channels.
 *   page_table  int32 [batch][max_pages].
 *   seq_lens    int32 [batch], each in [1, max_pages*128].
 *   sm_scale    normally 1/sqrt(128) whatever n_keep is (§3.2).
 *   num_splits  0 = automatic, else 1..max_pages.
 *   workspace   device scratch of at least dqk_decode_workspace_size() bytes.
 *   out         fp32 [batch][hq][128].
 *   lse         fp32 [batch][hq] or NULL: log-sum-exp of the logits.
 * Requires hq / hkv <= 16 (DQK_ERR_UNSUPPORTED).  Every group size runs the
 * same MFMA decode: the query heads of a KV head are taken in sets of four
 * (ceil(g / 4) workgroups per KV head and split, each reading the KV head's
 * pages; a set of fewer than four is padded with zero queries).
 * Arithmetic of the MFMA decode:
 *   - logits: fp32 sums; the query-side operand C q'_j s_j (C = sm_scale
 *     log2 e, s_j the key scale) enters as two binary16 limbs (>= 21
 *     significant bits) scaled per page by a power of two that brings the
 *     page's largest |C q' s| near 2^14; codes enter exactly; the zero-point
 *     term sum_j C q'_j z_j is an fp32 sum.  Requires |C q'_j s_j| and the
 *     logits finite in fp32.
 *   - probabilities P = 2^(x - m + 14), m the split's integer running
 *     maximum (log2 units), are rounded to binary16: relative error <= 2^-11;
 *     weights below 2^-28 of the split's largest are binary16 subnormals
 *     (absolute error 2^-39 of it) and below 2^-38 of it they are 0.
 *   - values: P s' is rounded to binary16 (<= 2^-11 relative), s' = s 2^-E
 *     with E in [-15, 15] the split's running exponent of the value scales;
 *     the zero points enter as sum_t P_t z_t (binary16 z, fp32 sums).  Value
 *     scales and zero points are binary16 by format (|value| <= 65504).
 *   Results therefore depend on the split count through these roundings
 *   (each split rounds relative to its own maxima), within about
 *   2^-10 sum_t p_t (|z_t + 1.5 s_t| + 2 |s_t (c_t - 1.5)|) per element.
 */
int dqk_decode_attn(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep, int32_t batch,
                    int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                    float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out, float *lse,
                    hipStream_t stream);

/*
 * dqk_select_channels followed by dqk_decode_attn, as one call: for the
 * group-4 MFMA decode (Hq = 4 Hkv, 17 <= n_keep <= 128) the selection runs in
 * the decode kernel's prologue, one launch instead of two; otherwise the two
 * calls are made in sequence.  Results are identical to the two calls
 * (q_prime and sel_idx bit for bit, then the same decode).
 *   q_bf16, t_q          as dqk_select_channels.
 *   q_prime, sel_idx     outputs as dqk_select_channels (required).
 * Other arguments, workspace size and errors as dqk_decode_attn.
 */
int dqk_select_decode_attn(const dqk_cache *c, const void *q_bf16, const float *t_q, int32_t n_keep, int32_t batch,
                           int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                           float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                           float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream);

/*
 * dqk_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Allocates nothing (no hipMalloc, no
 * allocating library call): the split partials live in a 16 MiB device array
 * inside the library, one per GPU, held until the process ends.  Its address
 * is looked up on the calling thread's current device (hipGetDevice), which
 * must be the device of the stream and of every buffer.
 *   Limit: batch * hq * splits * 528 bytes <= dqk_decode_noalloc_max_bytes()
 *   (16 MiB), splits as dqk_decode_attn resolves num_splits; larger requests
 *   return DQK_ERR_WORKSPACE before anything is enqueued.
 *   Calls that overlap on one GPU (different streams, or different host
 *   threads) share that array and race; serialize them.  Every call rewrites
 *   all the partials it reads, so nothing has to be cleared between calls.
 * Arguments, results and other errors as dqk_decode_attn.
 */
int dqk_decode_attn_noalloc(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                            int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, float sm_scale, int32_t num_splits, float *out, float *lse,
                            hipStream_t stream);

/* Size of the partials array dqk_decode_attn_noalloc uses (bytes). */
size_t dqk_decode_noalloc_max_bytes(void);

/*
 * Unpruned BF16 decode attention, the baseline the paper's throughput is
 * measured against (§4.4): softmax(q k^T * sm_scale) v in original
 * coordinates, no transform.
 *   k_pages, v_pages  bf16 [num_pages][hkv][128 tok][128 ch].
 *   q_bf16            bf16 [batch][hq][128].
 * Other arguments as dqk_decode_attn.
 */
int dqk_decode_attn_bf16(const void *k_pages, const void *v_pages, int32_t hkv, int32_t num_pages,
                         const void *q_bf16, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                         const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                         size_t ws_bytes, float *out, float *lse, hipStream_t stream);

/*
 * Protected BF16 tiers (§3.3: the first 64 and the most recent 256 tokens of
 * a sequence stay in BF16 for keys and values and use the same channel mask;
 * §3.4: one softmax over every token).  In the tiered layout a sequence of
 * length L keeps
 *   tokens [0, min(L, 64))        in the sink, slot t;
 *   tokens [64, 64 + 128 P)       in P INT2 pages, P = floor((L - 320) / 128)
 *                                 for L >= 320, else 0: logical INT2 page i
 *                                 (page_table[b][i]) holds tokens
 *                                 64 + 128 i .. 64 + 128 i + 127, all older
 *                                 than the 256 most recent tokens;
 *   tokens [64 + 128 P, L)        in the tail (256..383 tokens once L >= 320),
 *                                 slot (t - 64) mod 384.
 * Tier keys are k' = k T_K (fp32) rounded to bf16 (nearest even); tier values
 * are the bf16 inputs; the tail also keeps the raw bf16 keys, from which its
 * oldest page is packed when the sequence grows past it.
 */
#define DQK_TIER_SINK 64
#define DQK_TIER_RECENT 256
#define DQK_TIER_TAIL_SLOTS 384

typedef struct dqk_tiers {
    int32_t batch;        /* sequences                                   */
    int32_t num_kv_heads; /* must equal the cache's                      */
    uint16_t *sink_k;     /* bf16 [batch][Hkv][64][128]  k' of the sink   */
    uint16_t *sink_v;     /* bf16 [batch][Hkv][64][128]                   */
    uint16_t *tail_k;     /* bf16 [batch][Hkv][384][128] k' of the tail   */
    uint16_t *tail_v;     /* bf16 [batch][Hkv][384][128]                  */
    uint16_t *tail_kraw;  /* bf16 [batch][Hkv][384][128] raw k of the tail */
} dqk_tiers;

/*
 * Prefill into the tiered layout: sequence b (tokens cu_tokens[b] ..
 * cu_tokens[b+1]-1 of k_bf16 / v_bf16, as dqk_quantize_append) fills its
 * sink and tail slots and its INT2 pages page_table[b][0 .. P-1].
 * Requires n_seqs <= tiers->batch; other arguments and errors as
 * dqk_quantize_append.
 */
int dqk_prefill_tiered(const dqk_cache *c, const dqk_tiers *tiers, const void *k_bf16, const void *v_bf16,
                       const void *t_k_bf16, int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens,
                       const int32_t *page_table, int32_t max_pages, hipStream_t stream);

/*
 * Per-token append (a decode step): sequence b gains one token at position
 * lens_before[b] (device int32 [batch], its length before the call), keys
 * k_bf16 and values v_bf16 bf16 [batch][Hkv][128].  The token goes to its
 * sink or tail slot; if the new length lets a page leave the recent window,
 * that page is packed from the tail into page_table[b][P] (P = INT2 pages
 * before the call) exactly as the prefill would pack it.  The caller then
 * counts the token in its lengths.  Two kernels, stream-ordered.
 */
int dqk_append_token(const dqk_cache *c, const dqk_tiers *tiers, const void *k_bf16, const void *v_bf16,
                     const void *t_k_bf16, int32_t batch, const int32_t *lens_before, const int32_t *page_table,
                     int32_t max_pages, hipStream_t stream);

/* Bytes of workspace dqk_decode_attn_tiered needs. */
size_t dqk_decode_tiered_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t max_pages,
                                        int32_t num_splits);

/*
 * Decode attention over the tiered layout: the INT2 pages of each sequence
 * (as dqk_decode_attn, over its P pages) and its BF16 sink and tail tokens
 * (logit = sm_scale * sum_{j in M} q'_j k'_j with the bf16 k', value the
 * bf16 v) under one softmax, merged by log-sum-exp.  seq_lens[b] is the
 * sequence's full length L (>= 1).  Other arguments, the workspace (of
 * dqk_decode_tiered_workspace_size bytes) and errors as dqk_decode_attn.
 */
int dqk_decode_attn_tiered(const dqk_cache *c, const dqk_tiers *tiers, const float *q_prime, const int32_t *sel_idx,
                           int32_t n_keep, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                           size_t ws_bytes, float *out, float *lse, hipStream_t stream);

/*
 * dqk_select_channels + dqk_decode_attn_tiered as one call (the selection of
 * §3.2, then the tiered decode of §3.3-§3.4): q_prime and sel_idx receive the
 * selection as dqk_select_channels writes it, and the results are those of
 * the two calls (the entry makes them).  Arguments, workspace (of
 * dqk_decode_tiered_workspace_size bytes) and errors as dqk_select_decode_attn
 * and dqk_decode_attn_tiered; every check runs before the first launch.
 */
int dqk_select_decode_attn_tiered(const dqk_cache *c, const dqk_tiers *tiers, const void *q_bf16, const float *t_q,
                                  int32_t n_keep, int32_t batch, int32_t hq, const int32_t *page_table,
                                  int32_t max_pages, const int32_t *seq_lens, float sm_scale, int32_t num_splits,
                                  void *workspace, size_t ws_bytes, float *out, float *lse, float *q_prime,
                                  int32_t *sel_idx, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Rotated values and selection in base coordinates (§3.3: the calibrated
 * value rotation and clipping of App. B.2, and the diagonal refinement
 * A = A_0 D with selection on the base queries q A_0, App. C.2; §3.4: the
 * value rotation is undone after aggregation).  A cache written by
 * dqk_quantize_append_vrot holds v' = v R_V in its value pages; any decode
 * entry point aggregates v' unchanged and dqk_value_unrotate then maps each
 * output row back, o = o' R_V^-1.
 */

/*
 * dqk_quantize_append with rotated, clipped values.  Keys exactly as
 * dqk_quantize_append (not clipped).  Values: v' = v R_V on MFMA (bf16 x bf16
 * -> fp32 accumulator, no intermediate rounding), then per (token, KV head,
 * 32-channel group) the binary16 grid of the clipped range
 * [fp32(clip * min), fp32(clip * max)] of the group's v' (values beyond it
 * take code 0 or 3).
 *   r_v_bf16    bf16 [Hkv][128][128] value rotation R_V, [in ch][out ch].
 *   clip        clipping ratio, 0 < clip <= 1 (the paper uses 0.92; 1 fits
 *               the full range).
 *   vprime_dbg  fp32 [total_tokens][Hkv][128] or NULL: receives v' = v R_V.
 * Other arguments and errors as dqk_quantize_append; DQK_ERR_SHAPE for a clip
 * outside (0, 1].
 */
int dqk_quantize_append_vrot(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                             const void *r_v_bf16, float clip, int32_t n_seqs, const int32_t *cu_tokens,
                             int64_t total_tokens, const int32_t *page_table, int32_t max_pages, float *kprime_dbg,
                             float *vprime_dbg, hipStream_t stream);

/*
 * dqk_select_channels with the channels ranked in base coordinates: with the
 * refinement D folded into T_Q (q' = q A_0 D), the energy of channel j is
 * S_j = sum over the KV head's query heads of e^2, e = fp32(q'_j *
 * sel_scale[g][j]) (fp32 fma chain, ascending head), sel_scale = 1 / delta_j.
 * q_prime is q T_Q as in dqk_select_channels (the scoring coordinates).
 *   sel_scale  fp32 [hkv][128], finite.
 * Other arguments and errors as dqk_select_channels.
 */
int dqk_select_channels_base(const void *q_bf16, const float *t_q, const float *sel_scale, int32_t batch,
                             int32_t hq, int32_t hkv, int32_t n_keep, float *q_prime, int32_t *sel_idx,
                             hipStream_t stream);

/*
 * Inverse value rotation of decode outputs: for each sequence b and query
 * head h (KV head g = h / (hq / hkv)), out[b][h][c] = sum_j o_rot[b][h][j]
 * r_v_inv[g][j][c], an fp32 fma chain over ascending j.
 *   o_rot     fp32 [batch][hq][128], the output of a decode entry point.
 *   r_v_inv   fp32 [hkv][128][128] inverse of the stored R_V, [j][c].
 *   out       fp32 [batch][hq][128]; must not overlap o_rot
 *             (DQK_ERR_UNSUPPORTED if it does).
 * Requires hq % hkv == 0 (DQK_ERR_SHAPE) and hq / hkv <= 64
 * (DQK_ERR_UNSUPPORTED).  One kernel, stream-ordered after the decode.
 */
int dqk_value_unrotate(const float *o_rot, const float *r_v_inv, int32_t batch, int32_t hq, int32_t hkv,
                       float *out, hipStream_t stream);

/*
 * The rotated-value decode step as one call: selection in base coordinates
 * (as dqk_select_channels_base), decode (as dqk_decode_attn) and the split
 * merge followed by the inverse value rotation (as dqk_value_unrotate) in the
 * merge kernel.  For hq = 4 hkv and 17 <= n_keep <= 128 the selection runs in
 * the decode launch (two launches in all); otherwise the selection is a
 * launch of its own.  q_prime, sel_idx, out and lse are bit-identical to
 * those of dqk_select_channels_base + dqk_decode_attn + dqk_value_unrotate
 * (lse being that of the rotated output, which the rotation leaves as is).
 * Arguments as dqk_select_decode_attn, plus sel_scale (fp32 [hkv][128]) and
 * r_v_inv (fp32 [hkv][128][128]); errors as those calls.
 */
int dqk_select_decode_attn_vrot(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *sel_scale,
                                const float *r_v_inv, int32_t n_keep, int32_t batch, int32_t hq,
                                const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                                float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                                float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token key grids (§3.3 as the paper states it: one asymmetric INT2 grid
 * per token and KV head over channels 1..127, channel 0 kept in bf16 and left
 * out of the range).  The cache buffers are those of dqk_cache; only k_meta
 * is read differently: the (scale, zero) pairs of a block's eight pages are
 * token-major, [P/8][Hkv][8 slot][128 tok][2] fp16 (the same 4 KB per block
 * and KV head).  A cache is written and read in one of the two layouts only.
 */

/*
 * dqk_quantize_append with one key grid per (token, KV head): the grid of
 * token t is fitted to k'_{t,1..127} (z = round-down of the minimum, s =
 * round-up of (max - z)/3, both binary16), the codes are those of that grid.
 * Channel 0 and the values as dqk_quantize_append.  Arguments, slots past a
 * sequence's end and errors as dqk_quantize_append.
 */
int dqk_quantize_append_tokgrid(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                                int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens,
                                const int32_t *page_table, int32_t max_pages, float *kprime_dbg, hipStream_t stream);

/*
 * dqk_decode_attn over a cache written by dqk_quantize_append_tokgrid:
 * k^_{t,j} = code * s_t + z_t for j >= 1.  On MFMA the dot product of the
 * codes with q~ = C q' (two binary16 limbs, scaled once per split) is scaled
 * per token by s_t, and z_t multiplies the fp32 sum of C q'_j over the
 * selected channels; the rest as dqk_decode_attn.  Requires |C q'_j| s_t
 * finite in fp32.  Arguments, workspace and errors as dqk_decode_attn.
 */
int dqk_decode_attn_tokgrid(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                            int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                            size_t ws_bytes, float *out, float *lse, hipStream_t stream);

/*
 * dqk_select_decode_attn over a cache with per-token key grids: selection (in
 * the decode launch for hq = 4 hkv and 17 <= n_keep <= 128), decode as
 * dqk_decode_attn_tokgrid, merge.  Arguments and errors as
 * dqk_select_decode_attn; results identical to dqk_select_channels +
 * dqk_decode_attn_tokgrid.
 */
int dqk_select_decode_attn_tokgrid(const dqk_cache *c, const void *q_bf16, const float *t_q, int32_t n_keep,
                                   int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                                   const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                                   size_t ws_bytes, float *out, float *lse, float *q_prime, int32_t *sel_idx,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Bucket-relative RoPE (§3.4 and App. C.4).  Positions of a sequence fall in
 * buckets of 2048 (bucket k: positions 2048 k .. 2048 k + 2047, counted from
 * the sequence's start, i.e. logical pages 16 k .. 16 k + 15), with anchor
 * a_k = 2048 k.  A stored key is moved from its position n to n - a_k before
 * the key transform; for each bucket the current query is moved by the same
 * anchor before the query transform, gets its own channel mask, and scores
 * that bucket's tokens; one softmax spans every bucket.
 *   rope_cos, rope_sin  fp32 [n_buckets][64] device: cos(a_k theta_i) and
 *               -sin(a_k theta_i) for the rotate-half channel pairs (i, i + 64)
 *               (the checkpoint's rotary frequencies theta_i, any scaling
 *               included).  Vector x turned by table k: y_i = x_i c - x_{i+64} s,
 *               y_{i+64} = x_{i+64} c + x_i s, every product and sum in fp32.
 *   n_buckets   >= 1, with 16 n_buckets >= max_pages (every page of a
 *               sequence lies in a bucket that has a table).
 * The cache layout is that of dqk_quantize_append (per-channel key grids).
 */

/*
 * dqk_quantize_append with keys in their bucket frames: the key of token t
 * (position p = t - cu_tokens[i] in its sequence) is turned by table p / 2048,
 * rounded to bf16 (to nearest even), then multiplied by T_K.  kprime_dbg
 * receives that k'.  Other arguments, slots past a sequence's end and errors
 * as dqk_quantize_append; DQK_ERR_SHAPE also if n_buckets < 1 or
 * 16 n_buckets < max_pages.
 */
int dqk_quantize_append_rope(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                             const float *rope_cos, const float *rope_sin, int32_t n_buckets, int32_t n_seqs,
                             const int32_t *cu_tokens, int64_t total_tokens, const int32_t *page_table,
                             int32_t max_pages, float *kprime_dbg, hipStream_t stream);

/*
 * Per-bucket selection: for sequence b and bucket k, q turned by table k (fp32)
 * then q' = q T_Q and the mask of dqk_select_channels.
 *   q_prime     fp32 [batch][n_buckets][Hq][128] device (output).
 *   sel_idx     int32 [batch][n_buckets][Hkv][n_keep] device (output).
 * Other arguments and errors as dqk_select_channels; DQK_ERR_UNSUPPORTED if
 * batch * n_buckets > 65535.
 */
int dqk_select_channels_rope(const void *q_bf16, const float *t_q, const float *rope_cos, const float *rope_sin,
                             int32_t n_buckets, int32_t batch, int32_t hq, int32_t hkv, int32_t n_keep,
                             float *q_prime, int32_t *sel_idx, hipStream_t stream);

/*
 * Workspace bytes for dqk_decode_attn_rope / dqk_select_decode_attn_rope
 * (num_splits: splits per bucket, 0 = automatic); 0 on invalid sizes.
 */
size_t dqk_decode_rope_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t n_buckets,
                                      int32_t num_splits);

/*
 * Decode over a cache written by dqk_quantize_append_rope: token t of sequence
 * b scores with q_prime[b][t / 2048] masked by sel_idx[b][t / 2048] (the
 * output layout of dqk_select_channels_rope), and the scores of all buckets
 * share one softmax.  A split covers whole buckets and keeps their queries
 * and channel lists in LDS, switching at each bucket's first page;
 * num_splits (0 = automatic) is raised where a split would hold more buckets
 * than fit (8, or 4 to 5 for n_keep in 81..96 and above 112).  Other
 * arguments, outputs and errors as dqk_decode_attn; DQK_ERR_SHAPE also if
 * n_buckets < 1 or 16 n_buckets < max_pages; DQK_ERR_UNSUPPORTED also if
 * batch * n_buckets > 65535.
 */
int dqk_decode_attn_rope(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                         int32_t n_buckets, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                         const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                         size_t ws_bytes, float *out, float *lse, hipStream_t stream);

/*
 * dqk_select_channels_rope + dqk_decode_attn_rope in one call; q_prime and
 * sel_idx receive the selection as dqk_select_channels_rope writes it.
 * Results identical to the two calls.
 */
int dqk_select_decode_attn_rope(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *rope_cos,
                                const float *rope_sin, int32_t n_keep, int32_t n_buckets, int32_t batch, int32_t hq,
                                const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                                float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                                float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream);

/*
 * dqk_stream_read -- measurement helper, not part of the attention path: a
 * plain streaming read of `bytes` bytes (a multiple of 16 KiB) at `src`,
 * 16 bytes per lane through LDS, as the reference point for the decode
 * kernel's achieved HBM bandwidth.  `sink` (device, 4 bytes per 64-lane
 * workgroup: bytes / 16 KiB rounded to the grid the call picks, at most
 * 4096 * 4 bytes) receives a checksum so the reads cannot be elided.
 * Returns DQK_ERR_SHAPE if bytes is 0 or not a multiple of 16 KiB.
 */
int dqk_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Static text for a DQK_* status code. */
const char *dqk_status_string(int status);

/* The hipError_t of the last failed launch on the calling thread (0 if none). */
int dqk_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DQK_H */
