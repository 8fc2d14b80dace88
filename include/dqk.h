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
 * memory); the five buffers are device memory.  Per physical page p and KV
 * head g (all little-endian):
 *   k_codes u8   [num_pages][Hkv][128 ch][32]   channel j's 2-bit codes of the
 *                                              page's 128 tokens; token t at
 *                                              byte t>>2, bits 2*(t&3).
 *                                              Row 0 is unused (zero).
 *   k_meta  f16  [num_pages][Hkv][128 ch][2]    (scale, zero) of channel j over
 *                                              the page's valid tokens; entry 0
 *                                              unused (zero).
 *   k_ch0   bf16 [num_pages][Hkv][128 tok]      channel 0 of k', kept in bf16.
 *   v_codes u8   [num_pages][Hkv][128 tok][32]  token t's codes; channel c at
 *                                              byte c>>2, bits 2*(c&3).
 *   v_meta  f16  [num_pages][Hkv][2][4][128]    [0][q][t] scale, [1][q][t] zero
 *                                              of token t, channels 32q..32q+31.
 * Dequantized value = fma(code, scale, zero) in fp32.  Grid of a group with
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
 * pages ("each new key is transformed ... and stored", §3.4; layout §3.3).
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
 */
int dqk_decode_attn(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep, int32_t batch,
                    int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                    float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out, float *lse,
                    hipStream_t stream);

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
