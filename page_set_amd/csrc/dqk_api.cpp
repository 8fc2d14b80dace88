// libdqk C ABI: argument validation (host only, before anything is enqueued)
// and dispatch to the kernels.  See include/dqk.h for the contract.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "dqk_internal.h"

namespace {

thread_local int g_last_hip = 0;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return DQK_OK;
    g_last_hip = (int)e;
    return DQK_ERR_HIP;
}

int check_cache(const dqk_cache *c) {
    if (!c || !c->k_codes || !c->k_meta || !c->k_ch0 || !c->v_codes || !c->v_meta) return DQK_ERR_NULL;
    if (c->num_kv_heads < 1 || c->num_pages < 1) return DQK_ERR_SHAPE;
    if (c->num_kv_heads > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(c->k_codes) || !aligned16(c->k_meta) || !aligned16(c->k_ch0) || !aligned16(c->v_codes) ||
        !aligned16(c->v_meta))
        return DQK_ERR_ALIGN;
    return DQK_OK;
}

// n_keep = 0: the largest count any n_keep can resolve to (workspace sizing)
int resolve_splits(int batch, int hq, int hkv, int max_pages, int num_splits, int n_keep) {
    if (num_splits > 0) return num_splits;
    if (dqk::use_mfma_decode(hq, hkv)) return dqk::decode_splits_mfma(batch, hkv, max_pages, n_keep);
    return dqk::decode_splits_generic(batch, hkv, max_pages);
}

}  // namespace

extern "C" {

const char *dqk_status_string(int status) {
    switch (status) {
        case DQK_OK: return "ok";
        case DQK_ERR_NULL: return "a required pointer is null";
        case DQK_ERR_SHAPE: return "invalid shape (Hq % Hkv != 0, n_keep outside 1..128, or a non-positive size)";
        case DQK_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case DQK_ERR_UNSUPPORTED: return "request outside what the kernels implement";
        case DQK_ERR_WORKSPACE: return "workspace too small";
        case DQK_ERR_HIP: return "HIP launch failed (see dqk_last_hip_error)";
        default: return "unknown status";
    }
}

int dqk_last_hip_error(void) { return g_last_hip; }

int dqk_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (!src || !sink) return DQK_ERR_NULL;
    if (bytes == 0 || bytes % 16384 != 0) return DQK_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(sink)) return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_stream_read(src, bytes, sink, stream));
}

int dqk_select_channels(const void *q_bf16, const float *t_q, int32_t batch, int32_t hq, int32_t hkv,
                        int32_t n_keep, float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    if (!q_bf16 || !t_q || !q_prime || !sel_idx) return DQK_ERR_NULL;
    if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM) return DQK_ERR_SHAPE;
    if (hq / hkv > 64 || batch > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(q_prime) || !aligned16(sel_idx)) return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_select(static_cast<const uint16_t *>(q_bf16), t_q, batch, hq, hkv, n_keep, q_prime,
                                         sel_idx, stream));
}

int dqk_quantize_append(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                        int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens, const int32_t *page_table,
                        int32_t max_pages, float *kprime_dbg, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !cu_tokens || !page_table) return DQK_ERR_NULL;
    if (n_seqs < 1 || max_pages < 1 || total_tokens < 1) return DQK_ERR_SHAPE;
    if (n_seqs > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(cu_tokens) ||
        !aligned16(page_table) || (kprime_dbg && !aligned16(kprime_dbg)))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_append(*c, static_cast<const uint16_t *>(k_bf16),
                                         static_cast<const uint16_t *>(v_bf16),
                                         static_cast<const uint16_t *>(t_k_bf16), n_seqs, cu_tokens, page_table,
                                         max_pages, kprime_dbg, stream));
}

size_t dqk_decode_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t max_pages, int32_t num_splits) {
    if (batch < 1 || hq < 1 || hkv < 1 || max_pages < 1 || num_splits < 0) return 0;
    // enough for either decode entry point
    int s = resolve_splits(batch, hq, hkv, max_pages, num_splits, 0);
    const int s_gen = num_splits > 0 ? num_splits : dqk::decode_splits_generic(batch, hkv, max_pages);
    if (s_gen > s) s = s_gen;
    return (size_t)batch * hq * s * dqk::PART_FLOATS * sizeof(float);
}

int dqk_decode_attn(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep, int32_t batch,
                    int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                    float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out, float *lse,
                    hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!q_prime || !sel_idx || !page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || max_pages < 1 ||
        num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    const bool mfma = dqk::use_mfma_decode(hq, hkv);
    if (!mfma && hq / hkv > dqk::GENERIC_MAX_GROUP) return DQK_ERR_UNSUPPORTED;
    if ((int64_t)batch * hkv > 65535 || batch * hq > 2147483647 / 2) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_prime) || !aligned16(sel_idx) || !aligned16(page_table) || !aligned16(seq_lens) ||
        !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    dqk::DecodeArgs a{c,         q_prime,  sel_idx, n_keep, batch,  hq, hkv, page_table, max_pages, seq_lens,
                      sm_scale, splits, static_cast<float *>(workspace), out, lse};
    hipError_t e = mfma ? dqk::launch_decode_mfma(a, stream) : dqk::launch_decode_generic(a, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(dqk::launch_merge(a.partials, batch, hq, splits, out, lse, stream));
}

int dqk_decode_attn_bf16(const void *k_pages, const void *v_pages, int32_t hkv, int32_t num_pages,
                         const void *q_bf16, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                         const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                         size_t ws_bytes, float *out, float *lse, hipStream_t stream) {
    if (!k_pages || !v_pages || !q_bf16 || !page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    if (hkv < 1 || num_pages < 1 || batch < 1 || hq < 1 || hq % hkv != 0 || max_pages < 1 || num_splits < 0 ||
        num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (hq / hkv > dqk::GENERIC_MAX_GROUP || (int64_t)batch * hkv > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(q_bf16) || !aligned16(page_table) ||
        !aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = num_splits > 0 ? num_splits : dqk::decode_splits_generic(batch, hkv, max_pages);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    dqk::DecodeBf16Args a{static_cast<const uint16_t *>(k_pages), static_cast<const uint16_t *>(v_pages), hkv,
                          static_cast<const uint16_t *>(q_bf16), batch, hq, page_table, max_pages, seq_lens,
                          sm_scale, splits, static_cast<float *>(workspace), out, lse};
    return hip_status(dqk::launch_decode_bf16(a, stream));
}

}  // extern "C"
