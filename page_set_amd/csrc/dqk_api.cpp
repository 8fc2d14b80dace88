// libdqk C ABI: argument validation (host only, before anything is enqueued)
// and dispatch to the kernels.  See include/dqk.h for the contract.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>

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
    if (c->num_kv_heads < 1 || c->num_pages < 1 || c->num_pages % dqk::KBLK != 0) return DQK_ERR_SHAPE;
    if (c->num_kv_heads > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(c->k_codes) || !aligned16(c->k_meta) || !aligned16(c->k_ch0) || !aligned16(c->v_codes) ||
        !aligned16(c->v_meta))
        return DQK_ERR_ALIGN;
    return DQK_OK;
}

int check_tiers(const dqk_tiers *t, const dqk_cache *c) {
    if (!t || !t->sink_k || !t->sink_v || !t->tail_k || !t->tail_v || !t->tail_kraw) return DQK_ERR_NULL;
    if (t->batch < 1 || t->num_kv_heads != c->num_kv_heads) return DQK_ERR_SHAPE;
    if (!aligned16(t->sink_k) || !aligned16(t->sink_v) || !aligned16(t->tail_k) || !aligned16(t->tail_v) ||
        !aligned16(t->tail_kraw))
        return DQK_ERR_ALIGN;
    return DQK_OK;
}

// n_keep = 0: the largest count any n_keep can resolve to (workspace sizing)
int resolve_splits(int batch, int hq, int hkv, int max_pages, int num_splits, int n_keep) {
    if (num_splits > 0) return num_splits;
    return dqk::decode_splits_mfma(batch, hkv * dqk::mfma_head_sets(hq, hkv), max_pages, n_keep);
}

// ---- scratch of the entry point that allocates nothing: split partials in a
//      file-scope device array (each GPU the library runs on holds its own copy
//      until the process ends); host code uses only the address
//      hipGetSymbolAddress returns for the current device, never the name.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
__device__ __align__(256) float scratch[NOALLOC_SCRATCH_BYTES / sizeof(float)];
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return DQK_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return DQK_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DQK_OK;
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
    return hip_status(dqk::launch_select(static_cast<const uint16_t *>(q_bf16), t_q, nullptr, batch, hq, hkv, n_keep,
                                         q_prime, sel_idx, stream));
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

int dqk_quantize_append_vrot(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                             const void *r_v_bf16, float clip, int32_t n_seqs, const int32_t *cu_tokens,
                             int64_t total_tokens, const int32_t *page_table, int32_t max_pages, float *kprime_dbg,
                             float *vprime_dbg, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !r_v_bf16 || !cu_tokens || !page_table) return DQK_ERR_NULL;
    if (n_seqs < 1 || max_pages < 1 || total_tokens < 1 || !(clip > 0.0f && clip <= 1.0f)) return DQK_ERR_SHAPE;
    if (n_seqs > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(r_v_bf16) ||
        !aligned16(cu_tokens) || !aligned16(page_table) || (kprime_dbg && !aligned16(kprime_dbg)) ||
        (vprime_dbg && !aligned16(vprime_dbg)))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_append_vrot(
        *c, static_cast<const uint16_t *>(k_bf16), static_cast<const uint16_t *>(v_bf16),
        static_cast<const uint16_t *>(t_k_bf16), static_cast<const uint16_t *>(r_v_bf16), clip, n_seqs, cu_tokens,
        page_table, max_pages, kprime_dbg, vprime_dbg, stream));
}

int dqk_select_channels_base(const void *q_bf16, const float *t_q, const float *sel_scale, int32_t batch,
                             int32_t hq, int32_t hkv, int32_t n_keep, float *q_prime, int32_t *sel_idx,
                             hipStream_t stream) {
    if (!q_bf16 || !t_q || !sel_scale || !q_prime || !sel_idx) return DQK_ERR_NULL;
    if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM) return DQK_ERR_SHAPE;
    if (hq / hkv > 64 || batch > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(sel_scale) || !aligned16(q_prime) || !aligned16(sel_idx))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_select(static_cast<const uint16_t *>(q_bf16), t_q, sel_scale, batch, hq, hkv,
                                         n_keep, q_prime, sel_idx, stream));
}

int dqk_value_unrotate(const float *o_rot, const float *r_v_inv, int32_t batch, int32_t hq, int32_t hkv,
                       float *out, hipStream_t stream) {
    if (!o_rot || !r_v_inv || !out) return DQK_ERR_NULL;
    if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return DQK_ERR_SHAPE;
    if (hq / hkv > 64 || batch > 65535 || hkv > 65535) return DQK_ERR_UNSUPPORTED;
    const uintptr_t a = reinterpret_cast<uintptr_t>(o_rot), o = reinterpret_cast<uintptr_t>(out);
    const uintptr_t n = (uintptr_t)batch * hq * DQK_HEAD_DIM * sizeof(float);
    if (a < o + n && o < a + n) return DQK_ERR_UNSUPPORTED;  // the rows are read by several workgroups
    if (!aligned16(o_rot) || !aligned16(out) || !aligned16(r_v_inv)) return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_value_unrotate(o_rot, r_v_inv, batch, hq, hkv, out, stream));
}

size_t dqk_decode_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t max_pages, int32_t num_splits) {
    if (batch < 1 || hq < 1 || hkv < 1 || max_pages < 1 || num_splits < 0) return 0;
    // enough for either decode entry point (INT2 or the BF16 baseline)
    int s = resolve_splits(batch, hq, hkv, max_pages, num_splits, 0);
    const int s_bf = num_splits > 0 ? num_splits : dqk::decode_splits_bf16(batch, hkv, max_pages);
    if (s_bf > s) s = s_bf;
    return (size_t)batch * hq * s * dqk::PART_FLOATS * sizeof(float);
}

// Decode over the INT2 cache, then the split merge (r_inv non-null: the merge
// followed by the inverse value rotation).
static int decode_core(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                       int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                       const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes,
                       const float *r_inv, float *out, float *lse, hipStream_t stream, bool token_grid = false) {
    int st = check_cache(c);
    if (st) return st;
    if (!q_prime || !sel_idx || !page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || max_pages < 1 ||
        num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (!dqk::use_mfma_decode(hq, hkv, n_keep)) return DQK_ERR_UNSUPPORTED;  // more than MAX_GROUP heads per KV head
    if ((int64_t)batch * hkv * dqk::mfma_head_sets(hq, hkv) > 65535 || batch * hq > 2147483647 / 2)
        return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_prime) || !aligned16(sel_idx) || !aligned16(page_table) || !aligned16(seq_lens) ||
        !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    dqk::DecodeArgs a{c,         q_prime,  sel_idx, n_keep, batch,  hq, hkv, page_table, max_pages, seq_lens,
                      sm_scale, splits, static_cast<float *>(workspace), out, lse};
    a.token_grid = token_grid;
    hipError_t e = dqk::launch_decode_mfma(a, stream);
    if (e != hipSuccess) return hip_status(e);
    if (r_inv) return hip_status(dqk::launch_merge_unrotate(a.partials, batch, hq, hkv, splits, r_inv, out, lse, stream));
    return hip_status(dqk::launch_merge(a.partials, batch, hq, splits, out, lse, stream));
}

// Selection (sel_scale non-null: in base coordinates), decode and merge
// (r_inv non-null: with the inverse value rotation), the selection inside the
// decode launch where the kernel can run it.
static int select_decode_core(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *sel_scale,
                              const float *r_inv, int32_t n_keep, int32_t batch, int32_t hq,
                              const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens, float sm_scale,
                              int32_t num_splits, void *workspace, size_t ws_bytes, float *out, float *lse,
                              float *q_prime, int32_t *sel_idx, hipStream_t stream, bool token_grid = false) {
    int st = check_cache(c);
    if (st) return st;
    if (!q_bf16 || !t_q || !page_table || !seq_lens || !workspace || !out || !q_prime || !sel_idx) return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || max_pages < 1 ||
        num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    // every check of both paths before anything is enqueued
    if (!dqk::use_mfma_decode(hq, hkv, n_keep)) return DQK_ERR_UNSUPPORTED;  // more than MAX_GROUP heads per KV head
    if ((int64_t)batch * hkv * dqk::mfma_head_sets(hq, hkv) > 65535 || batch * hq > 2147483647 / 2)
        return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(q_prime) || !aligned16(sel_idx) ||
        !aligned16(page_table) || !aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    if (!dqk::fused_select_ok(hq, hkv, n_keep, token_grid)) {  // separate launches: selection, then decode
        st = sel_scale ? dqk_select_channels_base(q_bf16, t_q, sel_scale, batch, hq, hkv, n_keep, q_prime, sel_idx,
                                                  stream)
                       : dqk_select_channels(q_bf16, t_q, batch, hq, hkv, n_keep, q_prime, sel_idx, stream);
        if (st) return st;
        return decode_core(c, q_prime, sel_idx, n_keep, batch, hq, page_table, max_pages, seq_lens, sm_scale,
                           num_splits, workspace, ws_bytes, r_inv, out, lse, stream, token_grid);
    }
    dqk::DecodeArgs a{c,         nullptr,  nullptr, n_keep, batch,  hq, hkv, page_table, max_pages, seq_lens,
                      sm_scale, splits, static_cast<float *>(workspace), out, lse};
    a.q_bf16 = static_cast<const uint16_t *>(q_bf16);
    a.t_q = t_q;
    a.qp_out = q_prime;
    a.sel_out = sel_idx;
    a.sel_scale = sel_scale;
    a.token_grid = token_grid;
    hipError_t e = dqk::launch_decode_mfma(a, stream);
    if (e != hipSuccess) return hip_status(e);
    if (r_inv) return hip_status(dqk::launch_merge_unrotate(a.partials, batch, hq, hkv, splits, r_inv, out, lse, stream));
    return hip_status(dqk::launch_merge(a.partials, batch, hq, splits, out, lse, stream));
}

int dqk_decode_attn(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep, int32_t batch,
                    int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                    float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out, float *lse,
                    hipStream_t stream) {
    return decode_core(c, q_prime, sel_idx, n_keep, batch, hq, page_table, max_pages, seq_lens, sm_scale, num_splits,
                       workspace, ws_bytes, nullptr, out, lse, stream);
}

int dqk_decode_attn_tokgrid(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                            int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                            size_t ws_bytes, float *out, float *lse, hipStream_t stream) {
    return decode_core(c, q_prime, sel_idx, n_keep, batch, hq, page_table, max_pages, seq_lens, sm_scale, num_splits,
                       workspace, ws_bytes, nullptr, out, lse, stream, true);
}

int dqk_select_decode_attn_tokgrid(const dqk_cache *c, const void *q_bf16, const float *t_q, int32_t n_keep,
                                   int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                                   const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                                   size_t ws_bytes, float *out, float *lse, float *q_prime, int32_t *sel_idx,
                                   hipStream_t stream) {
    return select_decode_core(c, q_bf16, t_q, nullptr, nullptr, n_keep, batch, hq, page_table, max_pages, seq_lens,
                              sm_scale, num_splits, workspace, ws_bytes, out, lse, q_prime, sel_idx, stream, true);
}

int dqk_quantize_append_tokgrid(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                                int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens,
                                const int32_t *page_table, int32_t max_pages, float *kprime_dbg, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !cu_tokens || !page_table) return DQK_ERR_NULL;
    if (n_seqs < 1 || max_pages < 1 || total_tokens < 1) return DQK_ERR_SHAPE;
    if (n_seqs > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(cu_tokens) ||
        !aligned16(page_table) || (kprime_dbg && !aligned16(kprime_dbg)))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_append_tokgrid(*c, static_cast<const uint16_t *>(k_bf16),
                                                 static_cast<const uint16_t *>(v_bf16),
                                                 static_cast<const uint16_t *>(t_k_bf16), n_seqs, cu_tokens,
                                                 page_table, max_pages, kprime_dbg, stream));
}

int dqk_select_decode_attn(const dqk_cache *c, const void *q_bf16, const float *t_q, int32_t n_keep, int32_t batch,
                           int32_t hq, const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                           float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                           float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    return select_decode_core(c, q_bf16, t_q, nullptr, nullptr, n_keep, batch, hq, page_table, max_pages, seq_lens,
                              sm_scale, num_splits, workspace, ws_bytes, out, lse, q_prime, sel_idx, stream);
}

int dqk_select_decode_attn_vrot(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *sel_scale,
                                const float *r_v_inv, int32_t n_keep, int32_t batch, int32_t hq,
                                const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                                float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                                float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    if (!sel_scale || !r_v_inv) return DQK_ERR_NULL;
    if (!aligned16(sel_scale) || !aligned16(r_v_inv)) return DQK_ERR_ALIGN;
    return select_decode_core(c, q_bf16, t_q, sel_scale, r_v_inv, n_keep, batch, hq, page_table, max_pages,
                              seq_lens, sm_scale, num_splits, workspace, ws_bytes, out, lse, q_prime, sel_idx,
                              stream);
}

// ---- bucket-relative RoPE (Dual-QK §3.4, App. C.4)

int dqk_quantize_append_rope(const dqk_cache *c, const void *k_bf16, const void *v_bf16, const void *t_k_bf16,
                             const float *rope_cos, const float *rope_sin, int32_t n_buckets, int32_t n_seqs,
                             const int32_t *cu_tokens, int64_t total_tokens, const int32_t *page_table,
                             int32_t max_pages, float *kprime_dbg, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !rope_cos || !rope_sin || !cu_tokens || !page_table) return DQK_ERR_NULL;
    if (n_seqs < 1 || max_pages < 1 || total_tokens < 1 || n_buckets < 1 ||
        (int64_t)n_buckets * dqk::ROPE_PAGES < max_pages)
        return DQK_ERR_SHAPE;
    if (n_seqs > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(rope_cos) ||
        !aligned16(rope_sin) || !aligned16(cu_tokens) || !aligned16(page_table) ||
        (kprime_dbg && !aligned16(kprime_dbg)))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_append_rope(*c, static_cast<const uint16_t *>(k_bf16),
                                              static_cast<const uint16_t *>(v_bf16),
                                              static_cast<const uint16_t *>(t_k_bf16), rope_cos, rope_sin, n_seqs,
                                              cu_tokens, page_table, max_pages, kprime_dbg, stream));
}

int dqk_select_channels_rope(const void *q_bf16, const float *t_q, const float *rope_cos, const float *rope_sin,
                             int32_t n_buckets, int32_t batch, int32_t hq, int32_t hkv, int32_t n_keep,
                             float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    if (!q_bf16 || !t_q || !rope_cos || !rope_sin || !q_prime || !sel_idx) return DQK_ERR_NULL;
    if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || n_buckets < 1)
        return DQK_ERR_SHAPE;
    if (hq / hkv > 64 || (int64_t)batch * n_buckets > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(rope_cos) || !aligned16(rope_sin) ||
        !aligned16(q_prime) || !aligned16(sel_idx))
        return DQK_ERR_ALIGN;
    return hip_status(dqk::launch_select(static_cast<const uint16_t *>(q_bf16), t_q, nullptr, batch, hq, hkv, n_keep,
                                         q_prime, sel_idx, stream, rope_cos, rope_sin, n_buckets));
}

namespace {
// splits of the bucketed decode: the usual choice, raised so that every split
// holds few enough buckets for the kernel's LDS
int resolve_splits_rope(int batch, int hq, int hkv, int max_pages, int num_splits, int n_keep) {
    const int s = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    const int m = dqk::decode_splits_rope(max_pages, n_keep);
    return s > m ? s : m;
}

// Decode of a cache in bucket frames (one_call: the per-bucket selection
// first) and the split merge.
int rope_decode_core(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *rope_cos,
                     const float *rope_sin, const float *q_prime_in, const int32_t *sel_in, int32_t n_keep,
                     int32_t n_buckets, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                     const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes,
                     float *out, float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    const bool one_call = q_bf16 != nullptr;
    if (one_call ? (!t_q || !rope_cos || !rope_sin || !q_prime || !sel_idx) : (!q_prime_in || !sel_in))
        return DQK_ERR_NULL;
    if (!page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || max_pages < 1 ||
        n_buckets < 1 || (int64_t)n_buckets * dqk::ROPE_PAGES < max_pages || num_splits < 0 ||
        num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (!dqk::use_mfma_decode(hq, hkv, n_keep)) return DQK_ERR_UNSUPPORTED;  // more than MAX_GROUP heads per KV head
    if ((int64_t)batch * hkv * dqk::mfma_head_sets(hq, hkv) > 65535 || (int64_t)batch * n_buckets > 65535 ||
        (int64_t)batch * n_buckets * hq > 2147483647 / 2)
        return DQK_ERR_UNSUPPORTED;
    if (!aligned16(page_table) || !aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    if (one_call ? (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(rope_cos) || !aligned16(rope_sin) ||
                    !aligned16(q_prime) || !aligned16(sel_idx))
                 : (!aligned16(q_prime_in) || !aligned16(sel_in)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits_rope(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    dqk::DecodeArgs a{c,         q_prime_in, sel_in, n_keep, batch, hq, hkv, page_table, max_pages, seq_lens,
                      sm_scale, splits,     static_cast<float *>(workspace), out, lse};
    a.n_buckets = n_buckets;
    if (one_call) {  // the per-bucket selection, then the decode reads it
        hipError_t e = dqk::launch_select(static_cast<const uint16_t *>(q_bf16), t_q, nullptr, batch, hq, hkv, n_keep,
                                          q_prime, sel_idx, stream, rope_cos, rope_sin, n_buckets);
        if (e != hipSuccess) return hip_status(e);
        a.q_prime = q_prime;
        a.sel_idx = sel_idx;
    }
    hipError_t e = dqk::launch_decode_mfma(a, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(dqk::launch_merge(a.partials, batch, hq, splits, out, lse, stream));
}
}  // namespace

size_t dqk_decode_rope_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t n_buckets,
                                      int32_t num_splits) {
    if (batch < 1 || hq < 1 || hkv < 1 || n_buckets < 1 || num_splits < 0) return 0;
    // the splits grow with the page count: size for the most pages n_buckets cover
    const int mp = (int)((int64_t)n_buckets * dqk::ROPE_PAGES > 2147483647 ? 2147483647
                                                                            : n_buckets * dqk::ROPE_PAGES);
    return (size_t)batch * hq * resolve_splits_rope(batch, hq, hkv, mp, num_splits, 0) * dqk::PART_FLOATS *
           sizeof(float);
}

int dqk_decode_attn_rope(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                         int32_t n_buckets, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                         const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                         size_t ws_bytes, float *out, float *lse, hipStream_t stream) {
    return rope_decode_core(c, nullptr, nullptr, nullptr, nullptr, q_prime, sel_idx, n_keep, n_buckets, batch, hq,
                            page_table, max_pages, seq_lens, sm_scale, num_splits, workspace, ws_bytes, out, lse,
                            nullptr, nullptr, stream);
}

int dqk_select_decode_attn_rope(const dqk_cache *c, const void *q_bf16, const float *t_q, const float *rope_cos,
                                const float *rope_sin, int32_t n_keep, int32_t n_buckets, int32_t batch, int32_t hq,
                                const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                                float sm_scale, int32_t num_splits, void *workspace, size_t ws_bytes, float *out,
                                float *lse, float *q_prime, int32_t *sel_idx, hipStream_t stream) {
    if (!q_bf16) return DQK_ERR_NULL;
    return rope_decode_core(c, q_bf16, t_q, rope_cos, rope_sin, nullptr, nullptr, n_keep, n_buckets, batch, hq,
                            page_table, max_pages, seq_lens, sm_scale, num_splits, workspace, ws_bytes, out, lse,
                            q_prime, sel_idx, stream);
}

int dqk_decode_attn_noalloc(const dqk_cache *c, const float *q_prime, const int32_t *sel_idx, int32_t n_keep,
                            int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, float sm_scale, int32_t num_splits, float *out, float *lse,
                            hipStream_t stream) {
    // the checks dqk_decode_attn repeats, here so that the partials' size is
    // known (and rejected when too large) before any HIP call
    int st = check_cache(c);
    if (st) return st;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM || max_pages < 1 ||
        num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if ((size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float) > NOALLOC_SCRATCH_BYTES) return DQK_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st) return st;
    return dqk_decode_attn(c, q_prime, sel_idx, n_keep, batch, hq, page_table, max_pages, seq_lens, sm_scale,
                           num_splits, ws, NOALLOC_SCRATCH_BYTES, out, lse, stream);
}

size_t dqk_decode_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int dqk_prefill_tiered(const dqk_cache *c, const dqk_tiers *tiers, const void *k_bf16, const void *v_bf16,
                       const void *t_k_bf16, int32_t n_seqs, const int32_t *cu_tokens, int64_t total_tokens,
                       const int32_t *page_table, int32_t max_pages, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    st = check_tiers(tiers, c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !cu_tokens || !page_table) return DQK_ERR_NULL;
    if (n_seqs < 1 || n_seqs > tiers->batch || max_pages < 1 || total_tokens < 1) return DQK_ERR_SHAPE;
    if (n_seqs > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(cu_tokens) ||
        !aligned16(page_table))
        return DQK_ERR_ALIGN;
    const uint16_t *k = static_cast<const uint16_t *>(k_bf16), *v = static_cast<const uint16_t *>(v_bf16);
    const uint16_t *tk = static_cast<const uint16_t *>(t_k_bf16);
    hipError_t e = dqk::launch_tier_fill(*tiers, k, v, tk, n_seqs, cu_tokens, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(dqk::launch_append_tiered(*c, k, v, tk, n_seqs, cu_tokens, page_table, max_pages, stream));
}

int dqk_append_token(const dqk_cache *c, const dqk_tiers *tiers, const void *k_bf16, const void *v_bf16,
                     const void *t_k_bf16, int32_t batch, const int32_t *lens_before, const int32_t *page_table,
                     int32_t max_pages, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    st = check_tiers(tiers, c);
    if (st) return st;
    if (!k_bf16 || !v_bf16 || !t_k_bf16 || !lens_before || !page_table) return DQK_ERR_NULL;
    if (batch < 1 || batch > tiers->batch || max_pages < 1) return DQK_ERR_SHAPE;
    if (batch > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(t_k_bf16) || !aligned16(lens_before) ||
        !aligned16(page_table))
        return DQK_ERR_ALIGN;
    const uint16_t *k = static_cast<const uint16_t *>(k_bf16), *v = static_cast<const uint16_t *>(v_bf16);
    const uint16_t *tk = static_cast<const uint16_t *>(t_k_bf16);
    hipError_t e = dqk::launch_tier_token(*tiers, k, v, tk, batch, lens_before, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(dqk::launch_pack_tail(*c, *tiers, tk, batch, lens_before, page_table, max_pages, stream));
}

namespace {
// workspace of the tiered decode: INT2 split partials, one partial per row
// for the BF16 tokens, the INT2 lengths
size_t tiered_ws_bytes(int batch, int hq, int splits) {
    const size_t main = (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float);
    const size_t tier = (size_t)batch * hq * dqk::TIER_PARTIALS * dqk::PART_FLOATS * sizeof(float);
    const size_t lens = ((size_t)batch * sizeof(int32_t) + 15) / 16 * 16;
    return main + tier + lens;
}
}  // namespace

size_t dqk_decode_tiered_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t max_pages,
                                        int32_t num_splits) {
    if (batch < 1 || hq < 1 || hkv < 1 || max_pages < 1 || num_splits < 0) return 0;
    return tiered_ws_bytes(batch, hq, resolve_splits(batch, hq, hkv, max_pages, num_splits, 0));
}

int dqk_decode_attn_tiered(const dqk_cache *c, const dqk_tiers *tiers, const float *q_prime, const int32_t *sel_idx,
                           int32_t n_keep, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                           size_t ws_bytes, float *out, float *lse, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    st = check_tiers(tiers, c);
    if (st) return st;
    if (!q_prime || !sel_idx || !page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    if (batch < 1 || batch > tiers->batch || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM ||
        max_pages < 1 || num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (!dqk::use_mfma_decode(hq, hkv, n_keep)) return DQK_ERR_UNSUPPORTED;  // more than MAX_GROUP heads per KV head
    if ((int64_t)batch * hkv * dqk::mfma_head_sets(hq, hkv) > 65535 || batch * hq > 2147483647 / 2)
        return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_prime) || !aligned16(sel_idx) || !aligned16(page_table) || !aligned16(seq_lens) ||
        !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < tiered_ws_bytes(batch, hq, splits)) return DQK_ERR_WORKSPACE;
    float *parts = static_cast<float *>(workspace);
    float *tier_parts = parts + (size_t)batch * hq * splits * dqk::PART_FLOATS;
    int32_t *int2_lens =
        reinterpret_cast<int32_t *>(tier_parts + (size_t)batch * hq * dqk::TIER_PARTIALS * dqk::PART_FLOATS);
    // the BF16 tokens first: that kernel also writes the INT2 lengths the decode reads
    hipError_t e = dqk::launch_tier_decode(*tiers, q_prime, sel_idx, n_keep, batch, hq, seq_lens, sm_scale, tier_parts,
                                           int2_lens, stream);
    if (e != hipSuccess) return hip_status(e);
    dqk::DecodeArgs a{c,         q_prime,  sel_idx, n_keep, batch, hq, hkv, page_table, max_pages, int2_lens,
                      sm_scale, splits, parts,   out,    lse};
    e = dqk::launch_decode_mfma(a, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(
        dqk::launch_merge_extra(parts, batch, hq, splits, tier_parts, dqk::TIER_PARTIALS, out, lse, stream));
}

int dqk_select_decode_attn_tiered(const dqk_cache *c, const dqk_tiers *tiers, const void *q_bf16, const float *t_q,
                                  int32_t n_keep, int32_t batch, int32_t hq, const int32_t *page_table,
                                  int32_t max_pages, const int32_t *seq_lens, float sm_scale, int32_t num_splits,
                                  void *workspace, size_t ws_bytes, float *out, float *lse, float *q_prime,
                                  int32_t *sel_idx, hipStream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    st = check_tiers(tiers, c);
    if (st) return st;
    if (!q_bf16 || !t_q || !q_prime || !sel_idx || !page_table || !seq_lens || !workspace || !out)
        return DQK_ERR_NULL;
    const int hkv = c->num_kv_heads;
    // every check of both paths before anything is enqueued
    if (batch < 1 || batch > tiers->batch || hq < 1 || hq % hkv != 0 || n_keep < 1 || n_keep > DQK_HEAD_DIM ||
        max_pages < 1 || num_splits < 0 || num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (hq / hkv > 64) return DQK_ERR_UNSUPPORTED;  // the selection's limit
    if (!dqk::use_mfma_decode(hq, hkv, n_keep)) return DQK_ERR_UNSUPPORTED;
    if ((int64_t)batch * hkv * dqk::mfma_head_sets(hq, hkv) > 65535 || batch * hq > 2147483647 / 2)
        return DQK_ERR_UNSUPPORTED;
    if (!aligned16(q_bf16) || !aligned16(t_q) || !aligned16(q_prime) || !aligned16(sel_idx) ||
        !aligned16(page_table) || !aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = resolve_splits(batch, hq, hkv, max_pages, num_splits, n_keep);
    if (ws_bytes < tiered_ws_bytes(batch, hq, splits)) return DQK_ERR_WORKSPACE;
    // the selection, then the tiered decode (the BF16 tokens score with it).
    // Moving the selection into the INT2 decode's prologue, with the BF16
    // tokens scored after that launch, measured slower on this path than two
    // launches, so the entry makes the two calls.
    st = dqk_select_channels(q_bf16, t_q, batch, hq, hkv, n_keep, q_prime, sel_idx, stream);
    if (st) return st;
    return dqk_decode_attn_tiered(c, tiers, q_prime, sel_idx, n_keep, batch, hq, page_table, max_pages, seq_lens,
                                  sm_scale, num_splits, workspace, ws_bytes, out, lse, stream);
}

int dqk_decode_attn_bf16(const void *k_pages, const void *v_pages, int32_t hkv, int32_t num_pages,
                         const void *q_bf16, int32_t batch, int32_t hq, const int32_t *page_table, int32_t max_pages,
                         const int32_t *seq_lens, float sm_scale, int32_t num_splits, void *workspace,
                         size_t ws_bytes, float *out, float *lse, hipStream_t stream) {
    if (!k_pages || !v_pages || !q_bf16 || !page_table || !seq_lens || !workspace || !out) return DQK_ERR_NULL;
    if (hkv < 1 || num_pages < 1 || batch < 1 || hq < 1 || hq % hkv != 0 || max_pages < 1 || num_splits < 0 ||
        num_splits > max_pages)
        return DQK_ERR_SHAPE;
    if (hq / hkv > dqk::MAX_GROUP || (int64_t)batch * hkv > 65535) return DQK_ERR_UNSUPPORTED;
    if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(q_bf16) || !aligned16(page_table) ||
        !aligned16(seq_lens) || !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
        return DQK_ERR_ALIGN;
    const int splits = num_splits > 0 ? num_splits : dqk::decode_splits_bf16(batch, hkv, max_pages);
    if (ws_bytes < (size_t)batch * hq * splits * dqk::PART_FLOATS * sizeof(float)) return DQK_ERR_WORKSPACE;
    dqk::DecodeBf16Args a{static_cast<const uint16_t *>(k_pages), static_cast<const uint16_t *>(v_pages), hkv,
                          static_cast<const uint16_t *>(q_bf16), batch, hq, page_table, max_pages, seq_lens,
                          sm_scale, splits, static_cast<float *>(workspace), out, lse};
    return hip_status(dqk::launch_decode_bf16(a, stream));
}

}  // extern "C"
