// Internal declarations shared by libdqk's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqk.h"

namespace dqk {

constexpr int D = DQK_HEAD_DIM;
constexpr int PG = DQK_PAGE;
constexpr int ROW_BYTES = 32;     // 128 two-bit codes
constexpr int VGROUPS = 4;        // value groups of 32 channels

// BF16 tiers: sink tokens, the recent window, tail ring slots.
constexpr int TIER_SINK = DQK_TIER_SINK;
constexpr int TIER_RECENT = DQK_TIER_RECENT;
constexpr int TIER_TAIL_SLOTS = DQK_TIER_TAIL_SLOTS;
// partials of the BF16 tokens per (sequence, query head): 64 tokens each
constexpr int TIER_PARTIALS = (TIER_SINK + TIER_RECENT + 128 - 1 + 63) / 64;

// Physical pages come in aligned blocks of eight: key rows and key metadata of
// a channel sit side by side for the block's eight pages.
constexpr int KBLK = 8;

// Index of the 32-byte key row (and of the (scale, zero) pair) of channel j of
// physical page p, KV head g.
__host__ __device__ __forceinline__ size_t krow(int64_t p, int g, int hkv, int j) {
    return ((((size_t)(p / KBLK) * (size_t)hkv + (size_t)g) * D + (size_t)j) * KBLK) + (size_t)(p % KBLK);
}

// With one key grid per token (the layout of dqk_quantize_append_tokgrid):
// index of the (scale, zero) pair of token s of physical page p, KV head g --
// the block's key metadata read token-major, [P/8][Hkv][8 slot][128 tok][2].
__host__ __device__ __forceinline__ size_t ktok(int64_t p, int g, int hkv, int s) {
    return (((size_t)(p / KBLK) * (size_t)hkv + (size_t)g) * KBLK + (size_t)(p % KBLK)) * PG + (size_t)s;
}

// Partial of one (b, h, split): o[128] (unnormalised, relative to m), m (natural
// log units), l (the denominator matching o), l32 (fp32 sum of the unrounded
// probabilities, for the log-sum-exp), pad.
constexpr int PART_FLOATS = D + 4;

// ---------------------------------------------------------------- formats
// binary16 bits -> fp32 (exact).
__device__ __forceinline__ float h2f(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf_rne(float x) {
    uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- bucket-relative RoPE
// Stored keys live in the frame of their bucket's anchor (Dual-QK paper, §3.4
// and App. C.4): bucket k of a sequence holds positions 2048 k .. 2048 k + 2047
// (sixteen whole pages), anchor a_k = 2048 k.  A bucket's table holds
// cos(a_k theta_i) and -sin(a_k theta_i) for the rotate-half channel pairs
// (i, i + 64), i = 0..63.
constexpr int ROPE_BUCKET = 2048;
constexpr int ROPE_PAGES = ROPE_BUCKET / PG;

// Channel j of a vector turned by a table entry (c, s) of its pair: x is
// channel j, xp its partner j ^ 64; lower half x c - xp s, upper half
// x c + xp s, each product and the sum rounded to fp32.
__device__ __forceinline__ float rope_turn(float x, float xp, float c, float s, bool lower) {
    const float a = __fmul_rn(x, c), b = __fmul_rn(xp, s);
    return lower ? __fsub_rn(a, b) : __fadd_rn(a, b);
}

// ---------------------------------------------------------------- channel selection
// The n_keep channels of one mask (Dual-QK paper, §3.2 Eq. 4), found by one
// wave: lane l holds the pooled energies ea of channel l and eb of channel
// l + 64.  Channel j is kept iff fewer than n_keep channels beat it (larger
// energy, or equal energy at a lower index).  Energies are sums of squares
// (>= +0), whose bit patterns order like their values, so a radix select over
// the 32 bits (one ballot count per bit, from the top) finds the n_keep-th
// largest energy T; the channels above T and the lowest-indexed channels equal
// to T up to n_keep are kept.  pa / pb: output positions of the two channels
// in the ascending list.  Exactly n_keep channels are kept whatever the bits
// (NaN energies included), so positions stay below n_keep.
struct KeptPair {
    bool ka, kb;
    int pa, pb;
};
__device__ __forceinline__ KeptPair top_k_wave(float ea, float eb, int n_keep) {
    const int lane = __lane_id();
    const uint32_t ua = __float_as_uint(ea), ub = __float_as_uint(eb);
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        if (__popcll(__ballot(ua >= cand)) + __popcll(__ballot(ub >= cand)) >= n_keep) thr = cand;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    const unsigned long long eqa = __ballot(ua == thr), eqb = __ballot(ub == thr);
    const int need = n_keep - __popcll(__ballot(ua > thr)) - __popcll(__ballot(ub > thr));  // >= 1
    KeptPair r;
    r.ka = ua > thr || (ua == thr && __popcll(eqa & below) < need);
    r.kb = ub > thr || (ub == thr && __popcll(eqa) + __popcll(eqb & below) < need);
    const unsigned long long ma = __ballot(r.ka), mb = __ballot(r.kb);
    r.pa = __popcll(ma & below);
    r.pb = __popcll(ma) + __popcll(mb & below);
    return r;
}

// |x| onto the binary16 grid toward zero: bits of the magnitude, and whether
// the value was inexact.  Magnitudes above 65504 saturate to 65504 (inexact).
__device__ __forceinline__ uint32_t f16_mag_trunc(uint32_t ua, bool &inexact) {
    // ua: fp32 bits with the sign cleared
    if (ua > 0x477FE000u) {  // 65504.0f
        inexact = true;
        return 0x7BFFu;
    }
    int e = (int)(ua >> 23) - 127;
    if (e >= -14) {
        uint32_t m = ua & 0x7FFFFFu;
        inexact = (m & 0x1FFFu) != 0;
        return ((uint32_t)(e + 15) << 10) | (m >> 13);
    }
    // below the binary16 normal range: multiples of 2^-24
    float a = __uint_as_float(ua) * 16777216.0f;  // exact power-of-two scaling
    float fl = floorf(a);
    inexact = fl != a;
    return (uint32_t)fl;
}

// Largest binary16 <= x, and smallest binary16 >= x.  Sign of zero follows x.
__device__ __forceinline__ uint16_t f16_round_down(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 16) & 0x8000u;
    bool inexact;
    uint32_t m = f16_mag_trunc(u & 0x7FFFFFFFu, inexact);
    if (s && inexact) m += 1;  // negative: move the magnitude up
    return (uint16_t)(s | m);
}

__device__ __forceinline__ uint16_t f16_round_up(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 16) & 0x8000u;
    bool inexact;
    uint32_t m = f16_mag_trunc(u & 0x7FFFFFFFu, inexact);
    if (!s && inexact) m += 1;
    return (uint16_t)(s | m);
}

// INT2 grid of a group from its min and max (signed zeros taken as +0).
struct Grid {
    float s, z;
    uint16_t sb, zb;
};

__device__ __forceinline__ Grid make_grid(float mn, float mx) {
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    Grid g;
    g.zb = f16_round_down(mn);
    g.z = h2f(g.zb);
    float d = __fsub_rn(mx, g.z);
    float t = __fdiv_rn(d, 3.0f);
    g.sb = f16_round_up(t);
    g.s = h2f(g.sb);
    return g;
}

struct Thresholds {
    float t0, t1, t2;
};

__device__ __forceinline__ Thresholds thresholds(const Grid &g) {
    return {__builtin_fmaf(0.5f, g.s, g.z), __builtin_fmaf(1.5f, g.s, g.z), __builtin_fmaf(2.5f, g.s, g.z)};
}

__device__ __forceinline__ uint32_t code2(float x, const Thresholds &t) {
    return (uint32_t)(x >= t.t0) + (uint32_t)(x >= t.t1) + (uint32_t)(x >= t.t2);
}

// ---------------------------------------------------------------- split merge
// Log-sum-exp merge of one (sequence, query head) row: part(s) -> partial s
// (o[128], m, l, l32), s < nsplit.  Executed by 128 lanes (tid 0..127, lane =
// output channel) of a workgroup; every lane of the workgroup calls it (the
// barriers are workgroup-wide), `active` false for lanes that only take part
// in the barriers (a workgroup may merge several rows side by side).  w_lds: 128 floats, red: [3][2] floats of LDS owned by this
// row.  Writes out[c] = sum_s w_s o_s[c] / sum_s w_s l_s and *lse = M +
// log(sum_s w_s l32_s), w_s = exp(m_s - M) (0 for an empty partial).
constexpr int MERGE_FAST = 32;  // splits whose partials one lane keeps in registers

template <typename Part>
__device__ __forceinline__ void merge_row(Part part, int nsplit, int tid, bool active, float *__restrict__ out,
                                          float *__restrict__ lse, float *w_lds, float (*red)[D / 64]) {
    const int lane = tid & 63, wv = tid >> 6;
    // every load that does not depend on the maximum is issued up front
    float xf[MERGE_FAST];
    if (active && nsplit <= MERGE_FAST) {
#pragma unroll
        for (int s = 0; s < MERGE_FAST; ++s) xf[s] = s < nsplit ? part(s)[tid] : 0.0f;
    }
    float M = -__builtin_huge_valf(), m_own = -__builtin_huge_valf(), l_own = 0.0f, l32_own = 0.0f;
    if (active && tid < nsplit) {
        m_own = part(tid)[D];
        l_own = part(tid)[D + 1];
        l32_own = part(tid)[D + 2];
    }
    M = m_own;
    if (active)
        for (int s = tid + D; s < nsplit; s += D) M = fmaxf(M, part(s)[D]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (active && lane == 0) red[0][wv] = M;
    __syncthreads();
    if (active) M = fmaxf(red[0][0], red[0][1]);
    float lpart = 0.0f, l32part = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += D) {
        const int n = min(D, nsplit - s0);
        if (s0 > 0) __syncthreads();  // previous chunk's weights are consumed
        if (active && tid < n) {
            float m = m_own, l = l_own, l32 = l32_own;
            if (s0 > 0) {
                m = part(s0 + tid)[D];
                l = part(s0 + tid)[D + 1];
                l32 = part(s0 + tid)[D + 2];
            }
            const float w = l > 0.0f ? __expf(m - M) : 0.0f;
            w_lds[tid] = w;
            lpart = __builtin_fmaf(l, w, lpart);
            l32part = __builtin_fmaf(l32, w, l32part);
        }
        __syncthreads();
        if (!active) continue;
        if (nsplit <= MERGE_FAST) {
#pragma unroll
            for (int s = 0; s < MERGE_FAST; ++s)
                if (s < n) acc = __builtin_fmaf(xf[s], w_lds[s], acc);
        } else {
            int s = 0;
            for (; s + 8 <= n; s += 8) {  // eight independent loads in flight, sums kept in split order
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = part(s0 + s + e)[tid];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], w_lds[s + e], acc);
            }
            for (; s < n; ++s) acc = __builtin_fmaf(part(s0 + s)[tid], w_lds[s], acc);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lpart += __shfl_xor(lpart, o);
        l32part += __shfl_xor(l32part, o);
    }
    if (active && lane == 0) {
        red[1][wv] = lpart;
        red[2][wv] = l32part;
    }
    __syncthreads();
    if (!active) return;
    const float Lsum = red[1][0] + red[1][1];
    out[tid] = acc / Lsum;
    if (lse && tid == 0) *lse = M + __logf(red[2][0] + red[2][1]);
}

// ---------------------------------------------------------------- launchers
// rope_cos / rope_sin non-null: one selection per (sequence, bucket) of the
// query turned by the bucket's table, q_prime [batch][n_buckets][hq][128] and
// sel_idx [batch][n_buckets][hkv][n_keep]; null: n_buckets must be 1.
hipError_t launch_select(const uint16_t *q, const float *t_q, const float *sel_scale, int batch, int hq, int hkv,
                         int n_keep, float *q_prime, int32_t *sel_idx, hipStream_t s,
                         const float *rope_cos = nullptr, const float *rope_sin = nullptr, int n_buckets = 1);

hipError_t launch_append(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k, int n_seqs,
                         const int32_t *cu_tokens, const int32_t *page_table, int max_pages, float *kprime_dbg,
                         hipStream_t s);
hipError_t launch_append_tiered(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                                int n_seqs, const int32_t *cu_tokens, const int32_t *page_table, int max_pages,
                                hipStream_t s);
hipError_t launch_append_tokgrid(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                                 int n_seqs, const int32_t *cu_tokens, const int32_t *page_table, int max_pages,
                                 float *kprime_dbg, hipStream_t s);
hipError_t launch_append_vrot(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                              const uint16_t *r_v, float clip, int n_seqs, const int32_t *cu_tokens,
                              const int32_t *page_table, int max_pages, float *kprime_dbg, float *vprime_dbg,
                              hipStream_t s);
// keys turned back to their bucket's anchor before T_K (tables [n_buckets][64])
hipError_t launch_append_rope(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                              const float *rope_cos, const float *rope_sin, int n_seqs, const int32_t *cu_tokens,
                              const int32_t *page_table, int max_pages, float *kprime_dbg, hipStream_t s);
// inverse value rotation of decode outputs (dqk_vrot.hip); the split merge followed by it
hipError_t launch_value_unrotate(const float *o_rot, const float *r_inv, int batch, int hq, int hkv, float *out,
                                 hipStream_t s);
hipError_t launch_merge_unrotate(const float *partials, int batch, int hq, int hkv, int num_splits,
                                 const float *r_inv, float *out, float *lse, hipStream_t s);
hipError_t launch_pack_tail(const dqk_cache &c, const dqk_tiers &t, const uint16_t *t_k, int batch,
                            const int32_t *lens_before, const int32_t *page_table, int max_pages, hipStream_t s);
// BF16 tiers (dqk_tiers.hip)
hipError_t launch_tier_fill(const dqk_tiers &t, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                            int n_seqs, const int32_t *cu_tokens, hipStream_t s);
hipError_t launch_tier_token(const dqk_tiers &t, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                             int batch, const int32_t *lens_before, hipStream_t s);
hipError_t launch_tier_decode(const dqk_tiers &t, const float *q_prime, const int32_t *sel_idx, int n_keep, int batch,
                              int hq, const int32_t *seq_lens, float sm_scale, float *tier_partials,
                              int32_t *int2_lens, hipStream_t s);

struct DecodeArgs {
    const dqk_cache *c;
    const float *q_prime;
    const int32_t *sel_idx;
    int n_keep, batch, hq, hkv;
    const int32_t *page_table;
    int max_pages;
    const int32_t *seq_lens;
    float sm_scale;
    int num_splits;
    float *partials;
    float *out, *lse;
    // selection fused into the MFMA decode (dqk_select_decode_attn): q bf16
    // [batch][hq][128] and T_Q fp32 [hkv][128][128] replace q_prime / sel_idx
    // as inputs, which then receive the selection's results
    const uint16_t *q_bf16 = nullptr;
    const float *t_q = nullptr;
    float *qp_out = nullptr;
    int32_t *sel_out = nullptr;
    // selection in base coordinates (fused selection only): fp32 [hkv][128] or null
    const float *sel_scale = nullptr;
    // one key grid per token (dqk_quantize_append_tokgrid's layout)
    bool token_grid = false;
    // bucket-relative RoPE: n_buckets > 0 gives q_prime [batch][n_buckets][hq]
    // [128] and sel_idx [batch][n_buckets][hkv][n_keep]; the pages of bucket
    // k (16 k .. 16 k + 15) score with row k; num_splits at least
    // decode_splits_rope (each split holds whole buckets that fit in LDS)
    int n_buckets = 0;
};

// Query heads per KV head that the decode entry points serve.
constexpr int MAX_GROUP = 16;

// The INT2 decode on MFMA: any group size up to MAX_GROUP, the query heads of
// a KV head taken in sets of four (one workgroup per set and split; a set of
// fewer than four is padded with zero queries).
bool use_mfma_decode(int hq, int hkv, int n_keep);  // n_keep 0: any count it serves
int mfma_head_sets(int hq, int hkv);                // sets of four query heads per KV head
int decode_splits_mfma(int batch, int units_per_seq, int max_pages, int n_keep);  // n_keep 0: the largest
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s);
// Split count of the BF16 baseline decode.
int decode_splits_bf16(int batch, int hkv, int max_pages);
// Least split count of the bucketed decode for this context and n_keep.
int decode_splits_rope(int max_pages, int n_keep);
// Whether the MFMA decode can run the selection itself for this n_keep.
bool fused_select_ok(int hq, int hkv, int n_keep, bool token_grid = false);

struct DecodeBf16Args {
    const uint16_t *k_pages, *v_pages;
    int hkv;
    const uint16_t *q;
    int batch, hq;
    const int32_t *page_table;
    int max_pages;
    const int32_t *seq_lens;
    float sm_scale;
    int num_splits;
    float *partials;
    float *out, *lse;
    // selection fused into the MFMA decode (dqk_select_decode_attn): q bf16
    // [batch][hq][128] and T_Q fp32 [hkv][128][128] replace q_prime / sel_idx
    // as inputs, which then receive the selection's results
    const uint16_t *q_bf16 = nullptr;
    const float *t_q = nullptr;
    float *qp_out = nullptr;
    int32_t *sel_out = nullptr;
    // selection in base coordinates (fused selection only): fp32 [hkv][128] or null
    const float *sel_scale = nullptr;
    // one key grid per token (dqk_quantize_append_tokgrid's layout)
    bool token_grid = false;
};

hipError_t launch_decode_bf16(const DecodeBf16Args &a, hipStream_t s);

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);

hipError_t launch_merge(const float *partials, int batch, int hq, int num_splits, float *out, float *lse,
                        hipStream_t s);

// The merge with n_extra more partials per (sequence, query head) row at
// extra + (row * n_extra + i) * PART_FLOATS.
hipError_t launch_merge_extra(const float *partials, int batch, int hq, int num_splits, const float *extra,
                              int n_extra, float *out, float *lse, hipStream_t s);

}  // namespace dqk
