// Protected BF16 tiers (Dual-QK paper §3.3: the first 64 and the most recent
// 256 tokens stay in BF16 for keys and values under the same channel mask;
// §3.4: one softmax over every token).  Layout and the page/tail split are
// documented at dqk_tiers in dqk.h: sink slot t for t < 64, INT2 page i for
// tokens 64 + 128 i .. (P of them, all older than the 256 most recent), tail
// slot (t - 64) mod 384 for the rest.
//
//   tier_fill_kernel    prefill: k' = k T_K (fp32 fma chain over ascending
//                       input channel, rounded to bf16) of the sink and tail
//                       tokens, their values, and the tail's raw keys.
//   tier_token_kernel   one new token per sequence into its tier slot.
//   tier_lens_kernel    128 x (INT2 pages) per sequence, the length the INT2
//                       decode sees.
//   tier_decode_kernel  the BF16 tokens' partial (o, m, l) per query head,
//                       merged with the INT2 splits by the log-sum-exp merge.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t tier_pages(int64_t L) {
    return L >= TIER_SINK + TIER_RECENT ? (L - TIER_SINK - TIER_RECENT) / PG : 0;
}
__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Tier token i of a sequence of length L (sink tokens first, then the tail in
// token order) -> its token index; n_tier = number of tier tokens.
__device__ __forceinline__ void tier_extent(int64_t L, int &n_sink, int64_t &tail0, int &n_tier) {
    n_sink = (int)min<int64_t>(L, TIER_SINK);
    tail0 = TIER_SINK + (int64_t)PG * tier_pages(L);
    n_tier = n_sink + (int)(L > tail0 ? L - tail0 : 0);
}
__device__ __forceinline__ int64_t tier_token(int i, int n_sink, int64_t tail0) {
    return i < n_sink ? (int64_t)i : tail0 + (i - n_sink);
}
// slot row of token t of (sequence b, KV head g): sink [b][g][64], tail [b][g][384]
__device__ __forceinline__ size_t sink_row(int b, int g, int hkv, int64_t t) {
    return ((size_t)b * hkv + g) * TIER_SINK + (size_t)t;
}
__device__ __forceinline__ size_t tail_row(int b, int g, int hkv, int64_t t) {
    return ((size_t)b * hkv + g) * TIER_TAIL_SLOTS + (size_t)((t - TIER_SINK) % TIER_TAIL_SLOTS);
}

constexpr int FILL_TOK = 64;  // tier tokens per workgroup of the prefill fill

// grid (ceil(447 / 64), n_seqs, hkv), 256 lanes: T_K and the chunk's raw keys
// in LDS; thread (token tid / 4, output channels 32 (tid % 4) ..) sums over
// the input channels in ascending order.
__global__ __launch_bounds__(256) void tier_fill_kernel(dqk_tiers t, const uint16_t *__restrict__ kin,
                                                        const uint16_t *__restrict__ vin,
                                                        const uint16_t *__restrict__ t_k,
                                                        const int32_t *__restrict__ cu_tokens) {
    __shared__ float T[D][D + 1];
    __shared__ float kr[FILL_TOK][D + 1];
    const int b = blockIdx.y, g = blockIdx.z, hkv = t.num_kv_heads;
    const int64_t tok0 = cu_tokens[b];
    const int64_t L = (int64_t)cu_tokens[b + 1] - tok0;
    int n_sink, n_tier;
    int64_t tail0;
    tier_extent(L, n_sink, tail0, n_tier);
    const int i0 = blockIdx.x * FILL_TOK;
    if (i0 >= n_tier) return;
    const int n = min(FILL_TOK, n_tier - i0);
    const int tid = threadIdx.x;
    const uint16_t *Tg = t_k + (size_t)g * D * D;
    for (int e = tid; e < D * D; e += 256) T[e / D][e % D] = bf(Tg[e]);
    for (int e = tid; e < n * D; e += 256) {
        const int r = e / D, ch = e % D;
        const int64_t tok = tier_token(i0 + r, n_sink, tail0);
        kr[r][ch] = bf(kin[((size_t)(tok0 + tok) * hkv + g) * D + ch]);
    }
    __syncthreads();
    const int r = tid >> 2, j0 = (tid & 3) * 32;
    if (r < n) {
        const int64_t tok = tier_token(i0 + r, n_sink, tail0);
        const size_t src = ((size_t)(tok0 + tok) * hkv + g) * D;
        const bool in_sink = tok < TIER_SINK;
        const size_t row = in_sink ? sink_row(b, g, hkv, tok) : tail_row(b, g, hkv, tok);
        uint16_t *kdst = (in_sink ? t.sink_k : t.tail_k) + row * D;
        uint16_t *vdst = (in_sink ? t.sink_v : t.tail_v) + row * D;
        for (int j = j0; j < j0 + 32; ++j) {
            float acc = 0.0f;
            for (int i = 0; i < D; ++i) acc = __builtin_fmaf(kr[r][i], T[i][j], acc);
            kdst[j] = f2bf_rne(acc);
        }
        for (int j = j0; j < j0 + 32; ++j) {
            vdst[j] = vin[src + j];
            if (!in_sink) t.tail_kraw[row * D + j] = kin[src + j];
        }
    }
}

// grid (batch, hkv), 128 lanes: lane j computes k'_j of the sequence's new token.
__global__ __launch_bounds__(D) void tier_token_kernel(dqk_tiers t, const uint16_t *__restrict__ kin,
                                                       const uint16_t *__restrict__ vin,
                                                       const uint16_t *__restrict__ t_k,
                                                       const int32_t *__restrict__ lens_before) {
    __shared__ float kr[D];
    const int b = blockIdx.x, g = blockIdx.y, hkv = t.num_kv_heads, j = threadIdx.x;
    const int64_t tok = lens_before[b];
    const size_t src = ((size_t)b * hkv + g) * D;
    kr[j] = bf(kin[src + j]);
    __syncthreads();
    const uint16_t *Tg = t_k + (size_t)g * D * D;
    float acc = 0.0f;
    for (int i = 0; i < D; ++i) acc = __builtin_fmaf(kr[i], bf(Tg[(size_t)i * D + j]), acc);
    const bool in_sink = tok < TIER_SINK;
    const size_t row = in_sink ? sink_row(b, g, hkv, tok) : tail_row(b, g, hkv, tok);
    (in_sink ? t.sink_k : t.tail_k)[row * D + j] = f2bf_rne(acc);
    (in_sink ? t.sink_v : t.tail_v)[row * D + j] = vin[src + j];
    if (!in_sink) t.tail_kraw[row * D + j] = kin[src + j];
}

__global__ void tier_lens_kernel(const int32_t *__restrict__ seq_lens, int batch, int32_t *__restrict__ int2_lens) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < batch) int2_lens[b] = (int32_t)(PG * tier_pages(seq_lens[b]));
}

constexpr int MAX_TIER = TIER_SINK + TIER_RECENT + PG - 1;  // 447 tier tokens at most
constexpr int TD_MAXG = 16;                                  // query heads per KV head

// grid (batch * hkv), 256 lanes.  Logits of the tier tokens for the group's
// query heads (masked q' in LDS, one token per lane, fp32 fma over ascending
// channel), per-head maximum and exp-sum, then o[h][c] with lane c.
__global__ __launch_bounds__(256) void tier_decode_kernel(dqk_tiers t, const float *__restrict__ q_prime,
                                                          const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          float *__restrict__ part) {
    __shared__ float qm[TD_MAXG][D];
    __shared__ float x[TD_MAXG][MAX_TIER];
    __shared__ float red[4];
    __shared__ float m_s[TD_MAXG], l_s[TD_MAXG];
    const int hkv = t.num_kv_heads, grp = hq / hkv;
    const int b = blockIdx.x / hkv, g = blockIdx.x % hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t L = seq_lens[b];
    int n_sink, n_tier;
    int64_t tail0;
    tier_extent(L, n_sink, tail0, n_tier);

    for (int e = tid; e < grp * D; e += 256) qm[e / D][e % D] = 0.0f;
    __syncthreads();
    const int32_t *sel = sel_idx + ((size_t)b * hkv + g) * n_keep;
    for (int e = tid; e < grp * n_keep; e += 256) {
        const int h = e / n_keep, jj = sel[e % n_keep];
        qm[h][jj] = q_prime[((size_t)b * hq + (size_t)g * grp + h) * D + jj];
    }
    __syncthreads();
    // ---- logits
    for (int i = tid; i < n_tier; i += 256) {
        const int64_t tok = tier_token(i, n_sink, tail0);
        const uint16_t *kr = (tok < TIER_SINK ? t.sink_k + sink_row(b, g, hkv, tok) * D
                                              : t.tail_k + tail_row(b, g, hkv, tok) * D);
        float acc[TD_MAXG];
#pragma unroll
        for (int h = 0; h < TD_MAXG; ++h) acc[h] = 0.0f;
        for (int c8 = 0; c8 < D; c8 += 8) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(kr + c8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kv = __uint_as_float(e & 1 ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
#pragma unroll
                for (int h = 0; h < TD_MAXG; ++h)
                    if (h < grp) acc[h] = __builtin_fmaf(qm[h][c8 + e], kv, acc[h]);
            }
        }
#pragma unroll
        for (int h = 0; h < TD_MAXG; ++h)
            if (h < grp) x[h][i] = acc[h] * sm_scale;
    }
    __syncthreads();
    // ---- per head: maximum, weights exp(x - m), their sum
    for (int h = 0; h < grp; ++h) {
        float m = -__builtin_huge_valf();
        for (int i = tid; i < n_tier; i += 256) m = fmaxf(m, x[h][i]);
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (lane == 0) red[wv] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float l = 0.0f;
        for (int i = tid; i < n_tier; i += 256) {
            const float p = __expf(x[h][i] - m);
            x[h][i] = p;
            l += p;
        }
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
        if (lane == 0) red[wv] = l;
        __syncthreads();
        if (tid == 0) {
            m_s[h] = m;
            l_s[h] = red[0] + red[1] + red[2] + red[3];
        }
        __syncthreads();
    }
    // ---- o[h][c] = sum_i p[h][i] v[i][c]: lane c, heads h = half, half + 2, ...
    const int c = tid & (D - 1), half = tid >> 7;
    float o[TD_MAXG / 2];
#pragma unroll
    for (int k = 0; k < TD_MAXG / 2; ++k) o[k] = 0.0f;
    for (int i = 0; i < n_tier; ++i) {
        const int64_t tok = tier_token(i, n_sink, tail0);
        const float vv = bf(tok < TIER_SINK ? t.sink_v[sink_row(b, g, hkv, tok) * D + c]
                                            : t.tail_v[tail_row(b, g, hkv, tok) * D + c]);
#pragma unroll
        for (int k = 0; k < TD_MAXG / 2; ++k) {
            const int h = half + 2 * k;
            if (h < grp) o[k] = __builtin_fmaf(x[h][i], vv, o[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < TD_MAXG / 2; ++k) {
        const int h = half + 2 * k;
        if (h < grp) {
            float *dst = part + ((size_t)b * hq + (size_t)g * grp + h) * PART_FLOATS;
            dst[c] = o[k];
            if (c == 0) {
                dst[D] = m_s[h];
                dst[D + 1] = l_s[h];
                dst[D + 2] = l_s[h];
            }
        }
    }
}

}  // namespace

hipError_t launch_tier_fill(const dqk_tiers &t, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                            int n_seqs, const int32_t *cu_tokens, hipStream_t s) {
    dim3 grid((MAX_TIER + FILL_TOK - 1) / FILL_TOK, n_seqs, t.num_kv_heads);
    hipLaunchKernelGGL(tier_fill_kernel, grid, dim3(256), 0, s, t, k, v, t_k, cu_tokens);
    return hipGetLastError();
}

hipError_t launch_tier_token(const dqk_tiers &t, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                             int batch, const int32_t *lens_before, hipStream_t s) {
    hipLaunchKernelGGL(tier_token_kernel, dim3(batch, t.num_kv_heads), dim3(D), 0, s, t, k, v, t_k, lens_before);
    return hipGetLastError();
}

hipError_t launch_tier_lens(const int32_t *seq_lens, int batch, int32_t *int2_lens, hipStream_t s) {
    hipLaunchKernelGGL(tier_lens_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, seq_lens, batch, int2_lens);
    return hipGetLastError();
}

hipError_t launch_tier_decode(const dqk_tiers &t, const float *q_prime, const int32_t *sel_idx, int n_keep, int batch,
                              int hq, const int32_t *seq_lens, float sm_scale, float *tier_partials, hipStream_t s) {
    hipLaunchKernelGGL(tier_decode_kernel, dim3(batch * t.num_kv_heads), dim3(256), 0, s, t, q_prime, sel_idx, n_keep,
                       hq, seq_lens, sm_scale, tier_partials);
    return hipGetLastError();
}

}  // namespace dqk
