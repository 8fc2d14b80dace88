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
//   tier_decode_kernel  partials (o, m, l) per query head of the BF16 tokens,
//                       64 tokens per workgroup (TIER_PARTIALS per head),
//                       merged with the INT2 splits by the log-sum-exp merge;
//                       it also writes 128 x (INT2 pages) per sequence, the
//                       length the INT2 decode that follows it sees.
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

constexpr int MAX_TIER = TIER_SINK + TIER_RECENT + PG - 1;  // 447 tier tokens at most
constexpr int TD_MAXG = 16;                                  // query heads per KV head, at most
static_assert(TD_MAXG == MAX_GROUP, "the tiered decode serves every group the INT2 decode serves");
constexpr int TCH = 64;                                      // tier tokens per workgroup
constexpr int N_TCH = (MAX_TIER + TCH - 1) / TCH;           // 7 partials per (sequence, query head)

// grid (N_TCH, batch * hkv), 256 lanes: tier tokens 64 c .. 64 c + 63 of one
// (sequence, KV head).  Logits per (token, head) pair (masked q' in LDS, the
// bf16 k' row from memory, fp32 fma over ascending channel); one wave per
// head reduces the chunk's 64 logits to (m, l); lane c then sums p v over
// the chunk.  Writes one partial per query head (empty chunks: m = -inf,
// l = 0).
template <int GRP>
__global__ __launch_bounds__(256) void tier_decode_kernel(dqk_tiers t, const float *__restrict__ q_prime,
                                                          const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          float *__restrict__ part, int32_t *__restrict__ int2_lens) {
    __shared__ float qm[GRP][D];
    __shared__ float x[GRP][TCH];
    __shared__ float m_s[GRP], l_s[GRP];
    __shared__ int keep_s[D];
    constexpr int grp = GRP;
    const int hkv = t.num_kv_heads;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / hkv, g = blockIdx.y % hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t L = seq_lens[b];
    int n_sink, n_tier;
    int64_t tail0;
    tier_extent(L, n_sink, tail0, n_tier);
    const int i0 = chunk * TCH;
    const int n = max(0, min(TCH, n_tier - i0));
    if (chunk == 0 && g == 0 && threadIdx.x == 0) int2_lens[b] = (int32_t)(PG * tier_pages(L));

    if (n == 0) {  // a chunk past the tier tokens: empty partials
        for (int e = tid; e < grp * D; e += 256) {
            float *dst = part + (((size_t)b * hq + (size_t)g * grp + e / D) * N_TCH + chunk) * PART_FLOATS;
            dst[e % D] = 0.0f;
            if (e % D == 0) {
                dst[D] = -__builtin_huge_valf();
                dst[D + 1] = 0.0f;
                dst[D + 2] = 0.0f;
            }
        }
        return;
    }
    // row of chunk token r (r clamped to the chunk, so every load is unconditional):
    // sink slot, or tail slot (t - 64) mod 384 in 32-bit arithmetic
    const size_t sink0 = ((size_t)b * hkv + g) * TIER_SINK, tail_base = ((size_t)b * hkv + g) * TIER_TAIL_SLOTS;
    auto row_of = [&](int r, bool &in_sink) {
        const int i = i0 + min(r, n - 1);
        in_sink = i < n_sink;
        return in_sink ? sink0 + (size_t)i
                       : tail_base + (size_t)((uint32_t)(tail0 - TIER_SINK + (i - n_sink)) % (uint32_t)TIER_TAIL_SLOTS);
    };
    auto krow_of = [&](int r) {
        bool s0;
        const size_t row = row_of(r, s0);
        return (s0 ? t.sink_k : t.tail_k) + row * D;
    };
    // ---- every load that does not depend on q' first: this lane's key row
    //      (token tid / grp, for the logit of head tid % grp) and its channel's
    //      values over the chunk
    const int c = tid & (D - 1), half = tid >> 7;
    const int r_own = tid / grp, h_own = tid % grp;
    const bool has_pair = grp <= 4 && r_own < n;  // one (token, head) pair per lane when they fit
    u32x4 w[16];
    {
        const uint16_t *kr = krow_of(grp <= 4 ? r_own : 0);
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) w[cc] = *reinterpret_cast<const u32x4 *>(kr + 8 * cc);
    }
    uint16_t vraw[TCH];
#pragma unroll
    for (int r = 0; r < TCH; ++r) {
        bool s0;
        const size_t row = row_of(r, s0);
        vraw[r] = (s0 ? t.sink_v : t.tail_v)[row * D + c];
    }

    // the masked q' of the group: whole q' rows and the channel list load
    // together (no load waits for another), the list marks its channels in
    // LDS, and unmarked channels become 0
    constexpr int NQ = (GRP * D + 255) / 256;
    const int32_t *sel = sel_idx + ((size_t)b * hkv + g) * n_keep;
    const float *qrow = q_prime + ((size_t)b * hq + (size_t)g * grp) * D;
    float qv[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int e = tid + 256 * k;
        qv[k] = e < grp * D ? qrow[e] : 0.0f;
    }
    const int my_sel = tid < n_keep ? sel[tid] : -1;
    if (tid < D) keep_s[tid] = 0;
    __syncthreads();
    if (my_sel >= 0) keep_s[my_sel & (D - 1)] = 1;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int e = tid + 256 * k;
        if (e < grp * D) qm[e / D][e % D] = keep_s[e % D] ? qv[k] : 0.0f;
    }
    __syncthreads();
    // ---- logits of (token r, head h) pairs
    auto logit = [&](const u32x4 (&kw)[16], int h) {
        float acc = 0.0f;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float kv = __uint_as_float(e2 & 1 ? (kw[cc][e2 >> 1] & 0xFFFF0000u) : (kw[cc][e2 >> 1] << 16));
                acc = __builtin_fmaf(qm[h][8 * cc + e2], kv, acc);
            }
        return acc * sm_scale;
    };
    if (grp <= 4) {
        if (has_pair) x[h_own][r_own] = logit(w, h_own);
    } else {
        for (int e = tid; e < n * grp; e += 256) {
            const int r = e / grp, h = e % grp;
            const uint16_t *kr = krow_of(r);
            u32x4 kw[16];
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) kw[cc] = *reinterpret_cast<const u32x4 *>(kr + 8 * cc);
            x[h][r] = logit(kw, h);
        }
    }
    __syncthreads();
    // ---- per head (one wave each, lane = token): maximum, weights, their sum
    for (int h = wv; h < grp; h += 4) {
        const float xv = lane < n ? x[h][lane] : -__builtin_huge_valf();
        float m = xv;
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float p = lane < n ? __expf(xv - m) : 0.0f;
        float l = p;
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
        x[h][lane] = p;
        if (lane == 0) {
            m_s[h] = n > 0 ? m : -__builtin_huge_valf();
            l_s[h] = l;
        }
    }
    __syncthreads();
    // ---- o[h][c] = sum_r p[h][r] v[r][c] (p = 0 past the chunk's tokens): lane c,
    //      heads h = half, half + 2, ...
    constexpr int HH = (GRP + 1) / 2;  // heads per lane half
    float o[HH];
#pragma unroll
    for (int k = 0; k < HH; ++k) o[k] = 0.0f;
    if (GRP % 2 == 0 || half == 0) {
#pragma unroll
        for (int r = 0; r < TCH; ++r) {
            const float vv = bf(vraw[r]);
#pragma unroll
            for (int k = 0; k < HH; ++k) o[k] = __builtin_fmaf(x[half + 2 * k][r], vv, o[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < HH; ++k) {
        const int h = half + 2 * k;
        if (h < grp) {
            float *dst = part + (((size_t)b * hq + (size_t)g * grp + h) * N_TCH + chunk) * PART_FLOATS;
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

static_assert(N_TCH == TIER_PARTIALS, "tier partials per (sequence, query head)");

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

hipError_t launch_tier_decode(const dqk_tiers &t, const float *q_prime, const int32_t *sel_idx, int n_keep, int batch,
                              int hq, const int32_t *seq_lens, float sm_scale, float *tier_partials,
                              int32_t *int2_lens, hipStream_t s) {
    const dim3 grid(N_TCH, batch * t.num_kv_heads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, t, q_prime, sel_idx, n_keep, hq, seq_lens, sm_scale,
                           tier_partials, int2_lens);
        return hipGetLastError();
    };
    switch (hq / t.num_kv_heads) {  // 1 .. TD_MAXG (checked by the caller)
        case 1: return go(tier_decode_kernel<1>);
        case 2: return go(tier_decode_kernel<2>);
        case 3: return go(tier_decode_kernel<3>);
        case 4: return go(tier_decode_kernel<4>);
        case 5: return go(tier_decode_kernel<5>);
        case 6: return go(tier_decode_kernel<6>);
        case 7: return go(tier_decode_kernel<7>);
        case 8: return go(tier_decode_kernel<8>);
        case 9: return go(tier_decode_kernel<9>);
        case 10: return go(tier_decode_kernel<10>);
        case 11: return go(tier_decode_kernel<11>);
        case 12: return go(tier_decode_kernel<12>);
        case 13: return go(tier_decode_kernel<13>);
        case 14: return go(tier_decode_kernel<14>);
        case 15: return go(tier_decode_kernel<15>);
        default: return go(tier_decode_kernel<16>);
    }
}

}  // namespace dqk
