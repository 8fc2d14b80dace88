// Decode attention over the paged INT2 cache for 4 query heads per KV head
// (GQA 32/8-style), on MFMA (Dual-QK paper: masked scores over the selected
// channels with the full 1/sqrt(d) scale, §3.2; channel 0 from its bf16
// copy, INT2 channel-major key rows and token-major values, §3.3; one
// softmax over the context, §3.4).
//
// Workgroup = 4 waves per (split, sequence x KV head); each wave streams its
// own 4-page blocks ("quads") with an online softmax, and the waves are
// combined in LDS at the end.  Per quad:
//
//  * Scores S^T = codes x q~ on v_mfma_f32_16x16x32_f16, block-diagonal over
//    the quad's 4 pages: the 16 MFMA columns are (page slot p, head h), the
//    32-deep k dimension is (page slot, 8 selected channels), so every
//    column is a real (page, head) pair.  q~ = q' * scale_j (fp16) per page
//    and channel; the zero points fold into one bias per (page, head).
//    Token tile m, row i holds token 8i + m, so lane i reads the 16-bit word
//    i of each selected 32-byte key row: the 8 tokens it needs for all
//    tiles.
//  * 2-bit codes enter MFMA as binary16 subnormals: one AND of a (possibly
//    shifted) packed word gives code * 2^(offset - 24) exactly for two
//    tokens at once; the power of two is undone per tile after the MFMA.
//  * Online softmax in the log2 domain on the score layout (lane = page/head
//    column, 32 tokens per lane), wave-uniform running max per head.
//  * Values: per page, O[(group q, head h)][channel] += (P*scale_q)[.][token]
//    x codes[token][channel] on MFMA (M = 4 groups x 4 heads, all rows
//    real); P is moved to the operand layout with ds_swizzle; the zero
//    points accumulate as sum_t P z_{t,q} with v_dot2_f32_f16.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GRP = 4;    // query heads per KV head handled here
constexpr int WAVES = 4;  // waves per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Token (or channel) m of a packed 16-bit word sits at bits [2m, 2m+1] of each
// half.  Tile m takes it from X << 4 (m = 0, 1), X (m = 2, 3, 4) or X >> 6
// (m = 5, 6, 7), which puts every field at bit offset 4, 6 or 8 of its half:
// the binary16 subnormal code * 2^(offset - 24).  Offsets below 4 are avoided
// because MFMA sums truncate at a fixed absolute level, which would bias the
// smallest subnormal products.
__device__ __forceinline__ constexpr int tile_offset(int m) {
    return m <= 1 ? 4 + 2 * m : m <= 4 ? 2 * m : 2 * m - 6;
}
// undo code * 2^(offset - 24)
__device__ __forceinline__ constexpr float tile_comp(int m) {
    return 16777216.0f / (float)(1u << tile_offset(m));
}

__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ half2v as_half2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

struct Packed {
    u32x4 L, X, R;  // X << 4, X, X >> 6
};

__device__ __forceinline__ Packed pack_shifts(const u32x4 &X) { return {X << 4, X, X >> 6}; }

template <int m>
__device__ __forceinline__ u32x4 tile_codes(const Packed &P) {
    constexpr uint32_t mask = 0x00030003u << tile_offset(m);
    return (m <= 1 ? P.L : m <= 4 ? P.X : P.R) & mask;
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

template <int PAT>
__device__ __forceinline__ uint32_t swz(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, PAT);
}

__device__ __forceinline__ float sel4(const float (&a)[4], int i) {
    return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
}
__device__ __forceinline__ int64_t sel4i(const int64_t (&a)[4], int i) {
    return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
}
__device__ __forceinline__ int sel4n(const int (&a)[4], int i) {
    return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
}

__global__ __launch_bounds__(256) void decode_g4_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                           const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                           const int32_t *__restrict__ page_table, int max_pages,
                                                           const int32_t *__restrict__ seq_lens, float sm_scale,
                                                           int nsplit, float *__restrict__ partials) {
    __shared__ __attribute__((aligned(16))) float qsel[GRP][D];               // C * q'_{h, jrow[jj]}
    __shared__ __attribute__((aligned(16))) _Float16 qt[2][WAVES][4][GRP][D];  // q~ hi/lo per wave [p][h][jj]
    __shared__ __attribute__((aligned(16))) _Float16 zero16[16];
    __shared__ float comb[WAVES][GRP][D + 2];

    const int split = blockIdx.x, bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    const int b = bg / hkv, g = bg - b * hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    const int per = (((npages + nsplit - 1) / nsplit) + 15) & ~15;
    const int P0 = min(npages, split * per), P1 = min(npages, P0 + per);

    const float C = sm_scale * LOG2E;
    const int32_t *sel = sel_idx + ((size_t)b * hkv + g) * n_keep;
    const int has0 = sel[0] == 0;  // the list is ascending
    const int R = n_keep - has0;   // selected INT2 channels
    const int KS = (R + 7) >> 3;
    const float *qp = q_prime + ((size_t)b * hq + (size_t)g * GRP) * D;

    for (int i = tid; i < GRP * D; i += 256) {
        const int h = i >> 7, jj = i & (D - 1);
        qsel[h][jj] = jj < R ? qp[h * D + sel[jj + has0]] * C : 0.0f;
    }
    if (tid < 16) zero16[tid] = (_Float16)0.0f;
    __syncthreads();

    // score-layout lane: column n = (page slot pc, head hc)
    const int pc = n >> 2, hc = n & 3;
    const float q0c = has0 ? qp[hc * D] * C : 0.0f;
    // value-operand lane: row n = (group qv, head hv)
    const int qv = n >> 2, hv = n & 3;
    // staging lane: page slot G, channels 8n .. 8n+7 of the compacted list
    int chan[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int jj = 8 * n + e;
        chan[e] = jj < R ? sel[jj + has0] : 0;
    }

    float m_run[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) m_run[h] = -__builtin_huge_valf();
    float l_lane = 0.0f, z_lane = 0.0f;
    f32x4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = {0.f, 0.f, 0.f, 0.f};

    const int nq = (P1 - P0 + 3) >> 2;
    const int32_t *ptab = page_table + (size_t)b * max_pages;
    for (int u = w; u < nq; u += WAVES) {
        const int lp0 = P0 + 4 * u;
        int64_t pgi[4];  // (physical page * hkv + g), always a valid page
        int nv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int lp = lp0 + p;
            const bool ok = lp < P1;
            pgi[p] = (int64_t)ptab[ok ? lp : lp0] * hkv + g;
            nv[p] = ok ? min(PG, L - lp * PG) : 0;
        }

        // ---- stage q~ (fp16) for page slot G and channels 8n..8n+7; bias partials
        float bpart[GRP] = {0.f, 0.f, 0.f, 0.f};
        if (n < KS) {
            const uint16_t *km = c.k_meta + sel4i(pgi, G) * (D * 2);
            const bool pv = sel4n(nv, G) > 0;
            float s[8], z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sz = pv ? *reinterpret_cast<const uint32_t *>(km + chan[e] * 2) : 0u;
                const bool live = 8 * n + e < R;
                s[e] = live ? h2f((uint16_t)(sz & 0xFFFFu)) : 0.0f;
                z[e] = live ? h2f((uint16_t)(sz >> 16)) : 0.0f;
            }
#pragma unroll
            for (int h = 0; h < GRP; ++h) {
                const float4 qa = *reinterpret_cast<const float4 *>(&qsel[h][8 * n]);
                const float4 qb = *reinterpret_cast<const float4 *>(&qsel[h][8 * n + 4]);
                const float qv8[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
                half8 thi, tlo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = qv8[e] * s[e];
                    thi[e] = (_Float16)t;
                    tlo[e] = (_Float16)(t - (float)thi[e]);
                    bpart[h] = __builtin_fmaf(qv8[e], z[e], bpart[h]);
                }
                *reinterpret_cast<half8 *>(&qt[0][w][G][h][8 * n]) = thi;
                *reinterpret_cast<half8 *>(&qt[1][w][G][h][8 * n]) = tlo;
            }
        }
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
            bpart[h] += __shfl_xor(bpart[h], 1);
            bpart[h] += __shfl_xor(bpart[h], 2);
            bpart[h] += __shfl_xor(bpart[h], 4);
            bpart[h] += __shfl_xor(bpart[h], 8);
        }
        // lane (row p, n') offers the bias of head n' & 3; column (pc, hc) reads lane 16 pc + hc
        const float bias = __shfl(sel4(bpart, n & 3), 16 * pc + hc);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- scores
        f32x4 S[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = {0.f, 0.f, 0.f, 0.f};
        const uint8_t *krow = c.k_codes + sel4i(pgi, G) * (D * ROW_BYTES) + 2 * n;
        const _Float16 *bhi = pc == G ? &qt[0][w][pc][hc][0] : &zero16[0];
        const _Float16 *blo = pc == G ? &qt[1][w][pc][hc][0] : &zero16[0];
        const int bstep = pc == G ? 8 : 0;
        for (int kk = 0; kk < KS; ++kk) {
            const half8 Bq = *reinterpret_cast<const half8 *>(bhi + bstep * kk);
            const half8 Bl = *reinterpret_cast<const half8 *>(blo + bstep * kk);
            u32x4 X;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int j0 = 8 * kk + 2 * e2;
                const int ca = j0 < R ? sel[j0 + has0] : 0;
                const int cb = j0 + 1 < R ? sel[j0 + 1 + has0] : 0;
                X[e2] = ld_u16(krow + ca * ROW_BYTES) | (ld_u16(krow + cb * ROW_BYTES) << 16);
            }
            const Packed XP = pack_shifts(X);
            S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<0>(XP)), Bq, S[0], 0, 0, 0);
            S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<0>(XP)), Bl, S[0], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<1>(XP)), Bq, S[1], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<1>(XP)), Bl, S[1], 0, 0, 0);
            S[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<2>(XP)), Bq, S[2], 0, 0, 0);
            S[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<2>(XP)), Bl, S[2], 0, 0, 0);
            S[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<3>(XP)), Bq, S[3], 0, 0, 0);
            S[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<3>(XP)), Bl, S[3], 0, 0, 0);
            S[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<4>(XP)), Bq, S[4], 0, 0, 0);
            S[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<4>(XP)), Bl, S[4], 0, 0, 0);
            S[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<5>(XP)), Bq, S[5], 0, 0, 0);
            S[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<5>(XP)), Bl, S[5], 0, 0, 0);
            S[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<6>(XP)), Bq, S[6], 0, 0, 0);
            S[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<6>(XP)), Bl, S[6], 0, 0, 0);
            S[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<7>(XP)), Bq, S[7], 0, 0, 0);
            S[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<7>(XP)), Bl, S[7], 0, 0, 0);
        }

        // ---- logits (log2 domain) for tokens 32G + 8r + m of page slot pc, head hc
        const int nvl = sel4n(nv, pc);
        float x[8][4];
        {
            uint32_t k0w[16];
            if (has0) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(c.k_ch0 + sel4i(pgi, pc) * PG + 32 * G);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const u32x4 t4 = src[v4];
                    k0w[4 * v4 + 0] = t4[0];
                    k0w[4 * v4 + 1] = t4[1];
                    k0w[4 * v4 + 2] = t4[2];
                    k0w[4 * v4 + 3] = t4[3];
                }
            }
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tl = 8 * r + m;  // token within the lane's 32
                    float v = __builtin_fmaf(S[m][r], tile_comp(m), bias);
                    if (has0) {
                        const uint32_t wd = k0w[tl >> 1];
                        const float k0 = __uint_as_float((tl & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                        v = __builtin_fmaf(q0c, k0, v);
                    }
                    x[m][r] = 32 * G + tl < nvl ? v : -__builtin_huge_valf();
                }
        }
        float xm = x[0][0];
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) xm = fmaxf(xm, x[m][r]);
        xm = fmaxf(xm, __shfl_xor(xm, 16));
        xm = fmaxf(xm, __shfl_xor(xm, 32));
        xm = fmaxf(xm, __shfl_xor(xm, 4));
        xm = fmaxf(xm, __shfl_xor(xm, 8));
        float alpha[GRP];
        bool changed = false;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
            const float mq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xm), h));  // lane h: column (0, h)
            const float mn = fmaxf(m_run[h], mq);
            alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - mn);
            changed |= mn != m_run[h];
            m_run[h] = mn;
        }
        if (changed) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[t][r] *= alpha[r];
            z_lane *= sel4(alpha, hv);
            l_lane *= sel4(alpha, hc);
        }
        const float mh = sel4(m_run, hc);
        // probabilities, packed as fp16 pairs per value k-step: Pk[kv][e2] = (P[2e2][kv], P[2e2+1][kv])
        uint32_t Pk[4][4];
        {
            float ls = 0.0f;
#pragma unroll
            for (int kv = 0; kv < 4; ++kv)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float pa = __builtin_amdgcn_exp2f(x[2 * e2][kv] - mh);
                    const float pb = __builtin_amdgcn_exp2f(x[2 * e2 + 1][kv] - mh);
                    ls += pa + pb;
                    half2v hp;
                    hp[0] = (_Float16)pa;
                    hp[1] = (_Float16)pb;
                    Pk[kv][e2] = as_u32(hp);
                }
            l_lane += ls;
        }

        // ---- values, page by page
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (nv[p] == 0) continue;
            const uint8_t *vrow = c.v_codes + pgi[p] * (PG * ROW_BYTES) + 2 * n;
            const uint16_t *vm = c.v_meta + pgi[p] * (2 * VGROUPS * PG);
            const bool partial = nv[p] < PG;
#pragma unroll
            for (int kv = 0; kv < 4; ++kv) {
                const int tok0 = 32 * G + 8 * kv;
                // P of (page p, head hv) for tokens tok0 .. tok0+7, from lane 16G + 4p + hv
                uint32_t Pp[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    uint32_t v = Pk[kv][e2];
                    Pp[e2] = p == 0   ? swz<0x13 | (0 << 5)>(v)
                             : p == 1 ? swz<0x13 | (4 << 5)>(v)
                             : p == 2 ? swz<0x13 | (8 << 5)>(v)
                                      : swz<0x13 | (12 << 5)>(v);
                }
                u32x4 sp = *reinterpret_cast<const u32x4 *>(vm + (0 * VGROUPS + qv) * PG + tok0);
                u32x4 zp = *reinterpret_cast<const u32x4 *>(vm + (1 * VGROUPS + qv) * PG + tok0);
                if (partial) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const uint32_t keep = (tok0 + 2 * e2 < nv[p] ? 0x0000FFFFu : 0u) |
                                              (tok0 + 2 * e2 + 1 < nv[p] ? 0xFFFF0000u : 0u);
                        sp[e2] &= keep;
                        zp[e2] &= keep;
                        Pp[e2] &= keep;
                    }
                }
                u32x4 A;
                const half2v c15 = {(_Float16)1.5f, (_Float16)1.5f};
                const half2v m15 = {(_Float16)-1.5f, (_Float16)-1.5f};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const half2v a2 = as_half2(Pp[e2]) * as_half2(sp[e2]);
                    A[e2] = as_u32(a2);
                    // centred codes: v = (c - 1.5) s + (z + 1.5 s)
                    const half2v zc = __builtin_elementwise_fma(as_half2(sp[e2]), c15, as_half2(zp[e2]));
                    z_lane = __builtin_amdgcn_fdot2(as_half2(Pp[e2]), zc, z_lane, false);
                    z_lane = __builtin_amdgcn_fdot2(a2, m15, z_lane, false);
                }
                const half8 Ah = as_half8(A);
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    X[e2] = ld_u16(vrow + (tok0 + 2 * e2) * ROW_BYTES) |
                            (ld_u16(vrow + (tok0 + 2 * e2 + 1) * ROW_BYTES) << 16);
                const Packed XP = pack_shifts(X);
                O[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<0>(XP)), O[0], 0, 0, 0);
                O[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<1>(XP)), O[1], 0, 0, 0);
                O[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<2>(XP)), O[2], 0, 0, 0);
                O[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<3>(XP)), O[3], 0, 0, 0);
                O[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<4>(XP)), O[4], 0, 0, 0);
                O[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<5>(XP)), O[5], 0, 0, 0);
                O[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<6>(XP)), O[6], 0, 0, 0);
                O[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(tile_codes<7>(XP)), O[7], 0, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- per-wave totals
    l_lane += __shfl_xor(l_lane, 4);
    l_lane += __shfl_xor(l_lane, 8);
    l_lane += __shfl_xor(l_lane, 16);
    l_lane += __shfl_xor(l_lane, 32);   // lanes with hc = h hold l of head h
    z_lane += __shfl_xor(z_lane, 16);
    z_lane += __shfl_xor(z_lane, 32);   // lane (., 4q + h) holds Z_{q,h}
    float zq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) zq[r] = __shfl(z_lane, 16 * G + 4 * G + r);  // Z_{q = G, h = r}
    if ((n >> 2) == G) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) comb[w][r][8 * n + t] = __builtin_fmaf(O[t][r], tile_comp(t), zq[r]);
    }
    if (lane < GRP) {
        comb[w][lane][D] = sel4(m_run, lane);
        comb[w][lane][D + 1] = l_lane;
    }
    __syncthreads();

    // ---- combine the 4 waves and write the split partial (m in natural-log units)
    for (int i = tid; i < GRP * D; i += 256) {
        const int h = i >> 7, ch = i & (D - 1);
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) M = fmaxf(M, comb[ww][h][D]);
        float acc = 0.0f, lsum = 0.0f;
        if (M > -__builtin_huge_valf()) {
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) {
                const float mw = comb[ww][h][D];
                if (mw > -__builtin_huge_valf()) {
                    const float f = __builtin_amdgcn_exp2f(mw - M);
                    acc = __builtin_fmaf(comb[ww][h][ch], f, acc);
                    lsum = __builtin_fmaf(comb[ww][h][D + 1], f, lsum);
                }
            }
        }
        float *dst = partials + (((size_t)b * hq + (size_t)g * GRP + h) * nsplit + split) * PART_FLOATS;
        dst[ch] = acc;
        if (ch == 0) {
            dst[D] = M * LN2;
            dst[D + 1] = lsum;
        }
    }
}

}  // namespace

bool use_mfma_decode(int hq, int hkv) { return hkv > 0 && hq == GRP * hkv; }

int decode_splits_mfma(int batch, int hkv, int max_pages) {
    // about two workgroups of 4 waves per CU on 256 CUs, at least 16 pages per workgroup
    const int units = batch * hkv;
    int s = (512 + units - 1) / units;
    const int cap = (max_pages + 15) / 16;
    if (s > cap) s = cap;
    return s < 1 ? 1 : s;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_g4_kernel, grid, dim3(256), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    return hipGetLastError();
}

}  // namespace dqk
