// Query transform q' = q T_Q and dynamic query-channel selection (Dual-QK
// paper, §3.2 Eq. 4: pooled energy over the query heads of a KV head; the
// kept channels form one mask per KV head, §3.2-§3.3).
//
// One workgroup of 256 lanes per (KV head g, sequence b); lane (half, j)
// owns output channel j of every other query head.  Each q'_{h,j} is an fp32
// fma chain over ascending input channel (the heads of the group run as
// independent chains for ILP; each chain's order is unchanged).  S_j accumulates e^2 over ascending head by fma,
// e = q'_{h,j} or, with per-channel selection scales w (§3.3 diagonal
// refinement, App. C.2: selection in the base coordinates q A_0 = q' D^-1,
// w_j = 1 / delta_j), e = fp32(q'_{h,j} w_j); q' itself is left unscaled.
// Channel j is kept iff fewer than n_keep channels beat it (larger S, or
// equal S at a lower index); kept channels are written in ascending order.
//
// Bucket-relative RoPE (§3.4, App. C.4): block y = (sequence b, bucket k)
// turns q by bucket k's anchor table while it stages it (fp32, each product
// and sum rounded), then runs the same chains and rank test; its q' and mask
// go to row (b, k) of [batch][n_buckets][..] outputs.
// Built with -ffp-contract=off: only the written fmas fuse.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int THREADS = 256;
constexpr int HALVES = THREADS / D;  // query-head interleave across the two lane halves

// Stage T_Q[g] (64 KB) and q of the group (bf16 -> fp32, turned by the
// bucket's table rcs / rsn when they are non-null) into LDS; every load of
// the transform is issued before any is stored.
__device__ __forceinline__ void stage_inputs(const uint16_t *__restrict__ q, const float *__restrict__ t_q, int g,
                                             int b, int hq, int grp, float *t_lds, float *q_lds,
                                             const float *__restrict__ rcs, const float *__restrict__ rsn) {
    const int tid = threadIdx.x;
    const float4 *tsrc = reinterpret_cast<const float4 *>(t_q + (size_t)g * D * D);
    float4 *tdst = reinterpret_cast<float4 *>(t_lds);
    constexpr int PER = D * D / 4 / THREADS;  // 16 float4 per lane
    float4 stage[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) stage[k] = tsrc[tid + k * THREADS];
    const uint16_t *qg = q + ((size_t)b * hq + (size_t)g * grp) * D;
    if (rcs) {
        for (int i = tid; i < grp * D; i += THREADS) {
            const int j = i & (D - 1), jp = j & (D / 2 - 1);
            q_lds[i] = rope_turn(bf2f(qg[i]), bf2f(qg[i ^ (D / 2)]), rcs[jp], rsn[jp], j < D / 2);
        }
    } else {
        for (int i = tid; i < grp * D; i += THREADS) q_lds[i] = bf2f(qg[i]);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) tdst[tid + k * THREADS] = stage[k];
}

// Pooled energies of channels lane and lane + 64 (fma chains over ascending
// head) and the mask by top_k_wave, all in wave 0; the kept channels are
// written in ascending order.
__device__ __forceinline__ void select_tail(const float *qpl, int grp, int n_keep, const float *__restrict__ wsel,
                                            int32_t *__restrict__ dst) {
    const int tid = threadIdx.x;
    if (tid >= 64) return;
    const float wa = wsel ? wsel[tid] : 1.0f, wb = wsel ? wsel[tid + 64] : 1.0f;  // x * 1 is x exactly
    float sa = 0.0f, sb = 0.0f;
    for (int h = 0; h < grp; ++h) {
        const float va = __fmul_rn(qpl[h * D + tid], wa), vb = __fmul_rn(qpl[h * D + tid + 64], wb);
        sa = __builtin_fmaf(va, va, sa);
        sb = __builtin_fmaf(vb, vb, sb);
    }
    const KeptPair kp = top_k_wave(sa, sb, n_keep);
    if (kp.ka && kp.pa < n_keep) dst[kp.pa] = tid;
    if (kp.kb && kp.pb < n_keep) dst[kp.pb] = tid + 64;
}

// Group size fixed at compile time: lane (half, j) runs the chains of heads
// half, half + 2, ..., four input channels per step (one broadcast LDS read of
// q per head, four reads of T_Q column j), ascending i within each chain.
template <int GRP>
__global__ __launch_bounds__(THREADS) void select_kernel_g(const uint16_t *__restrict__ q,
                                                           const float *__restrict__ t_q, int hq, int hkv,
                                                           int n_keep, const float *__restrict__ sel_scale,
                                                           float *__restrict__ q_prime,
                                                           int32_t *__restrict__ sel_idx,
                                                           const float *__restrict__ rope_cos,
                                                           const float *__restrict__ rope_sin, int nbk) {
    constexpr int NH = GRP >= HALVES ? GRP / HALVES : 1;  // chains per lane
    __shared__ __attribute__((aligned(16))) float t_lds[D * D];
    __shared__ __attribute__((aligned(16))) float q_lds[GRP * D];
    __shared__ __attribute__((aligned(16))) float qp_lds[GRP * D];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;  // b: row (sequence, bucket) of the outputs
    const int sq = b / nbk, bk = b - sq * nbk;
    stage_inputs(q, t_q, g, sq, hq, GRP, t_lds, q_lds, rope_cos ? rope_cos + bk * (D / 2) : nullptr,
                 rope_sin ? rope_sin + bk * (D / 2) : nullptr);
    __syncthreads();
    const int j = tid & (D - 1), half = tid >> 7;
    if (GRP >= HALVES || half == 0) {
        float acc[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) acc[k] = 0.0f;
#pragma unroll 2
        for (int i = 0; i < D; i += 4) {
            const float t0 = t_lds[(i + 0) * D + j], t1 = t_lds[(i + 1) * D + j];
            const float t2 = t_lds[(i + 2) * D + j], t3 = t_lds[(i + 3) * D + j];
#pragma unroll
            for (int k = 0; k < NH; ++k) {
                const float4 qv = *reinterpret_cast<const float4 *>(&q_lds[(half + HALVES * k) * D + i]);
                float a = acc[k];
                a = __builtin_fmaf(qv.x, t0, a);
                a = __builtin_fmaf(qv.y, t1, a);
                a = __builtin_fmaf(qv.z, t2, a);
                a = __builtin_fmaf(qv.w, t3, a);
                acc[k] = a;
            }
        }
        float *qp = q_prime + ((size_t)b * hq + (size_t)g * GRP) * D + j;
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            const int h = half + HALVES * k;
            qp[(size_t)h * D] = acc[k];
            qp_lds[h * D + j] = acc[k];
        }
    }
    __syncthreads();
    select_tail(qp_lds, GRP, n_keep, sel_scale ? sel_scale + (size_t)g * D : nullptr,
                sel_idx + ((size_t)b * hkv + g) * n_keep);
}

// Any group size up to 64 (runtime loop bounds).
__global__ __launch_bounds__(THREADS) void select_kernel(const uint16_t *__restrict__ q, const float *__restrict__ t_q,
                                                         int hq, int hkv, int n_keep,
                                                         const float *__restrict__ sel_scale,
                                                         float *__restrict__ q_prime,
                                                         int32_t *__restrict__ sel_idx,
                                                         const float *__restrict__ rope_cos,
                                                         const float *__restrict__ rope_sin, int nbk) {
    __shared__ __attribute__((aligned(16))) float t_lds[D * D];  // T_Q of this KV head (64 KB)
    extern __shared__ __attribute__((aligned(16))) float q_lds[];  // [grp][128] q (bf16 -> fp32), then [grp][128] q'
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;  // b: row (sequence, bucket) of the outputs
    const int grp = hq / hkv;
    const int sq = b / nbk, bk = b - sq * nbk;
    stage_inputs(q, t_q, g, sq, hq, grp, t_lds, q_lds, rope_cos ? rope_cos + bk * (D / 2) : nullptr,
                 rope_sin ? rope_sin + bk * (D / 2) : nullptr);
    __syncthreads();

    float *qpl = q_lds + grp * D;  // q' [grp][128]
    const int j = tid & (D - 1), half = tid >> 7;
    float *qp = q_prime + ((size_t)b * hq + (size_t)g * grp) * D + j;
    for (int h = half; h < grp; h += HALVES) {
        float acc = 0.0f;
#pragma unroll 8
        for (int i = 0; i < D; ++i) acc = __builtin_fmaf(q_lds[h * D + i], t_lds[i * D + j], acc);
        qp[(size_t)h * D] = acc;
        qpl[h * D + j] = acc;
    }
    __syncthreads();
    select_tail(qpl, grp, n_keep, sel_scale ? sel_scale + (size_t)g * D : nullptr,
                sel_idx + ((size_t)b * hkv + g) * n_keep);
}

// Selection of KB = 32 / GRP buckets per workgroup (bucket-relative RoPE):
// T_Q[g] is staged once for the workgroup's buckets kb0 .. kb0 + KB - 1 of
// sequence b, and the 32 (bucket, head) rows of q, each turned by its
// bucket's table, sit in LDS.  Lane (wave w, half r, quad c) runs the sixteen
// chains of rows 8w + 4r .. 8w + 4r + 3 and output channels 4c .. 4c + 3: per
// four input channels one 16-byte read of T_Q per input channel and one
// 16-byte read of q per row serve sixteen fmas.  Each chain is the fma chain
// over ascending input channel of select_kernel.  The mask of a bucket is
// then found by one wave (pooled energy by fma over ascending head, then
// top_k_wave).
template <int GRP>
__global__ __launch_bounds__(THREADS) void select_rope_kernel(const uint16_t *__restrict__ q,
                                                              const float *__restrict__ t_q, int hq, int hkv,
                                                              int n_keep, int nbk, const float *__restrict__ rope_cos,
                                                              const float *__restrict__ rope_sin,
                                                              float *__restrict__ q_prime,
                                                              int32_t *__restrict__ sel_idx) {
    constexpr int RW = 32, KB = RW / GRP;
    __shared__ __attribute__((aligned(16))) float t_lds[D * D];
    __shared__ __attribute__((aligned(16))) float q_lds[RW * D];  // row (bucket kl, head h) = kl GRP + h
    const int g = blockIdx.x, b = blockIdx.y, kb0 = blockIdx.z * KB, tid = threadIdx.x;
    const int nbl = min(KB, nbk - kb0);
    {
        const float4 *tsrc = reinterpret_cast<const float4 *>(t_q + (size_t)g * D * D);
        constexpr int PER = D * D / 4 / THREADS;
        float4 stage[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) stage[k] = tsrc[tid + k * THREADS];
        // element e = (head h, channel j) of the group's q and its partner
        // j ^ 64, then every bucket's table entries: all loads issued before use
        const uint16_t *qg = q + ((size_t)b * hq + (size_t)g * GRP) * D;
        constexpr int NE = (GRP * D + THREADS - 1) / THREADS;
        float x[NE], xp[NE], cv[KB][NE], sv[KB][NE];
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const int e = tid + k * THREADS;
            const bool ok = e < GRP * D;
            x[k] = ok ? bf2f(qg[e]) : 0.0f;
            xp[k] = ok ? bf2f(qg[e ^ (D / 2)]) : 0.0f;
        }
#pragma unroll
        for (int kl = 0; kl < KB; ++kl)
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                const int jp = (tid + k * THREADS) & (D / 2 - 1);
                const bool ok = kl < nbl;
                cv[kl][k] = ok ? rope_cos[(size_t)(kb0 + kl) * (D / 2) + jp] : 0.0f;
                sv[kl][k] = ok ? rope_sin[(size_t)(kb0 + kl) * (D / 2) + jp] : 0.0f;
            }
#pragma unroll
        for (int kl = 0; kl < KB; ++kl)
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                const int e = tid + k * THREADS, j = e & (D - 1);
                if (e < GRP * D)  // row kl GRP + h holds bucket kl's turned head h (zero past the last bucket)
                    q_lds[kl * GRP * D + e] = rope_turn(x[k], xp[k], cv[kl][k], sv[kl][k], j < D / 2);
            }
        float4 *tdst = reinterpret_cast<float4 *>(t_lds);
#pragma unroll
        for (int k = 0; k < PER; ++k) tdst[tid + k * THREADS] = stage[k];
    }
    __syncthreads();
    const int lane = tid & 63, w = tid >> 6;
    const int c4 = 4 * (lane & 31), r0 = 8 * w + 4 * (lane >> 5);
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
    // operands of four input channels: T_Q rows i .. i + 3 (this lane's four
    // columns) and q of the lane's four rows; two sets, so that the reads of
    // the next four channels are in flight while the fmas of these run
    float4 tv[2][4], qv[2][4];
    auto load = [&](int i, int st) {
#pragma unroll
        for (int k = 0; k < 4; ++k) tv[st][k] = *reinterpret_cast<const float4 *>(&t_lds[(i + k) * D + c4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) qv[st][r] = *reinterpret_cast<const float4 *>(&q_lds[(r0 + r) * D + i]);
    };
    auto step = [&](int st) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 x = qv[st][r];
            float a0 = acc[r][0], a1 = acc[r][1], a2 = acc[r][2], a3 = acc[r][3];
            a0 = __builtin_fmaf(x.x, tv[st][0].x, a0);
            a1 = __builtin_fmaf(x.x, tv[st][0].y, a1);
            a2 = __builtin_fmaf(x.x, tv[st][0].z, a2);
            a3 = __builtin_fmaf(x.x, tv[st][0].w, a3);
            a0 = __builtin_fmaf(x.y, tv[st][1].x, a0);
            a1 = __builtin_fmaf(x.y, tv[st][1].y, a1);
            a2 = __builtin_fmaf(x.y, tv[st][1].z, a2);
            a3 = __builtin_fmaf(x.y, tv[st][1].w, a3);
            a0 = __builtin_fmaf(x.z, tv[st][2].x, a0);
            a1 = __builtin_fmaf(x.z, tv[st][2].y, a1);
            a2 = __builtin_fmaf(x.z, tv[st][2].z, a2);
            a3 = __builtin_fmaf(x.z, tv[st][2].w, a3);
            a0 = __builtin_fmaf(x.w, tv[st][3].x, a0);
            a1 = __builtin_fmaf(x.w, tv[st][3].y, a1);
            a2 = __builtin_fmaf(x.w, tv[st][3].z, a2);
            a3 = __builtin_fmaf(x.w, tv[st][3].w, a3);
            acc[r][0] = a0;
            acc[r][1] = a1;
            acc[r][2] = a2;
            acc[r][3] = a3;
        }
    };
    load(0, 0);
#pragma unroll
    for (int i = 0; i < D; i += 8) {
        load(i + 4, 1);
        step(0);
        load((i + 8) & (D - 1), 0);  // the last pass rereads channels 0..3, unused
        step(1);
    }
    __syncthreads();  // every chain has read the turned q: q' replaces it
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = r0 + r, kl = row / GRP, h = row - kl * GRP;
        const float4 v = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
        *reinterpret_cast<float4 *>(&q_lds[row * D + c4]) = v;
        if (kl < nbl)
            *reinterpret_cast<float4 *>(
                &q_prime[(((size_t)b * nbk + kb0 + kl) * hq + (size_t)g * GRP + h) * D + c4]) = v;
    }
    __syncthreads();
    // wave w selects buckets w, w + 4, ..; lane holds channels lane and lane + 64
    for (int kl = w; kl < nbl; kl += THREADS / 64) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
            const float va = q_lds[(kl * GRP + h) * D + lane], vb = q_lds[(kl * GRP + h) * D + lane + 64];
            sa = __builtin_fmaf(va, va, sa);
            sb = __builtin_fmaf(vb, vb, sb);
        }
        const KeptPair kp = top_k_wave(sa, sb, n_keep);
        int32_t *dst = sel_idx + (((size_t)b * nbk + kb0 + kl) * hkv + g) * n_keep;
        if (kp.ka && kp.pa < n_keep) dst[kp.pa] = lane;
        if (kp.kb && kp.pb < n_keep) dst[kp.pb] = lane + 64;
    }
}

}  // namespace

hipError_t launch_select(const uint16_t *q, const float *t_q, const float *sel_scale, int batch, int hq, int hkv,
                         int n_keep, float *q_prime, int32_t *sel_idx, hipStream_t s, const float *rope_cos,
                         const float *rope_sin, int n_buckets) {
    const int grp = hq / hkv;
    if (rope_cos && !sel_scale) {  // buckets: 32 / grp of them per workgroup
#define DQK_SELECT_ROPE(G)                                                                                      \
    case G: {                                                                                                   \
        dim3 grid_r(hkv, batch, (n_buckets + 32 / G - 1) / (32 / G));                                           \
        hipLaunchKernelGGL(select_rope_kernel<G>, grid_r, dim3(THREADS), 0, s, q, t_q, hq, hkv, n_keep,         \
                           n_buckets, rope_cos, rope_sin, q_prime, sel_idx);                                    \
        return hipGetLastError();                                                                               \
    }
        switch (grp) {
            DQK_SELECT_ROPE(1)
            DQK_SELECT_ROPE(2)
            DQK_SELECT_ROPE(4)
            DQK_SELECT_ROPE(8)
            DQK_SELECT_ROPE(16)
            default: break;
        }
#undef DQK_SELECT_ROPE
    }
    dim3 grid(hkv, batch * n_buckets);
#define DQK_SELECT_G(G)                                                                                      \
    case G:                                                                                                   \
        hipLaunchKernelGGL(select_kernel_g<G>, grid, dim3(THREADS), 0, s, q, t_q, hq, hkv, n_keep, sel_scale, \
                           q_prime, sel_idx, rope_cos, rope_sin, n_buckets);                                  \
        return hipGetLastError();
    switch (grp) {
        DQK_SELECT_G(1)
        DQK_SELECT_G(2)
        DQK_SELECT_G(4)
        DQK_SELECT_G(8)
        DQK_SELECT_G(16)
        DQK_SELECT_G(32)
        default: break;
    }
#undef DQK_SELECT_G
    const size_t lds = 2 * (size_t)grp * D * sizeof(float);
    hipLaunchKernelGGL(select_kernel, grid, dim3(THREADS), lds, s, q, t_q, hq, hkv, n_keep, sel_scale, q_prime,
                       sel_idx, rope_cos, rope_sin, n_buckets);
    return hipGetLastError();
}

}  // namespace dqk
