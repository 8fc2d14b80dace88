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
// Built with -ffp-contract=off: only the written fmas fuse.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int THREADS = 256;
constexpr int HALVES = THREADS / D;  // query-head interleave across the two lane halves

// Stage T_Q[g] (64 KB) and q of the group (bf16 -> fp32) into LDS; every
// load of the transform is issued before any is stored.
__device__ __forceinline__ void stage_inputs(const uint16_t *__restrict__ q, const float *__restrict__ t_q, int g,
                                             int b, int hq, int grp, float *t_lds, float *q_lds) {
    const int tid = threadIdx.x;
    const float4 *tsrc = reinterpret_cast<const float4 *>(t_q + (size_t)g * D * D);
    float4 *tdst = reinterpret_cast<float4 *>(t_lds);
    constexpr int PER = D * D / 4 / THREADS;  // 16 float4 per lane
    float4 stage[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) stage[k] = tsrc[tid + k * THREADS];
    const uint16_t *qg = q + ((size_t)b * hq + (size_t)g * grp) * D;
    for (int i = tid; i < grp * D; i += THREADS) q_lds[i] = bf2f(qg[i]);
#pragma unroll
    for (int k = 0; k < PER; ++k) tdst[tid + k * THREADS] = stage[k];
}

// Pooled energy of channel j (fma chain over ascending head), then the rank
// test and the ascending write of the kept channels.
__device__ __forceinline__ void select_tail(const float *qpl, int grp, int n_keep, const float *__restrict__ wsel,
                                            float *s_lds, unsigned long long *mask0, int32_t *__restrict__ dst) {
    const int tid = threadIdx.x, j = tid & (D - 1);
    if (tid < D) {
        const float w = wsel ? wsel[j] : 1.0f;  // x * 1 is x exactly
        float S = 0.0f;
        for (int h = 0; h < grp; ++h) {
            const float v = __fmul_rn(qpl[h * D + j], w);
            S = __builtin_fmaf(v, v, S);
        }
        s_lds[j] = S;
    }
    __syncthreads();
    bool keep = false;
    if (tid < D) {
        const float S = s_lds[j];
        int rank = 0;
#pragma unroll 4
        for (int jj = 0; jj < D; jj += 4) {
            const float4 o = *reinterpret_cast<const float4 *>(&s_lds[jj]);
            rank += (o.x > S) | ((o.x == S) & (jj < j));
            rank += (o.y > S) | ((o.y == S) & (jj + 1 < j));
            rank += (o.z > S) | ((o.z == S) & (jj + 2 < j));
            rank += (o.w > S) | ((o.w == S) & (jj + 3 < j));
        }
        keep = rank < n_keep;
    }
    // ascending output position = kept channels below j (lanes 0..63 are channels 0..63)
    const unsigned long long m = __ballot(keep);
    if (tid == 0) *mask0 = m;
    __syncthreads();
    if (keep) {
        const int lane = tid & 63;
        const unsigned long long below = lane ? (m & ((1ull << lane) - 1ull)) : 0ull;
        const int pos = __popcll(below) + (tid >= 64 ? __popcll(*mask0) : 0);
        if (pos < n_keep) dst[pos] = j;  // NaN inputs cannot overrun
    }
}

// Group size fixed at compile time: lane (half, j) runs the chains of heads
// half, half + 2, ..., four input channels per step (one broadcast LDS read of
// q per head, four reads of T_Q column j), ascending i within each chain.
template <int GRP>
__global__ __launch_bounds__(THREADS) void select_kernel_g(const uint16_t *__restrict__ q,
                                                           const float *__restrict__ t_q, int hq, int hkv,
                                                           int n_keep, const float *__restrict__ sel_scale,
                                                           float *__restrict__ q_prime,
                                                           int32_t *__restrict__ sel_idx) {
    constexpr int NH = GRP >= HALVES ? GRP / HALVES : 1;  // chains per lane
    __shared__ __attribute__((aligned(16))) float t_lds[D * D];
    __shared__ __attribute__((aligned(16))) float q_lds[GRP * D];
    __shared__ __attribute__((aligned(16))) float qp_lds[GRP * D];
    __shared__ __attribute__((aligned(16))) float s_lds[D];
    __shared__ unsigned long long mask0;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    stage_inputs(q, t_q, g, b, hq, GRP, t_lds, q_lds);
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
    select_tail(qp_lds, GRP, n_keep, sel_scale ? sel_scale + (size_t)g * D : nullptr, s_lds, &mask0,
                sel_idx + ((size_t)b * hkv + g) * n_keep);
}

// Any group size up to 64 (runtime loop bounds).
__global__ __launch_bounds__(THREADS) void select_kernel(const uint16_t *__restrict__ q, const float *__restrict__ t_q,
                                                         int hq, int hkv, int n_keep,
                                                         const float *__restrict__ sel_scale,
                                                         float *__restrict__ q_prime,
                                                         int32_t *__restrict__ sel_idx) {
    __shared__ __attribute__((aligned(16))) float t_lds[D * D];  // T_Q of this KV head (64 KB)
    extern __shared__ __attribute__((aligned(16))) float q_lds[];  // [grp][128] q (bf16 -> fp32), then [grp][128] q'
    __shared__ __attribute__((aligned(16))) float s_lds[D];
    __shared__ unsigned long long mask0;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int grp = hq / hkv;
    stage_inputs(q, t_q, g, b, hq, grp, t_lds, q_lds);
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
    select_tail(qpl, grp, n_keep, sel_scale ? sel_scale + (size_t)g * D : nullptr, s_lds, &mask0,
                sel_idx + ((size_t)b * hkv + g) * n_keep);
}

}  // namespace

hipError_t launch_select(const uint16_t *q, const float *t_q, const float *sel_scale, int batch, int hq, int hkv,
                         int n_keep, float *q_prime, int32_t *sel_idx, hipStream_t s) {
    const int grp = hq / hkv;
    dim3 grid(hkv, batch);
#define DQK_SELECT_G(G)                                                                                      \
    case G:                                                                                                   \
        hipLaunchKernelGGL(select_kernel_g<G>, grid, dim3(THREADS), 0, s, q, t_q, hq, hkv, n_keep, sel_scale, \
                           q_prime, sel_idx);                                                                 \
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
                       sel_idx);
    return hipGetLastError();
}

}  // namespace dqk
