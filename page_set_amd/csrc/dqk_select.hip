// Query transform q' = q T_Q and dynamic query-channel selection (Dual-QK
// paper, §3.2 Eq. 4: pooled energy over the query heads of a KV head; the
// kept channels form one mask per KV head, §3.2-§3.3).
//
// One workgroup of 128 lanes per (KV head g, sequence b); lane j owns output
// channel j.  Each q'_{h,j} is an fp32 fma chain over ascending input channel
// (the heads of the group run as independent chains for ILP; each chain's
// order is unchanged).  S_j accumulates q'^2 over ascending head by fma.
// Channel j is kept iff fewer than n_keep channels beat it (larger S, or
// equal S at a lower index); kept channels are written in ascending order.
// Built with -ffp-contract=off: only the written fmas fuse.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int HCHUNK = 8;  // query heads per register chunk

__global__ __launch_bounds__(128) void select_kernel(const uint16_t *__restrict__ q, const float *__restrict__ t_q,
                                                     int hq, int hkv, int n_keep, float *__restrict__ q_prime,
                                                     int32_t *__restrict__ sel_idx) {
    extern __shared__ float q_lds[];  // [grp][128] bf16 -> fp32 (exact)
    __shared__ float s_lds[D];
    __shared__ int keep_lds[D];
    const int g = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
    const int grp = hq / hkv;
    const uint16_t *qg = q + ((size_t)b * hq + (size_t)g * grp) * D;
    for (int i = j; i < grp * D; i += D) q_lds[i] = bf2f(qg[i]);
    __syncthreads();

    const float *T = t_q + (size_t)g * D * D + j;
    float *qp = q_prime + ((size_t)b * hq + (size_t)g * grp) * D + j;
    float S = 0.0f;
    for (int h0 = 0; h0 < grp; h0 += HCHUNK) {
        const int nh = grp - h0 < HCHUNK ? grp - h0 : HCHUNK;
        float acc[HCHUNK];
#pragma unroll
        for (int k = 0; k < HCHUNK; ++k) acc[k] = 0.0f;
        for (int i = 0; i < D; ++i) {
            const float t = T[(size_t)i * D];
#pragma unroll
            for (int k = 0; k < HCHUNK; ++k)
                if (k < nh) acc[k] = __builtin_fmaf(q_lds[(h0 + k) * D + i], t, acc[k]);
        }
#pragma unroll
        for (int k = 0; k < HCHUNK; ++k)
            if (k < nh) {
                qp[(size_t)(h0 + k) * D] = acc[k];
                S = __builtin_fmaf(acc[k], acc[k], S);
            }
    }
    s_lds[j] = S;
    __syncthreads();
    int rank = 0;
    for (int jj = 0; jj < D; ++jj) {
        const float o = s_lds[jj];
        rank += (o > S) | ((o == S) & (jj < j));
    }
    const int keep = rank < n_keep;
    keep_lds[j] = keep;
    __syncthreads();
    if (keep) {
        int pos = 0;
        for (int jj = 0; jj < j; ++jj) pos += keep_lds[jj];
        if (pos < n_keep) sel_idx[((size_t)b * hkv + g) * n_keep + pos] = j;  // NaN inputs cannot overrun
    }
}

}  // namespace

hipError_t launch_select(const uint16_t *q, const float *t_q, int batch, int hq, int hkv, int n_keep, float *q_prime,
                         int32_t *sel_idx, hipStream_t s) {
    const int grp = hq / hkv;
    dim3 grid(hkv, batch);
    const size_t lds = (size_t)grp * D * sizeof(float);
    hipLaunchKernelGGL(select_kernel, grid, dim3(D), lds, s, q, t_q, hq, hkv, n_keep, q_prime, sel_idx);
    return hipGetLastError();
}

}  // namespace dqk
