// Inverse value rotation after aggregation (Dual-QK paper, §3.4: scores of
// every tier share one softmax, then the values are aggregated and the value
// rotation is undone; the rotation itself is the calibrated value rotation
// composed with a Hadamard transform of §3.3 and App. B.2).
//
// The decode aggregates rotated values, o' = sum_t p_t v'_t with v' = v R_V,
// so the output is o = o' R_V^-1: one 128 x 128 product per query head, with
// R_V^-1 shared by the query heads of a KV head.
//
// One workgroup of 128 lanes per (KV head g, sequence b, quarter of the
// output channels): the quarter's 32 columns of R_V^-1[g] (16 KB) and the
// group's rows of o' are staged in LDS (every load of the matrix issued
// before any is stored), then lane (r, c) computes output channel c of query
// heads r, r + 4, ... as an fp32 fma chain over ascending j.  Every
// workgroup reads whole rows of o', so the output must not overlap them.
// Built with -ffp-contract=off: only the written fmas fuse.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int THREADS = 128;
constexpr int QCOLS = 32;               // output channels per workgroup
constexpr int ROWS = THREADS / QCOLS;   // query heads computed side by side

__global__ __launch_bounds__(THREADS) void value_unrotate_kernel(const float *__restrict__ o_rot,
                                                                 const float *__restrict__ r_inv, int hq, int hkv,
                                                                 float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) float r_lds[D * QCOLS];  // [j][c]
    extern __shared__ __attribute__((aligned(16))) float o_lds[];    // [grp][128]
    const int g = blockIdx.x, b = blockIdx.y, q0 = blockIdx.z * QCOLS, tid = threadIdx.x;
    const int grp = hq / hkv;
    constexpr int PER = D * QCOLS / 4 / THREADS;  // 8 float4 per lane
    const float *src = r_inv + (size_t)g * D * D + q0;
    float4 stage[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int idx = tid + k * THREADS, j = idx / (QCOLS / 4), c4 = idx % (QCOLS / 4);
        stage[k] = *reinterpret_cast<const float4 *>(src + (size_t)j * D + 4 * c4);
    }
    const size_t row0 = (size_t)b * hq + (size_t)g * grp;
    const float *rows = o_rot + row0 * D;
    for (int i = tid; i < grp * D; i += THREADS) o_lds[i] = rows[i];
#pragma unroll
    for (int k = 0; k < PER; ++k) reinterpret_cast<float4 *>(r_lds)[tid + k * THREADS] = stage[k];
    __syncthreads();
    const int c = tid % QCOLS, r = tid / QCOLS;
    for (int h = r; h < grp; h += ROWS) {
        float acc = 0.0f;
#pragma unroll 8
        for (int j = 0; j < D; ++j) acc = __builtin_fmaf(o_lds[h * D + j], r_lds[j * QCOLS + c], acc);
        out[(row0 + h) * D + q0 + c] = acc;
    }
}

// The split merge of one (sequence, query head) row followed by the inverse
// rotation: block (b, h) of 128 lanes merges its partials into LDS (the log-
// sum-exp merge of the plain decode), then lane c forms out_c = sum_j o'_j
// R_V^-1[g][j][c] with the fp32 fma chain over ascending j of
// value_unrotate_kernel, reading R_V^-1 (shared by the KV head's query heads,
// so mostly from L2) one coalesced 512-byte row per j.
__global__ __launch_bounds__(D) void merge_unrotate_kernel(const float *__restrict__ partials, int nsplit,
                                                           const float *__restrict__ r_inv, int hq, int hkv,
                                                           float *__restrict__ out, float *__restrict__ lse) {
    __shared__ float w_lds[D];
    __shared__ float red[3][D / 64];
    __shared__ float o_lds[D];
    const int bh = blockIdx.x, h = bh % hq, g = h / (hq / hkv), c = threadIdx.x;
    const float *P = partials + (size_t)bh * nsplit * PART_FLOATS;
    auto part = [&](int s) { return P + (size_t)s * PART_FLOATS; };
    merge_row(part, nsplit, c, true, o_lds, lse ? lse + bh : nullptr, w_lds, red);
    __syncthreads();
    const float *r = r_inv + (size_t)g * D * D + c;
    float acc = 0.0f;
#pragma unroll 16
    for (int j = 0; j < D; ++j) acc = __builtin_fmaf(o_lds[j], r[(size_t)j * D], acc);
    out[(size_t)bh * D + c] = acc;
}

}  // namespace

hipError_t launch_merge_unrotate(const float *partials, int batch, int hq, int hkv, int num_splits,
                                 const float *r_inv, float *out, float *lse, hipStream_t s) {
    hipLaunchKernelGGL(merge_unrotate_kernel, dim3(batch * hq), dim3(D), 0, s, partials, num_splits, r_inv, hq, hkv,
                       out, lse);
    return hipGetLastError();
}

hipError_t launch_value_unrotate(const float *o_rot, const float *r_inv, int batch, int hq, int hkv, float *out,
                                 hipStream_t s) {
    const int grp = hq / hkv;
    hipLaunchKernelGGL(value_unrotate_kernel, dim3(hkv, batch, D / QCOLS), dim3(THREADS),
                       (size_t)grp * D * sizeof(float), s, o_rot, r_inv, hq, hkv, out);
    return hipGetLastError();
}

}  // namespace dqk
