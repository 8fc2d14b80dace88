// Inverse value rotation after aggregation (Dual-QK paper, §3.4: scores of
// every tier share one softmax, then the values are aggregated and the value
// rotation is undone; the rotation itself is the calibrated value rotation
// composed with a Hadamard transform of §3.3 and App. B.2).
//
// The decode aggregates rotated values, o' = sum_t p_t v'_t with v' = v R_V,
// so the output is o = o' R_V^-1: one 128 x 128 product per query head, with
// R_V^-1 shared by the query heads of a KV head.
//
// One workgroup of 256 lanes per (KV head g, sequence b): R_V^-1[g] (64 KB)
// and the group's rows of o' are staged in LDS (every load of the matrix is
// issued before any is stored), then lane (half, c) computes output channel c
// of every other query head as an fp32 fma chain over ascending j.  The rows
// are read completely before any is written, so the product runs in place.
// Built with -ffp-contract=off: only the written fmas fuse.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int THREADS = 256;
constexpr int HALVES = THREADS / D;

__global__ __launch_bounds__(THREADS) void value_unrotate_kernel(float *__restrict__ out,
                                                                 const float *__restrict__ r_inv, int hq, int hkv) {
    __shared__ __attribute__((aligned(16))) float r_lds[D * D];
    extern __shared__ __attribute__((aligned(16))) float o_lds[];  // [grp][128]
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int grp = hq / hkv;
    const float4 *src = reinterpret_cast<const float4 *>(r_inv + (size_t)g * D * D);
    float4 *dst = reinterpret_cast<float4 *>(r_lds);
    constexpr int PER = D * D / 4 / THREADS;  // 16 float4 per lane
    float4 stage[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) stage[k] = src[tid + k * THREADS];
    float *rows = out + ((size_t)b * hq + (size_t)g * grp) * D;
    for (int i = tid; i < grp * D; i += THREADS) o_lds[i] = rows[i];
#pragma unroll
    for (int k = 0; k < PER; ++k) dst[tid + k * THREADS] = stage[k];
    __syncthreads();
    const int c = tid & (D - 1), half = tid >> 7;
    for (int h = half; h < grp; h += HALVES) {
        float acc = 0.0f;
#pragma unroll 8
        for (int j = 0; j < D; ++j) acc = __builtin_fmaf(o_lds[h * D + j], r_lds[j * D + c], acc);
        rows[(size_t)h * D + c] = acc;
    }
}

}  // namespace

hipError_t launch_value_unrotate(float *out, const float *r_inv, int batch, int hq, int hkv, hipStream_t s) {
    const int grp = hq / hkv;
    hipLaunchKernelGGL(value_unrotate_kernel, dim3(hkv, batch), dim3(THREADS), (size_t)grp * D * sizeof(float), s,
                       out, r_inv, hq, hkv);
    return hipGetLastError();
}

}  // namespace dqk
