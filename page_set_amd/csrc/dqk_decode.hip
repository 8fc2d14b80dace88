// The split-K log-sum-exp merge of the INT2 decode, the unpruned BF16
// baseline decode and a streaming-read reference kernel.  The INT2 decode
// itself (every group size) is the MFMA kernel of dqk_decode_blk.hip.
//
// Dual-QK paper: one softmax spans the whole context (§3.4), realised as an
// online softmax per split and a log-sum-exp merge of the splits.  The BF16
// baseline is the unpruned reference of §4.4: full-width scores on the bf16
// keys and values in their original coordinates.
#include "dqk_internal.h"

namespace dqk {

namespace {

constexpr int MAXG = 16;
constexpr int HPER = MAXG / 2;  // heads per lane (two lane halves)

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ void split_range(int npages, int nsplit, int s, int &p0, int &p1) {
    const int per = (npages + nsplit - 1) / nsplit;
    p0 = min(npages, s * per);
    p1 = min(npages, p0 + per);
}

// Online-softmax step for one head over one page of logits held in LDS
// (overwritten by the probabilities).  Executed by one wave.
__device__ __forceinline__ void softmax_page(float *lg, int nvalid, float *m_lds, float *l_lds, float *a_lds,
                                             int lane) {
    const float x0 = lane < nvalid ? lg[lane] : -__builtin_huge_valf();
    const float x1 = lane + 64 < nvalid ? lg[lane + 64] : -__builtin_huge_valf();
    const float pm = wave_max(fmaxf(x0, x1));
    const float m_old = *m_lds;
    const float m_new = fmaxf(m_old, pm);
    const float p0 = lane < nvalid ? __expf(x0 - m_new) : 0.0f;
    const float p1 = lane + 64 < nvalid ? __expf(x1 - m_new) : 0.0f;
    lg[lane] = p0;
    lg[lane + 64] = p1;
    const float ps = wave_sum(p0 + p1);
    if (lane == 0) {
        const float alpha = __expf(m_old - m_new);  // 0 on the first page (m_old = -inf)
        *a_lds = alpha;
        *l_lds = *l_lds * alpha + ps;
        *m_lds = m_new;
    }
}

// Unpruned BF16 baseline on a paged bf16 cache [P][Hkv][128 tok][128 ch].
// Lane (token or channel t, half): heads half + 2 k, k < HP (HP = ceil(group
// / 2); the query rows of heads past the group are zero, so their unused
// results cost no branches).  Each page: the lane's whole key row in flight,
// scores, the online softmax of §3.4 per head, then the values 32 tokens at a
// time.
template <int HP>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const uint16_t *__restrict__ kp,
                                                          const uint16_t *__restrict__ vp, int hkv,
                                                          const uint16_t *__restrict__ q, int hq,
                                                          const int32_t *__restrict__ page_table, int max_pages,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          int nsplit, float *__restrict__ partials) {
    __shared__ float q_lds[MAXG][D];
    __shared__ float lg[MAXG][PG];
    __shared__ float m_lds[MAXG], l_lds[MAXG], a_lds[MAXG];
    const int split = blockIdx.x, bg = blockIdx.y;
    const int b = bg / hkv, g = bg % hkv;
    const int grp = hq / hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    int p0, p1;
    split_range(npages, nsplit, split, p0, p1);
    for (int i = tid; i < MAXG * D; i += 256)
        q_lds[i / D][i % D] = i / D < grp ? bf2f(q[((size_t)b * hq + (size_t)g * grp) * D + i]) : 0.0f;
    if (tid < MAXG) {
        m_lds[tid] = -__builtin_huge_valf();
        l_lds[tid] = 0.0f;
    }
    __syncthreads();
    const int t = tid & (PG - 1), half = tid >> 7;
    float o[HP];
#pragma unroll
    for (int k = 0; k < HP; ++k) o[k] = 0.0f;
    for (int pi = p0; pi < p1; ++pi) {
        const int64_t p = page_table[(size_t)b * max_pages + pi];
        const size_t pg = (size_t)p * hkv + g;
        const int nvalid = min(PG, L - pi * PG);
        {
            float acc[HP];
#pragma unroll
            for (int k = 0; k < HP; ++k) acc[k] = 0.0f;
            // the whole key row in flight at once (tokens past the end re-read row 0)
            const uint4 *kr = reinterpret_cast<const uint4 *>(kp + (pg * PG + (t < nvalid ? t : 0)) * D);
            uint4 krow[D / 8];
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) krow[c8] = kr[c8];
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) {
                const uint4 raw = krow[c8];
                const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k_lo = __uint_as_float(wds[e] << 16), k_hi = __uint_as_float(wds[e] & 0xFFFF0000u);
                    const int cc = c8 * 8 + 2 * e;
#pragma unroll
                    for (int k = 0; k < HP; ++k) {
                        const int h = half + 2 * k;
                        acc[k] = __builtin_fmaf(q_lds[h][cc + 1], k_hi, __builtin_fmaf(q_lds[h][cc], k_lo, acc[k]));
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < HP; ++k) lg[half + 2 * k][t] = acc[k] * sm_scale;
        }
        __syncthreads();
        for (int h = wv; h < grp; h += 4) softmax_page(lg[h], nvalid, &m_lds[h], &l_lds[h], &a_lds[h], lane);
        __syncthreads();
        {
            const int cch = t;
#pragma unroll
            for (int k = 0; k < HP; ++k) o[k] *= a_lds[half + 2 * k];
            const uint16_t *vc = vp + pg * PG * D + cch;
            // 32 tokens' values in flight per batch (weights past the end are 0)
            for (int t0 = 0; t0 < nvalid; t0 += 32) {
                uint16_t vraw[32];
#pragma unroll
                for (int e = 0; e < 32; ++e) vraw[e] = vc[(size_t)min(t0 + e, nvalid - 1) * D];
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const float vv = bf2f(vraw[e]);
#pragma unroll
                    for (int k = 0; k < HP; ++k) o[k] = __builtin_fmaf(lg[half + 2 * k][t0 + e], vv, o[k]);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < HP; ++k) {
        const int h = half + 2 * k;
        if (h < grp) {
            float *dst = partials + (((size_t)b * hq + (size_t)g * grp + h) * nsplit + split) * PART_FLOATS;
            dst[t] = o[k];
            if (t == 0) {
                dst[D] = m_lds[h];
                dst[D + 1] = l_lds[h];
                dst[D + 2] = l_lds[h];  // fp32 probabilities: the same sum
            }
        }
    }
}

// Log-sum-exp merge of the split partials: one workgroup (128 lanes) per
// (sequence, query head), lane = channel (merge_row in dqk_internal.h).
__global__ __launch_bounds__(D) void merge_kernel(const float *__restrict__ partials, int nsplit_main,
                                                  const float *__restrict__ extra, int n_extra,
                                                  float *__restrict__ out, float *__restrict__ lse) {
    __shared__ float w_lds[D];
    __shared__ float red[3][D / 64];
    const int bh = blockIdx.x;
    const float *P = partials + (size_t)bh * nsplit_main * PART_FLOATS;
    // partial s: split s of the decode, or (s >= nsplit_main) extra partial s - nsplit_main of this row
    const int nsplit = nsplit_main + (extra ? n_extra : 0);
    const float *X = extra ? extra + (size_t)bh * n_extra * PART_FLOATS : nullptr;
    auto part = [&](int s) {
        return s < nsplit_main ? P + (size_t)s * PART_FLOATS : X + (size_t)(s - nsplit_main) * PART_FLOATS;
    };
    merge_row(part, nsplit, (int)threadIdx.x, true, out + (size_t)bh * D, lse ? lse + bh : nullptr, w_lds, red);
}

// Plain streaming read (measurement reference): block i reads chunk i of
// `per` bytes, 8 KB stages through LDS, two stages in flight.
__global__ __launch_bounds__(64) void stream_read_kernel(const uint8_t *__restrict__ src, size_t per,
                                                         uint32_t *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[2][8192];
    const uint8_t *p = src + (size_t)blockIdx.x * per;
    const int lane = threadIdx.x;
    const int nst = (int)(per / 8192);
    const uint32_t b0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)&buf[0][0];
    auto issue = [&](int s) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint8_t *a = p + (size_t)s * 8192 + k * 1024 + lane * 16;
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(a),
                         "s"(b0 + (uint32_t)(s & 1) * 8192 + k * 1024)
                         : "memory", "m0");
        }
    };
    issue(0);
    uint32_t acc = 0;
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) {
            issue(s + 1);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        acc ^= *(volatile __attribute__((address_space(3))) uint32_t *)(uintptr_t)(b0 + (uint32_t)(s & 1) * 8192 + lane * 4);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    acc += __shfl_xor(acc, 1);
    if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s) {
    // up to 4096 single-wave blocks, each a whole number of 16 KiB
    const size_t units = bytes / 16384;
    int blocks = (int)(units < 4096 ? units : 4096);
    while (units % (size_t)blocks) --blocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(64), 0, s, static_cast<const uint8_t *>(src),
                       bytes / (size_t)blocks, sink);
    return hipGetLastError();
}

int decode_splits_bf16(int batch, int hkv, int max_pages) {
    const int units = batch * hkv;
    int s = (1024 + units - 1) / units;
    if (s > max_pages) s = max_pages;
    return s < 1 ? 1 : s;
}

hipError_t launch_decode_bf16(const DecodeBf16Args &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    const int grp = a.hq / a.hkv;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a.k_pages, a.v_pages, a.hkv, a.q, a.hq, a.page_table,
                           a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    };
    if (grp <= 2)
        go(decode_bf16_kernel<1>);
    else if (grp <= 4)
        go(decode_bf16_kernel<2>);
    else if (grp <= 8)
        go(decode_bf16_kernel<4>);
    else
        go(decode_bf16_kernel<HPER>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(a.partials, a.batch, a.hq, a.num_splits, a.out, a.lse, s);
}

hipError_t launch_merge(const float *partials, int batch, int hq, int num_splits, float *out, float *lse,
                        hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3(batch * hq), dim3(D), 0, s, partials, num_splits, nullptr, 0, out, lse);
    return hipGetLastError();
}

hipError_t launch_merge_extra(const float *partials, int batch, int hq, int num_splits, const float *extra,
                              int n_extra, float *out, float *lse, hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3(batch * hq), dim3(D), 0, s, partials, num_splits, extra, n_extra, out,
                       lse);
    return hipGetLastError();
}

}  // namespace dqk
