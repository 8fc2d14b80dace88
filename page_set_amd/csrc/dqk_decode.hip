// Decode attention over the paged INT2 cache -- generic path (any group size
// up to 16 query heads per KV head), the split-K log-sum-exp merge, and the
// unpruned BF16 baseline.
//
// Dual-QK paper: scores use only the KV head's selected channels and keep the
// full 1/sqrt(d) normalisation (§3.2); channel 0 comes from its bf16 copy,
// the others are dequantized from the channel-major rows (§3.3); values are
// read for every token (§3.2); one softmax spans the whole context (§3.4),
// realised as an online softmax per split and a log-sum-exp merge.
//
// Workgroup (256 lanes) per (split, sequence x KV head).  Per page: the
// selected key rows, their metadata, channel 0 and the value page are staged
// in LDS; lane (token, half) scores its token for half of the group's heads;
// one wave per head updates the running max/sum; lane (channel, half)
// accumulates its channel for half of the heads.  The group size 4 case runs
// on the MFMA kernel in dqk_decode_mfma.hip instead.
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

// The cache description is passed by value (kernel arguments live in constant memory).
__global__ __launch_bounds__(256) void decode_int2_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                          const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                          const int32_t *__restrict__ page_table, int max_pages,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          int nsplit, float *__restrict__ partials) {
    __shared__ float q_lds[MAXG][D];
    __shared__ int jrow[D];                // compacted selected INT2 channels
    __shared__ __attribute__((aligned(16))) uint8_t krows[D][ROW_BYTES];
    __shared__ float ks_lds[D], kz_lds[D];
    __shared__ float k0_lds[PG];
    __shared__ __attribute__((aligned(16))) uint8_t vrows[PG][ROW_BYTES];
    __shared__ float vs_lds[VGROUPS][PG], vz_lds[VGROUPS][PG];
    __shared__ float lg[MAXG][PG];
    __shared__ float m_lds[MAXG], l_lds[MAXG], a_lds[MAXG];
    __shared__ int nrow_lds, has0_lds;

    const int split = blockIdx.x;
    const int bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    const int b = bg / hkv, g = bg % hkv;
    const int grp = hq / hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    int p0, p1;
    split_range(npages, nsplit, split, p0, p1);

    for (int i = tid; i < grp * D; i += 256) q_lds[i / D][i % D] = q_prime[((size_t)b * hq + (size_t)g * grp) * D + i];
    if (tid == 0) {
        const int32_t *sel = sel_idx + ((size_t)b * hkv + g) * n_keep;
        int nr = 0, h0 = 0;
        for (int m = 0; m < n_keep; ++m) {
            const int j = sel[m];
            if (j == 0)
                h0 = 1;
            else
                jrow[nr++] = j;
        }
        nrow_lds = nr;
        has0_lds = h0;
    }
    if (tid < MAXG) {
        m_lds[tid] = -__builtin_huge_valf();
        l_lds[tid] = 0.0f;
    }
    __syncthreads();
    const int nrow = nrow_lds, has0 = has0_lds;

    const int t = tid & (PG - 1), half = tid >> 7;
    float o[HPER];
#pragma unroll
    for (int k = 0; k < HPER; ++k) o[k] = 0.0f;

    for (int pi = p0; pi < p1; ++pi) {
        const int64_t p = page_table[(size_t)b * max_pages + pi];
        const size_t pg = (size_t)p * hkv + g;
        const int nvalid = min(PG, L - pi * PG);
        // ---- stage the page
        for (int r = tid; r < nrow * 2; r += 256) {
            const int jj = r >> 1, hf = r & 1;
            const int j = jrow[jj];
            *reinterpret_cast<uint4 *>(&krows[jj][hf * 16]) =
                *reinterpret_cast<const uint4 *>(c.k_codes + (pg * D + j) * ROW_BYTES + hf * 16);
            if (hf == 0) {
                const uint32_t sz = *reinterpret_cast<const uint32_t *>(c.k_meta + (pg * D + j) * 2);
                ks_lds[jj] = h2f((uint16_t)(sz & 0xFFFFu));
                kz_lds[jj] = h2f((uint16_t)(sz >> 16));
            }
        }
        if (tid < PG) k0_lds[tid] = has0 ? bf2f(c.k_ch0[pg * PG + tid]) : 0.0f;
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(c.v_codes + pg * PG * ROW_BYTES);
            uint4 *dst = reinterpret_cast<uint4 *>(&vrows[0][0]);
            dst[tid] = src[tid];  // 4096 bytes = 256 x 16
            const uint16_t *vm = c.v_meta + pg * 2 * VGROUPS * PG;
            for (int i = tid; i < VGROUPS * PG; i += 256) {
                vs_lds[i / PG][i % PG] = h2f(vm[i]);
                vz_lds[i / PG][i % PG] = h2f(vm[VGROUPS * PG + i]);
            }
        }
        __syncthreads();
        // ---- logits: lane (t, half) for heads half, half+2, ...
        {
            float acc[HPER];
#pragma unroll
            for (int k = 0; k < HPER; ++k) acc[k] = 0.0f;
            const int byte = t >> 2, sh = 2 * (t & 3);
            for (int jj = 0; jj < nrow; ++jj) {
                const float code = (float)((krows[jj][byte] >> sh) & 3);
                const float kv = __builtin_fmaf(code, ks_lds[jj], kz_lds[jj]);
                const int j = jrow[jj];
#pragma unroll
                for (int k = 0; k < HPER; ++k) {
                    const int h = half + 2 * k;
                    if (h < grp) acc[k] = __builtin_fmaf(q_lds[h][j], kv, acc[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < HPER; ++k) {
                const int h = half + 2 * k;
                if (h < grp) {
                    float x = acc[k];
                    if (has0) x = __builtin_fmaf(q_lds[h][0], k0_lds[t], x);
                    lg[h][t] = x * sm_scale;
                }
            }
        }
        __syncthreads();
        for (int h = wv; h < grp; h += 4) softmax_page(lg[h], nvalid, &m_lds[h], &l_lds[h], &a_lds[h], lane);
        __syncthreads();
        // ---- values: lane (channel t, half)
        {
            const int cch = t, q = cch >> 5, byte = cch >> 2, sh = 2 * (cch & 3);
#pragma unroll
            for (int k = 0; k < HPER; ++k) {
                const int h = half + 2 * k;
                if (h < grp) o[k] *= a_lds[h];
            }
            for (int tt = 0; tt < nvalid; ++tt) {
                const float code = (float)((vrows[tt][byte] >> sh) & 3);
                const float vv = __builtin_fmaf(code, vs_lds[q][tt], vz_lds[q][tt]);
#pragma unroll
                for (int k = 0; k < HPER; ++k) {
                    const int h = half + 2 * k;
                    if (h < grp) o[k] = __builtin_fmaf(lg[h][tt], vv, o[k]);
                }
            }
        }
        __syncthreads();
    }
    // ---- partials
#pragma unroll
    for (int k = 0; k < HPER; ++k) {
        const int h = half + 2 * k;
        if (h < grp) {
            float *dst = partials + (((size_t)b * hq + (size_t)g * grp + h) * nsplit + split) * PART_FLOATS;
            dst[t] = o[k];
            if (t == 0) {
                dst[D] = m_lds[h];
                dst[D + 1] = l_lds[h];
            }
        }
    }
}

// Unpruned BF16 baseline on a paged bf16 cache [P][Hkv][128 tok][128 ch].
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
    for (int i = tid; i < grp * D; i += 256) q_lds[i / D][i % D] = bf2f(q[((size_t)b * hq + (size_t)g * grp) * D + i]);
    if (tid < MAXG) {
        m_lds[tid] = -__builtin_huge_valf();
        l_lds[tid] = 0.0f;
    }
    __syncthreads();
    const int t = tid & (PG - 1), half = tid >> 7;
    float o[HPER];
#pragma unroll
    for (int k = 0; k < HPER; ++k) o[k] = 0.0f;
    for (int pi = p0; pi < p1; ++pi) {
        const int64_t p = page_table[(size_t)b * max_pages + pi];
        const size_t pg = (size_t)p * hkv + g;
        const int nvalid = min(PG, L - pi * PG);
        {
            float acc[HPER];
#pragma unroll
            for (int k = 0; k < HPER; ++k) acc[k] = 0.0f;
            const uint4 *kr = reinterpret_cast<const uint4 *>(kp + (pg * PG + t) * D);
            for (int c8 = 0; c8 < D / 8; ++c8) {
                const uint4 raw = kr[c8];
                const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k_lo = __uint_as_float(wds[e] << 16), k_hi = __uint_as_float(wds[e] & 0xFFFF0000u);
                    const int cc = c8 * 8 + 2 * e;
#pragma unroll
                    for (int k = 0; k < HPER; ++k) {
                        const int h = half + 2 * k;
                        if (h < grp) acc[k] = __builtin_fmaf(q_lds[h][cc + 1], k_hi, __builtin_fmaf(q_lds[h][cc], k_lo, acc[k]));
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < HPER; ++k) {
                const int h = half + 2 * k;
                if (h < grp) lg[h][t] = acc[k] * sm_scale;
            }
        }
        __syncthreads();
        for (int h = wv; h < grp; h += 4) softmax_page(lg[h], nvalid, &m_lds[h], &l_lds[h], &a_lds[h], lane);
        __syncthreads();
        {
            const int cch = t;
#pragma unroll
            for (int k = 0; k < HPER; ++k) {
                const int h = half + 2 * k;
                if (h < grp) o[k] *= a_lds[h];
            }
            const uint16_t *vc = vp + pg * PG * D + cch;
            for (int tt = 0; tt < nvalid; ++tt) {
                const float vv = bf2f(vc[(size_t)tt * D]);
#pragma unroll
                for (int k = 0; k < HPER; ++k) {
                    const int h = half + 2 * k;
                    if (h < grp) o[k] = __builtin_fmaf(lg[h][tt], vv, o[k]);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < HPER; ++k) {
        const int h = half + 2 * k;
        if (h < grp) {
            float *dst = partials + (((size_t)b * hq + (size_t)g * grp + h) * nsplit + split) * PART_FLOATS;
            dst[t] = o[k];
            if (t == 0) {
                dst[D] = m_lds[h];
                dst[D + 1] = l_lds[h];
            }
        }
    }
}

// Log-sum-exp merge of the split partials: one workgroup (128 lanes) per
// (sequence, query head), lane = channel.
constexpr int MERGE_FAST = 32;  // splits whose partials one lane keeps in registers

__global__ __launch_bounds__(D) void merge_kernel(const float *__restrict__ partials, int nsplit,
                                                  float *__restrict__ out, float *__restrict__ lse) {
    // one block of 128 lanes per (sequence, query head); lane c owns output channel c
    __shared__ float w_lds[D];
    __shared__ float red[2][D / 64];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float *P = partials + (size_t)bh * nsplit * PART_FLOATS;
    // every load that does not depend on the maximum is issued up front
    float xf[MERGE_FAST];
    if (nsplit <= MERGE_FAST) {
#pragma unroll
        for (int s = 0; s < MERGE_FAST; ++s) xf[s] = s < nsplit ? P[(size_t)s * PART_FLOATS + tid] : 0.0f;
    }
    float M = -__builtin_huge_valf(), m_own = -__builtin_huge_valf(), l_own = 0.0f;
    if (tid < nsplit) {
        m_own = P[(size_t)tid * PART_FLOATS + D];
        l_own = P[(size_t)tid * PART_FLOATS + D + 1];
    }
    M = m_own;
    for (int s = tid + D; s < nsplit; s += D) M = fmaxf(M, P[(size_t)s * PART_FLOATS + D]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) red[0][wv] = M;
    __syncthreads();
    M = fmaxf(red[0][0], red[0][1]);
    float lpart = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += D) {
        const int n = min(D, nsplit - s0);
        if (s0 > 0) __syncthreads();  // previous chunk's weights are consumed
        if (tid < n) {
            float m = m_own, l = l_own;
            if (s0 > 0) {
                m = P[(size_t)(s0 + tid) * PART_FLOATS + D];
                l = P[(size_t)(s0 + tid) * PART_FLOATS + D + 1];
            }
            const float w = l > 0.0f ? __expf(m - M) : 0.0f;
            w_lds[tid] = w;
            lpart = __builtin_fmaf(l, w, lpart);
        }
        __syncthreads();
        if (nsplit <= MERGE_FAST) {
#pragma unroll
            for (int s = 0; s < MERGE_FAST; ++s)
                if (s < n) acc = __builtin_fmaf(xf[s], w_lds[s], acc);
        } else {
            const float *Pc = P + (size_t)s0 * PART_FLOATS + tid;
            int s = 0;
            for (; s + 8 <= n; s += 8) {  // eight independent loads in flight, sums kept in split order
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = Pc[(size_t)(s + e) * PART_FLOATS];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], w_lds[s + e], acc);
            }
            for (; s < n; ++s) acc = __builtin_fmaf(Pc[(size_t)s * PART_FLOATS], w_lds[s], acc);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lpart += __shfl_xor(lpart, o);
    if (lane == 0) red[1][wv] = lpart;
    __syncthreads();
    const float Lsum = red[1][0] + red[1][1];
    out[(size_t)bh * D + tid] = acc / Lsum;
    if (lse && tid == 0) lse[bh] = M + __logf(Lsum);
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

int decode_splits_generic(int batch, int hkv, int max_pages) {
    const int units = batch * hkv;
    int s = (1024 + units - 1) / units;
    if (s > max_pages) s = max_pages;
    return s < 1 ? 1 : s;
}

hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_int2_kernel, grid, dim3(256), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeBf16Args &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_bf16_kernel, grid, dim3(256), 0, s, a.k_pages, a.v_pages, a.hkv, a.q, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(a.partials, a.batch, a.hq, a.num_splits, a.out, a.lse, s);
}

hipError_t launch_merge(const float *partials, int batch, int hq, int num_splits, float *out, float *lse,
                        hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3(batch * hq), dim3(D), 0, s, partials, num_splits, out, lse);
    return hipGetLastError();
}

}  // namespace dqk
