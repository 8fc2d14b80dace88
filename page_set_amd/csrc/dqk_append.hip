// Quantize-append: k' = k T_K on MFMA and INT2 packing of keys and values
// into 128-token pages (Dual-QK paper: keys are transformed before they are
// stored, §3.4; channel-major 32-byte key rows with channel 0 in bf16 outside
// the INT2 range and token-major values with separate metadata, §3.3).
//
// One workgroup (4 waves) per (logical page, sequence, KV head).
//   1. The page's 128x128 bf16 key tile and T_K (transposed, so that the
//      contraction index is contiguous) are staged in LDS with padded rows.
//   2. Wave w computes k' for output channels 32w..32w+31 and all 128 tokens
//      with v_mfma_f32_16x16x32_bf16 (8 token tiles x 2 channel tiles x 4
//      k-steps).  Token tile mt, row i holds token 32*(i/4) + 4*mt + i%4, so
//      every lane ends up with 32 consecutive tokens of two channels: the
//      8-byte slice of each channel row it packs and stores directly.
//   3. Per channel: min/max over valid tokens (in-lane, then across the four
//      16-lane rows), the binary16 grid, codes, one 8-byte store per lane.
//   4. Values: 512 (token, 32-channel group) units, two per lane.
// Built with -ffp-contract=off: the grid arithmetic must round as written.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int LDS_ROW = D + 8;  // bf16 elements per padded LDS row (272 bytes)

__device__ __forceinline__ float wave_row_min(float x) {
    x = fminf(x, __shfl_xor(x, 16));
    return fminf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_row_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__global__ __launch_bounds__(256) void append_kernel(dqk_cache c, const uint16_t *__restrict__ kin,
                                                     const uint16_t *__restrict__ vin,
                                                     const uint16_t *__restrict__ t_k,
                                                     const int32_t *__restrict__ cu_tokens,
                                                     const int32_t *__restrict__ page_table, int max_pages,
                                                     float *__restrict__ kprime_dbg) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[PG * LDS_ROW];  // [token][in ch]
    __shared__ __attribute__((aligned(16))) uint16_t tt[D * LDS_ROW];   // [out ch][in ch]

    const int pi = blockIdx.x, sq = blockIdx.y, g = blockIdx.z;
    const int hkv = c.num_kv_heads;
    const int64_t tok0 = cu_tokens[sq];
    const int64_t L = (int64_t)cu_tokens[sq + 1] - tok0;
    if ((int64_t)pi * PG >= L) return;
    const int nvalid = (int)min<int64_t>(PG, L - (int64_t)pi * PG);
    const int64_t p = page_table[(size_t)sq * max_pages + pi];
    const int64_t t0 = tok0 + (int64_t)pi * PG;
    const int tid = threadIdx.x;

    // ---- stage keys and T_K^T in LDS
    for (int ch = tid; ch < PG * (D / 8); ch += 256) {
        const int t = ch >> 4, part = ch & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (t < nvalid)
            val = *reinterpret_cast<const u32x4 *>(kin + ((size_t)(t0 + t) * hkv + g) * D + part * 8);
        *reinterpret_cast<u32x4 *>(&ks[t * LDS_ROW + part * 8]) = val;
    }
    const uint16_t *T = t_k + (size_t)g * D * D;
    for (int ch = tid; ch < D * (D / 8); ch += 256) {
        const int i = ch >> 4, j0 = (ch & 15) * 8;
        u32x4 val = *reinterpret_cast<const u32x4 *>(T + (size_t)i * D + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tt[(j0 + 2 * e) * LDS_ROW + i] = (uint16_t)(val[e] & 0xFFFFu);
            tt[(j0 + 2 * e + 1) * LDS_ROW + i] = (uint16_t)(val[e] >> 16);
        }
    }

    // ---- values (independent of the key tile): two (token, group) units per lane
    const size_t pg = (size_t)p * hkv + g;
    for (int u = tid; u < PG * VGROUPS; u += 256) {
        const int t = u >> 2, q = u & 3;
        uint64_t bits = 0;
        uint16_t sb = 0, zb = 0;
        if (t < nvalid) {
            const uint16_t *src = vin + ((size_t)(t0 + t) * hkv + g) * D + q * 32;
            float x[32];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                u32x4 raw = *reinterpret_cast<const u32x4 *>(src + w4 * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[w4 * 8 + 2 * e] = __uint_as_float(raw[e] << 16);
                    x[w4 * 8 + 2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
                }
            }
            float mn = x[0], mx = x[0];
#pragma unroll
            for (int e = 1; e < 32; ++e) {
                mn = fminf(mn, x[e]);
                mx = fmaxf(mx, x[e]);
            }
            const Grid gr = make_grid(mn, mx);
            const Thresholds th = thresholds(gr);
#pragma unroll
            for (int e = 0; e < 32; ++e) bits |= (uint64_t)code2(x[e], th) << (2 * e);
            sb = gr.sb;
            zb = gr.zb;
        }
        *reinterpret_cast<uint64_t *>(c.v_codes + (pg * PG + t) * ROW_BYTES + q * 8) = bits;
        c.v_meta[(pg * 2 + 0) * VGROUPS * PG + q * PG + t] = sb;
        c.v_meta[(pg * 2 + 1) * VGROUPS * PG + q * PG + t] = zb;
    }
    __syncthreads();

    // ---- k' = k T_K on MFMA
    const int lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
    f32x4 acc[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        bf16x8 bop[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            bop[nt] = *reinterpret_cast<const bf16x8 *>(&tt[(32 * w + 16 * nt + n) * LDS_ROW + 32 * kk + 8 * G]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int i = n;  // A row held by this lane
            const int tok = 32 * (i >> 2) + 4 * mt + (i & 3);
            const bf16x8 aop = *reinterpret_cast<const bf16x8 *>(&ks[tok * LDS_ROW + 32 * kk + 8 * G]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[nt], acc[mt][nt], 0, 0, 0);
        }
    }

    // ---- epilogue: lane holds tokens 32G .. 32G+31 of channels 32w + 16nt + n
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int ch = 32 * w + 16 * nt + n;
        if (kprime_dbg) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 32 * G + 4 * mt + r;
                    if (tok < nvalid) kprime_dbg[((size_t)(t0 + tok) * hkv + g) * D + ch] = acc[mt][nt][r];
                }
        }
        uint8_t *row = c.k_codes + krow(p, g, hkv, ch) * ROW_BYTES + 8 * G;
        if (ch == 0) {
            uint16_t *k0 = c.k_ch0 + pg * PG + 32 * G;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 32 * G + 4 * mt + r;
                    k0[4 * mt + r] = tok < nvalid ? f2bf_rne(acc[mt][nt][r]) : (uint16_t)0;
                }
            *reinterpret_cast<uint64_t *>(row) = 0;
            if (G == 0) *reinterpret_cast<uint32_t *>(c.k_meta + krow(p, g, hkv, ch) * 2) = 0u;
            continue;
        }
        float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 32 * G + 4 * mt + r;
                if (tok < nvalid) {
                    mn = fminf(mn, acc[mt][nt][r]);
                    mx = fmaxf(mx, acc[mt][nt][r]);
                }
            }
        mn = wave_row_min(mn);
        mx = wave_row_max(mx);
        const Grid gr = make_grid(mn, mx);
        const Thresholds th = thresholds(gr);
        uint64_t bits = 0;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 32 * G + 4 * mt + r;
                const uint64_t cd = tok < nvalid ? code2(acc[mt][nt][r], th) : 0u;
                bits |= cd << (8 * mt + 2 * r);
            }
        *reinterpret_cast<uint64_t *>(row) = bits;
        if (G == 0)
            *reinterpret_cast<uint32_t *>(c.k_meta + krow(p, g, hkv, ch) * 2) = (uint32_t)gr.sb | ((uint32_t)gr.zb << 16);
    }
}

}  // namespace

hipError_t launch_append(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k, int n_seqs,
                         const int32_t *cu_tokens, const int32_t *page_table, int max_pages, float *kprime_dbg,
                         hipStream_t s) {
    dim3 grid(max_pages, n_seqs, c.num_kv_heads);
    hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, s, c, k, v, t_k, cu_tokens, page_table, max_pages,
                       kprime_dbg);
    return hipGetLastError();
}

}  // namespace dqk
