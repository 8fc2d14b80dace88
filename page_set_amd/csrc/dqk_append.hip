// Quantize-append: k' = k T_K on MFMA and INT2 packing of keys and values
// into 128-token pages (Dual-QK paper: keys are transformed before they are
// stored, §3.4; channel-major 32-byte key rows with channel 0 in bf16 outside
// the INT2 range and token-major values with separate metadata, §3.3).
//
// One workgroup (4 waves) per (run of NPW logical pages, sequence, KV head).
//   1. T_K is staged once in LDS, transposed so that the contraction index is
//      contiguous (pairs of rows per 4-byte store), and each wave keeps the B
//      fragments of its 32 output channels in VGPRs for all pages of the run.
//      The LDS buffer then holds one page's key tile.
//   2. Per page: the key tile goes global -> LDS by direct loads (16-byte
//      chunks XOR-swizzled within each 256-byte row so that the MFMA operand
//      reads are conflict-free), and the values, which do not need the tile,
//      are packed while it is in flight.
//   3. Wave w computes k' for output channels 32w..32w+31 and all 128 tokens
//      with v_mfma_f32_16x16x32_bf16 (8 token tiles x 2 channel tiles x 4
//      k-steps).  Token tile mt, row i holds token 32*(i/4) + 4*mt + i%4, so
//      every lane ends up with 32 consecutive tokens of two channels: the
//      8-byte slice of each channel row it packs and stores directly.
//   4. Per channel: min/max over valid tokens (in-lane, then across the four
//      16-lane rows), the binary16 grid, codes, one 8-byte store per lane.
//   5. Values: 512 (token, 32-channel group) units per page, two per lane,
//      consecutive lanes on consecutive tokens of one group.
// Full pages take a path without per-token checks.
//
// Rotated values (§3.3 values paragraph, App. B.2 value quantization): the
// values are multiplied by R_V on MFMA too, v' = v R_V, and each (token,
// 32-channel group) grid is fitted to the clipped range [clip min, clip max].
// R_V^T is staged like T_K^T and wave w keeps the A fragments of output
// channels 32w..32w+31 (value group w) in VGPRs.  After a page's keys the
// value tile replaces the key tile in LDS (rows = tokens, chunk c of row r at
// slot c ^ (r & 15)); the 16 x 16 output tiles are (channel, token), so a lane
// holds four consecutive channels of one token (one code byte) and the
// group's other 24 channels sit in the lanes 16 and 32 apart.
//
// Bucket-relative RoPE (§3.4, App. C.4): a page lies inside one 2048-token
// bucket (logical page i in bucket i / 16), so once its key tile has landed
// each lane turns the channel pairs (i, i + 64) of its chunk pair back by the
// bucket's anchor in place (fp32, rounded to bf16 to nearest even) before the
// MFMA reads the tile.
// Built with -ffp-contract=off: the grid arithmetic must round as written.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NPW = 4;                     // logical pages per workgroup
constexpr int KLD = PG * (D / 8) / 256;     // 16-byte key-tile chunks per thread
constexpr int VLD = PG * VGROUPS / 256;     // value units per thread

// 16-byte chunk c of LDS row r sits at slot c ^ swz(r), rows of 256 bytes.
// Key tile (rows = tokens): the 16 rows an operand read touches,
// 32 (i / 4) + 4 mt + i % 4, get distinct slots.  T_K^T (rows = output
// channels): 16 consecutive rows get distinct slots.
__device__ __forceinline__ uint32_t swz_k(int r) { return (uint32_t)((r & 3) | ((r >> 3) & 12)); }
__device__ __forceinline__ uint32_t swz_t(int r) { return (uint32_t)(r & 15); }
// Value tile (rows = tokens): an operand read touches rows 16 tt + n, n = 0..15.
__device__ __forceinline__ uint32_t swz_v(int r) { return (uint32_t)(r & 15); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
    return *(__attribute__((address_space(3))) const T *)(uintptr_t)a;
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t a, T v) {
    *(__attribute__((address_space(3))) T *)(uintptr_t)a = v;
}
// 16 bytes per lane global -> LDS at M0 + 16 lane (the LDS base must be uniform)
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %0" ::"s"(sbase), "v"(voff),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
// The thread index as a value the compiler cannot see through: per-page
// address arithmetic derived from it is redone in each page iteration instead
// of being hoisted out of the loop into registers held across all of it.
__device__ __forceinline__ int fresh_tid() {
    int t = (int)threadIdx.x;
    __asm__ volatile("" : "+v"(t));
    return t;
}
// every load of this wave done, own LDS accesses done, then the barrier
__device__ __forceinline__ void wait_all_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float wave_row_min(float x) {
    x = fminf(x, __shfl_xor(x, 16));
    return fminf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_row_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ uint32_t wave_row_or(uint32_t x) {
    x |= (uint32_t)__shfl_xor((int)x, 16);
    return x | (uint32_t)__shfl_xor((int)x, 32);
}

// Reductions over the 16 lanes of a DPP row (rotations by 8 and 4, then the
// quad permutations xor 2 and xor 1 cover every lane of the row).
template <int CTL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_min(float x) {
    x = fminf(x, dpp<0x128>(x));  // row_ror:8
    x = fminf(x, dpp<0x124>(x));  // row_ror:4
    x = fminf(x, dpp<0x4E>(x));   // quad_perm [2, 3, 0, 1]
    return fminf(x, dpp<0xB1>(x));  // quad_perm [1, 0, 3, 2]
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0x128>(x));
    x = fmaxf(x, dpp<0x124>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    return fmaxf(x, dpp<0xB1>(x));
}

// M^T of a bf16 [in ch][out ch] matrix into LDS rows of 256 bytes ([out ch][in
// ch]): thread (row pair rp, column octet oc) stores the two rows' elements of
// each column as one 4-byte word; chunk c of row r at slot c ^ swz_t(r).
__device__ __forceinline__ void stage_transposed(const uint16_t *__restrict__ M, uint32_t ks) {
    for (int it = threadIdx.x; it < (D / 2) * (D / 8); it += 256) {
        const int rp = it & (D / 2 - 1), oc = it / (D / 2);
        const u32x4 a = *reinterpret_cast<const u32x4 *>(M + (size_t)(2 * rp) * D + oc * 8);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(M + (size_t)(2 * rp + 1) * D + oc * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int row = oc * 8 + e;
            const uint32_t word = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
            lds_st<uint32_t>(ks + row * 256 + ((((uint32_t)rp >> 2) ^ swz_t(row)) << 4) + (rp & 3) * 4, word);
        }
    }
}

// Fragments of the staged M^T for output channels 32 w + 16 nt + n and the
// four 32-deep k-steps (k-octet G), kept in VGPRs for all pages of a run.
__device__ __forceinline__ void load_frags(uint32_t ks, bf16x8 (&f)[2][4]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int row = 32 * w + 16 * nt + n;
            f[nt][kk] = lds_ld<bf16x8>(ks + row * 256 + (((4 * kk + G) ^ swz_t(row)) << 4));
        }
}

// Values of one (token, group) unit from its 64 loaded bytes: 32 channels ->
// codes (2 bits each, channel e at bits 2e), scale and zero point.
__device__ __forceinline__ void pack_value_unit(const u32x4 (&raw)[4], uint64_t &bits, uint16_t &sb, uint16_t &zb) {
    float x[32];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[w4 * 8 + 2 * e] = __uint_as_float(raw[w4][e] << 16);
            x[w4 * 8 + 2 * e + 1] = __uint_as_float(raw[w4][e] & 0xFFFF0000u);
        }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    const Grid gr = make_grid(mn, mx);
    const Thresholds th = thresholds(gr);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        lo |= code2(x[e], th) << (2 * e);
        hi |= code2(x[16 + e], th) << (2 * e);
    }
    bits = (uint64_t)lo | ((uint64_t)hi << 32);
    sb = gr.sb;
    zb = gr.zb;
}

// The values of one page (token t's 128 values at vpage + t vstride): thread
// tid packs units (token t, group q0 + 2 k), t = tid % 128, q0 = tid / 128.
// FULL: all 128 tokens valid.
template <bool FULL>
__device__ __forceinline__ void values_of_page(const dqk_cache &c, const uint16_t *__restrict__ vpage,
                                               size_t vstride, int tid, size_t pg, int nvalid) {
    const int t = tid & (PG - 1), q0 = tid / PG;
    const bool valid = FULL || t < nvalid;
    const uint16_t *vsrc = vpage + (size_t)(valid ? t : 0) * vstride + q0 * 32;
    u32x4 raw[VLD][4];
#pragma unroll
    for (int k = 0; k < VLD; ++k)
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) raw[k][w4] = *reinterpret_cast<const u32x4 *>(vsrc + 64 * k + w4 * 8);
#pragma unroll
    for (int k = 0; k < VLD; ++k) {
        __builtin_amdgcn_sched_barrier(0);  // one unit's values live at a time
        const int q = q0 + 2 * k;
        uint64_t bits = 0;
        uint16_t sb = 0, zb = 0;
        if (valid) pack_value_unit(raw[k], bits, sb, zb);
        *reinterpret_cast<uint64_t *>(c.v_codes + (pg * PG + t) * ROW_BYTES + q * 8) = bits;
        c.v_meta[(pg * 2 + 0) * VGROUPS * PG + q * PG + t] = sb;
        c.v_meta[(pg * 2 + 1) * VGROUPS * PG + q * PG + t] = zb;
    }
}

// Rotated values of the page whose value tile is in LDS at ks: wave w
// computes v' = v R_V for value group w (channels 32w..32w+31) and all 128
// tokens, two token tiles at a time, and packs them: per token the group's
// extremes (in-lane over 8 channels, then across the four 16-lane rows),
// the clipped grid, one code byte per lane and channel tile, gathered into
// the group's 8 bytes by OR across the rows.
template <bool FULL, bool DBG>
__device__ __forceinline__ void values_rot_of_page(const dqk_cache &c, uint32_t ks, const bf16x8 (&rop)[2][4],
                                                   size_t pg, int g, int hkv, int nvalid, int64_t t0, float clip,
                                                   float *__restrict__ vprime_dbg) {
    const int tid = fresh_tid(), lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
    // B fragment of token tile tt, k-step kk: row 16 tt + n, chunk 4 kk + G
    const uint32_t brow = ks + (uint32_t)n * 256;
#pragma unroll
    for (int tp = 0; tp < 4; ++tp) {
        f32x4 acc[2][2];
        bf16x8 bv[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                bv[j][kk] = lds_ld<bf16x8>(brow + (uint32_t)(2 * tp + j) * 4096 + (((uint32_t)(4 * kk + G) ^ (uint32_t)n) << 4));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[j][ct] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    acc[j][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rop[ct][kk], bv[j][kk], acc[j][ct], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // lane holds channels 32 w + 16 ct + 4 G + r of token tok
            const int tok = 16 * (2 * tp + j) + n;
            const bool valid = FULL || tok < nvalid;
            if (DBG && vprime_dbg && valid) {
                float *dst = vprime_dbg + ((size_t)(t0 + tok) * hkv + g) * D + 32 * w + 4 * G;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[16 * ct + r] = acc[j][ct][r];
            }
            float mn = acc[j][0][0], mx = acc[j][0][0];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    mn = fminf(mn, acc[j][ct][r]);
                    mx = fmaxf(mx, acc[j][ct][r]);
                }
            mn = wave_row_min(mn);
            mx = wave_row_max(mx);
            const Grid gr = make_grid(__fmul_rn(clip, mn), __fmul_rn(clip, mx));
            const Thresholds th = thresholds(gr);
            uint32_t e = 0, o = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                e |= code2(acc[j][0][r], th) << (2 * r);
                o |= code2(acc[j][1][r], th) << (2 * r);
            }
            // group bytes 0..3 come from channel tile 0 (rows G = 0..3), 4..7 from tile 1
            const uint32_t lo = wave_row_or(e << (8 * G)), hi = wave_row_or(o << (8 * G));
            if (G == 0) {
                const uint64_t bits = valid ? ((uint64_t)lo | ((uint64_t)hi << 32)) : 0ull;
                *reinterpret_cast<uint64_t *>(c.v_codes + (pg * PG + tok) * ROW_BYTES + 8 * w) = bits;
                c.v_meta[(pg * 2 + 0) * VGROUPS * PG + w * PG + tok] = valid ? gr.sb : (uint16_t)0;
                c.v_meta[(pg * 2 + 1) * VGROUPS * PG + w * PG + tok] = valid ? gr.zb : (uint16_t)0;
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one token-tile pair live at a time
    }
}

// k' of the tile in LDS for 16 output channels (channel tile nt of this
// wave's 32), then the packed key rows, metadata and channel 0.  FULL: all 128
// tokens valid; DBG: k' also goes to kprime_dbg.
template <bool FULL, bool DBG>
__device__ __forceinline__ void keys_of_page(const dqk_cache &c, uint32_t ks, const bf16x8 (&bop)[4], int nt,
                                             int64_t p, int g, int hkv, int nvalid, int64_t t0,
                                             float *__restrict__ kprime_dbg) {
    const int tid = fresh_tid(), lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = {0.f, 0.f, 0.f, 0.f};
    // A row n of token tile mt is token 32 (n / 4) + 4 mt + n % 4, whose swizzle
    // swz_k is n for every mt: one address per k-step, mt in the offset field
    const uint32_t arow = ks + (uint32_t)(32 * (n >> 2) + (n & 3)) * 256;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t ak = arow + ((uint32_t)((4 * kk + G) ^ n) << 4);
        bf16x8 aop[8];  // the k-step's eight A fragments in flight together
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) aop[mt] = lds_ld<bf16x8>(ak + mt * 1024);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mt], bop[kk], acc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const size_t pg = (size_t)p * hkv + g;
    // lane holds tokens 32G .. 32G+31 of channel 32w + 16nt + n
    const int ch = 32 * w + 16 * nt + n;
    if (DBG && kprime_dbg) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 32 * G + 4 * mt + r;
                if (FULL || tok < nvalid) kprime_dbg[((size_t)(t0 + tok) * hkv + g) * D + ch] = acc[mt][r];
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
                k0[4 * mt + r] = (FULL || tok < nvalid) ? f2bf_rne(acc[mt][r]) : (uint16_t)0;
            }
        *reinterpret_cast<uint64_t *>(row) = 0;
        if (G == 0) *reinterpret_cast<uint32_t *>(c.k_meta + krow(p, g, hkv, ch) * 2) = 0u;
        return;
    }
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = 32 * G + 4 * mt + r;
            if (FULL || tok < nvalid) {
                mn = fminf(mn, acc[mt][r]);
                mx = fmaxf(mx, acc[mt][r]);
            }
        }
    mn = wave_row_min(mn);
    mx = wave_row_max(mx);
    const Grid gr = make_grid(mn, mx);
    const Thresholds th = thresholds(gr);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = 32 * G + 4 * mt + r;
            const uint32_t cd = (FULL || tok < nvalid) ? code2(acc[mt][r], th) : 0u;
            if (mt < 4)
                lo |= cd << (8 * mt + 2 * r);
            else
                hi |= cd << (8 * (mt - 4) + 2 * r);
        }
    *reinterpret_cast<uint64_t *>(row) = (uint64_t)lo | ((uint64_t)hi << 32);
    if (G == 0)
        *reinterpret_cast<uint32_t *>(c.k_meta + krow(p, g, hkv, ch) * 2) = (uint32_t)gr.sb | ((uint32_t)gr.zb << 16);
}

// Keys of the page with one grid per token and KV head over channels 1..127
// (§3.3 as the paper states it; channel 0 stays in bf16, outside the range).
// A token's grid needs all its channels, so both channel tiles of the wave
// are computed first.  Per-token extremes: in-lane over the lane's two
// channels (channel 0 left out), over the 16 lanes of a row by DPP, over the
// four waves through LDS, which reuses the key tile once every wave has read
// it; thread t < 128 then fits token t's grid, writes its (scale, zero) and
// leaves the thresholds in LDS for the code pass.
template <bool FULL, bool DBG>
__device__ __forceinline__ void keys_of_page_tok(const dqk_cache &c, uint32_t ks, const bf16x8 (&bop)[2][4],
                                                 int64_t p, int g, int hkv, int nvalid, int64_t t0,
                                                 float *__restrict__ kprime_dbg) {
    const int tid = fresh_tid(), lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, n = lane & 15;
    f32x4 acc[2][8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = {0.f, 0.f, 0.f, 0.f};
    const uint32_t arow = ks + (uint32_t)(32 * (n >> 2) + (n & 3)) * 256;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t ak = arow + ((uint32_t)((4 * kk + G) ^ n) << 4);
        bf16x8 aop[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) aop[mt] = lds_ld<bf16x8>(ak + mt * 1024);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mt], bop[nt][kk], acc[nt][mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const size_t pg = (size_t)p * hkv + g;
    // lane holds tokens 32G .. 32G+31 of channels 32w + n (tile 0) and 32w + 16 + n (tile 1)
    if (DBG && kprime_dbg) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 32 * G + 4 * mt + r;
                    if (FULL || tok < nvalid)
                        kprime_dbg[((size_t)(t0 + tok) * hkv + g) * D + 32 * w + 16 * nt + n] = acc[nt][mt][r];
                }
    }
    const bool has_ch0 = w == 0 && n == 0;  // tile 0 of this lane is channel 0
    if (has_ch0) {
        uint16_t *k0 = c.k_ch0 + pg * PG + 32 * G;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 32 * G + 4 * mt + r;
                k0[4 * mt + r] = (FULL || tok < nvalid) ? f2bf_rne(acc[0][mt][r]) : (uint16_t)0;
            }
    }
    float mn[32], mx[32];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float a0 = acc[0][mt][r], a1 = acc[1][mt][r];
            mn[4 * mt + r] = has_ch0 ? a1 : fminf(a0, a1);
            mx[4 * mt + r] = has_ch0 ? a1 : fmaxf(a0, a1);
        }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        mn[k] = row16_min(mn[k]);
        mx[k] = row16_max(mx[k]);
    }
    __syncthreads();  // every wave has read the key tile: it now holds [4 waves][128 tokens][min, max]
    if (n == 0) {
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            f32x2 e;
            e[0] = mn[k];
            e[1] = mx[k];
            lds_st<f32x2>(ks + (uint32_t)((w * PG + 32 * G + k) * 8), e);
        }
    }
    __syncthreads();
    const uint32_t thr = ks + 4 * PG * 8;  // [128 tokens][4] thresholds after the extremes
    if (tid < PG) {
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const f32x2 e = lds_ld<f32x2>(ks + (uint32_t)((v * PG + tid) * 8));
            lo = fminf(lo, e[0]);
            hi = fmaxf(hi, e[1]);
        }
        const bool valid = FULL || tid < nvalid;
        const Grid gr = make_grid(lo, hi);
        const Thresholds th = thresholds(gr);
        f32x4 t4;
        t4[0] = th.t0;
        t4[1] = th.t1;
        t4[2] = th.t2;
        t4[3] = 0.0f;
        lds_st<f32x4>(thr + tid * 16, t4);
        *reinterpret_cast<uint32_t *>(c.k_meta + ktok(p, g, hkv, tid) * 2) =
            valid ? ((uint32_t)gr.sb | ((uint32_t)gr.zb << 16)) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int ch = 32 * w + 16 * nt + n;
        uint32_t lo = 0, hi = 0;
        if (ch != 0) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 32 * G + 4 * mt + r;
                    const f32x4 t4 = lds_ld<f32x4>(thr + tok * 16);
                    const Thresholds th{t4[0], t4[1], t4[2]};
                    const uint32_t cd = (FULL || tok < nvalid) ? code2(acc[nt][mt][r], th) : 0u;
                    if (mt < 4)
                        lo |= cd << (8 * mt + 2 * r);
                    else
                        hi |= cd << (8 * (mt - 4) + 2 * r);
                }
        }
        *reinterpret_cast<uint64_t *>(c.k_codes + krow(p, g, hkv, ch) * ROW_BYTES + 8 * G) =
            (uint64_t)lo | ((uint64_t)hi << 32);
    }
}

// Where the pages of a launch come from.
//   APPEND_PLAIN   sequence sq = blockIdx.y, tokens cu_tokens[sq] ..; logical
//                  page i holds tokens 128 i .. (the last one may be partial).
//   APPEND_TIERED  the same inputs, but page i holds tokens 64 + 128 i .. and
//                  only the tier_pages(L) whole pages older than the 256 most
//                  recent tokens are written (the rest stays in the BF16 tiers).
//   APPEND_TAIL    sequence b = blockIdx.y gains token lens_before[b]; if the
//                  new length completes a page's age, that page (tier_pages of
//                  the old length) is packed from the tail's raw keys and
//                  values (slots (128 i .. 128 i + 127) mod 384).
enum { APPEND_PLAIN = 0, APPEND_TIERED = 1, APPEND_TAIL = 2 };

struct AppendSrc {
    const uint16_t *kin, *vin;
    const int32_t *cu_tokens;
    const int32_t *lens_before;
    const uint16_t *tail_kraw, *tail_v;
    const uint16_t *r_v;  // rotated values only: R_V bf16 [Hkv][128][128], the clip ratio, v' output or null
    float clip;
    float *vprime_dbg;
    const float *rope_cos = nullptr, *rope_sin = nullptr;  // bucket-relative RoPE only: tables [n_buckets][64]
};

__device__ __forceinline__ int64_t tier_pages_of(int64_t L) {
    return L >= TIER_SINK + TIER_RECENT ? (L - TIER_SINK - TIER_RECENT) / PG : 0;
}

// Variants: plain; rotated values (a second set of fragments in VGPRs);
// per-token key grids (both channel tiles' accumulators live at once);
// bucket-relative RoPE (plain, with the key tile turned in LDS).  Rotated
// values and per-token grids run two workgroups a CU.
enum { VAR_PLAIN = 0, VAR_VROT = 1, VAR_TOKGRID = 2, VAR_ROPE = 3 };

// Turn the key tile at ks (rows = tokens, chunk c of row r at slot
// c ^ swz_k(r)) back by one bucket's anchor: lane tid owns chunk pair
// (c, c + 8), c = tid % 8 (channels 8c .. 8c + 7 and their partners 64 later),
// of rows tid / 8 + 32 j.  Rows past the sequence end hold token 0 again;
// turning them is harmless (their k' is never used).
__device__ __forceinline__ void rope_turn_tile(uint32_t ks, const float *__restrict__ cs,
                                               const float *__restrict__ sn) {
    const int tid = fresh_tid(), c = tid & 7;
    float cv[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cv[e] = cs[8 * c + e];
        sv[e] = sn[8 * c + e];
    }
#pragma unroll
    for (int j = 0; j < PG * 8 / 256; ++j) {
        const int r = (tid >> 3) + 32 * j;
        const uint32_t alo = ks + (uint32_t)r * 256 + (((uint32_t)c ^ swz_k(r)) << 4);
        const uint32_t ahi = ks + (uint32_t)r * 256 + (((uint32_t)(c + 8) ^ swz_k(r)) << 4);
        const u32x4 lo = lds_ld<u32x4>(alo), hi = lds_ld<u32x4>(ahi);
        u32x4 ylo, yhi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t pl = 0, ph = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * w + h;
                const float x = bf2f((uint16_t)(lo[w] >> (16 * h))), xp = bf2f((uint16_t)(hi[w] >> (16 * h)));
                pl |= (uint32_t)f2bf_rne(rope_turn(x, xp, cv[e], sv[e], true)) << (16 * h);
                ph |= (uint32_t)f2bf_rne(rope_turn(xp, x, cv[e], sv[e], false)) << (16 * h);
            }
            ylo[w] = pl;
            yhi[w] = ph;
        }
        lds_st<u32x4>(alo, ylo);
        lds_st<u32x4>(ahi, yhi);
    }
}

template <bool DBG, int MODE, int VAR>
__global__ __launch_bounds__(256, (VAR == VAR_PLAIN || VAR == VAR_ROPE) ? 4 : 2) void append_kernel(dqk_cache c, AppendSrc src, const uint16_t *__restrict__ t_k,
                                                     const int32_t *__restrict__ page_table, int max_pages,
                                                     float *__restrict__ kprime_dbg) {
    // T_K^T [out ch][in ch] first, then each page's key tile [token][in ch]; rows of 256 bytes
    __shared__ __attribute__((aligned(16))) uint16_t lds_tile[PG * D];
    const uint32_t ks = lds_addr(lds_tile);

    const int sq = blockIdx.y, g = blockIdx.z;
    const int hkv = c.num_kv_heads;
    int64_t tok0 = 0, first0 = 0;  // input token of the sequence's start and of page 0
    int pi0, pi_end;
    if constexpr (MODE == APPEND_TAIL) {
        const int64_t Lb = src.lens_before[sq];
        const int64_t P0 = tier_pages_of(Lb);
        if (tier_pages_of(Lb + 1) == P0 || P0 >= max_pages) return;
        pi0 = (int)P0;
        pi_end = pi0 + 1;
    } else {
        tok0 = src.cu_tokens[sq];
        const int64_t L = (int64_t)src.cu_tokens[sq + 1] - tok0;
        const int64_t npg = MODE == APPEND_TIERED ? tier_pages_of(L) : (L + PG - 1) / PG;
        first0 = tok0 + (MODE == APPEND_TIERED ? TIER_SINK : 0);
        pi0 = blockIdx.x * NPW;
        if (pi0 >= npg) return;
        pi_end = (int)min<int64_t>(min(pi0 + NPW, max_pages), npg);
    }
    const int64_t L_plain = MODE == APPEND_PLAIN ? (int64_t)src.cu_tokens[sq + 1] - tok0 : 0;
    // ---- T_K^T (and R_V^T) staged in turn, their fragments kept in VGPRs
    stage_transposed(t_k + (size_t)g * D * D, ks);
    __syncthreads();
    bf16x8 bop[2][4];  // [channel tile][k-step]
    load_frags(ks, bop);
    bf16x8 rop[2][4];
    if constexpr (VAR == VAR_VROT) {
        __syncthreads();
        stage_transposed(src.r_v + (size_t)g * D * D, ks);
        __syncthreads();
        load_frags(ks, rop);
    }
    const int G = ((int)threadIdx.x & 63) >> 4;

    for (int pi = pi0; pi < pi_end; ++pi) {
        const int nvalid = MODE == APPEND_PLAIN ? (int)min<int64_t>(PG, L_plain - (int64_t)pi * PG) : PG;
        const int64_t p = page_table[(size_t)sq * max_pages + pi];
        const int64_t t0 = first0 + (int64_t)pi * PG;  // input token of the page's slot 0 (not APPEND_TAIL)
        const size_t pg = (size_t)p * hkv + g;
        // the page's token rows: row t at kpage + t kstride (and the same for values)
        const uint16_t *kpage, *vpage;
        size_t kstride;
        if constexpr (MODE == APPEND_TAIL) {
            const size_t slot0 = ((size_t)sq * hkv + g) * TIER_TAIL_SLOTS + (size_t)((PG * pi) % TIER_TAIL_SLOTS);
            kpage = src.tail_kraw + slot0 * D;
            vpage = src.tail_v + slot0 * D;
            kstride = D;
        } else {
            kpage = src.kin + ((size_t)t0 * hkv + g) * D;
            vpage = src.vin + ((size_t)t0 * hkv + g) * D;
            kstride = (size_t)hkv * D;
        }

        __syncthreads();  // the previous tile (or T_K^T) has been read by every wave
        const int tid = fresh_tid(), lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
        // ---- key tile: chunk slot s of row r <- input chunk s ^ swz_k(r).  Load i
        //      of wave w covers rows 32 w + 4 i + G, whose swizzle is G | 4 w for
        //      every i: full pages step a scalar base and keep one lane offset;
        //      rows past the sequence end re-read token 0 (their k' is never used).
        const int row0 = 4 * KLD * w + G;
        const uint32_t slot_off = ((uint32_t)(lane & 15) ^ (uint32_t)(G | 4 * w)) * 16;
        const uint32_t tile_w = ks + (uint32_t)(KLD * w) * 1024;
        if (nvalid == PG) {
            const uint32_t voff = (uint32_t)(G * kstride) * 2 + slot_off;
#pragma unroll
            for (int i = 0; i < KLD; ++i)
                dma16(kpage + (size_t)(4 * KLD * w + 4 * i) * kstride, voff, tile_w + i * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < KLD; ++i) {
                const int row = row0 + 4 * i;
                const int srow = row < nvalid ? row : 0;
                dma16(kpage, (uint32_t)(srow * kstride) * 2 + slot_off, tile_w + i * 1024);
            }
        }

        // ---- values: unit k is (token t, group q0 + 2 k), consecutive lanes on
        //      consecutive tokens; both units of a lane share the token
        if constexpr (VAR != VAR_VROT) {
            if (nvalid == PG)
                values_of_page<true>(c, vpage, kstride, tid, pg, nvalid);
            else
                values_of_page<false>(c, vpage, kstride, tid, pg, nvalid);
        }

        wait_all_barrier();  // the tile has landed
        if constexpr (VAR == VAR_ROPE) {
            const int bk = pi / ROPE_PAGES;
            rope_turn_tile(ks, src.rope_cos + bk * (D / 2), src.rope_sin + bk * (D / 2));
            __syncthreads();
        }
        if constexpr (VAR == VAR_TOKGRID) {
            if (nvalid == PG)
                keys_of_page_tok<true, DBG>(c, ks, bop, p, g, hkv, nvalid, t0, kprime_dbg);
            else
                keys_of_page_tok<false, DBG>(c, ks, bop, p, g, hkv, nvalid, t0, kprime_dbg);
        } else {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if (nvalid == PG)
                    keys_of_page<true, DBG>(c, ks, bop[nt], nt, p, g, hkv, nvalid, t0, kprime_dbg);
                else
                    keys_of_page<false, DBG>(c, ks, bop[nt], nt, p, g, hkv, nvalid, t0, kprime_dbg);
                __builtin_amdgcn_sched_barrier(0);  // one channel tile's accumulators live at a time
            }
        }
        if constexpr (VAR == VAR_VROT) {
            __syncthreads();  // every wave has read the key tile
            // ---- value tile: load i of wave w covers rows 32 w + 4 i + G, LDS slot
            //      lane & 15 of a row receiving input chunk slot ^ swz_v(row)
            const int tid = fresh_tid(), lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
            const uint32_t tile_w = ks + (uint32_t)(32 * w) * 256;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 32 * w + 4 * i + G;
                const int srow = (nvalid == PG || row < nvalid) ? row : 0;
                const uint32_t chunk = (uint32_t)(lane & 15) ^ swz_v(row);
                dma16(vpage, (uint32_t)(srow * kstride) * 2 + chunk * 16, tile_w + i * 1024);
            }
            wait_all_barrier();
            if (nvalid == PG)
                values_rot_of_page<true, DBG>(c, ks, rop, pg, g, hkv, nvalid, t0, src.clip, src.vprime_dbg);
            else
                values_rot_of_page<false, DBG>(c, ks, rop, pg, g, hkv, nvalid, t0, src.clip, src.vprime_dbg);
        }
    }
}

}  // namespace

hipError_t launch_append(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k, int n_seqs,
                         const int32_t *cu_tokens, const int32_t *page_table, int max_pages, float *kprime_dbg,
                         hipStream_t s) {
    dim3 grid((max_pages + NPW - 1) / NPW, n_seqs, c.num_kv_heads);
    const AppendSrc src{k, v, cu_tokens, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr};
    if (kprime_dbg)
        hipLaunchKernelGGL((append_kernel<true, APPEND_PLAIN, VAR_PLAIN>), grid, dim3(256), 0, s, c, src, t_k, page_table,
                           max_pages, kprime_dbg);
    else
        hipLaunchKernelGGL((append_kernel<false, APPEND_PLAIN, VAR_PLAIN>), grid, dim3(256), 0, s, c, src, t_k, page_table,
                           max_pages, kprime_dbg);
    return hipGetLastError();
}

hipError_t launch_append_tiered(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                                int n_seqs, const int32_t *cu_tokens, const int32_t *page_table, int max_pages,
                                hipStream_t s) {
    dim3 grid((max_pages + NPW - 1) / NPW, n_seqs, c.num_kv_heads);
    const AppendSrc src{k, v, cu_tokens, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr};
    hipLaunchKernelGGL((append_kernel<false, APPEND_TIERED, VAR_PLAIN>), grid, dim3(256), 0, s, c, src, t_k, page_table,
                       max_pages, nullptr);
    return hipGetLastError();
}

hipError_t launch_append_vrot(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                              const uint16_t *r_v, float clip, int n_seqs, const int32_t *cu_tokens,
                              const int32_t *page_table, int max_pages, float *kprime_dbg, float *vprime_dbg,
                              hipStream_t s) {
    dim3 grid((max_pages + NPW - 1) / NPW, n_seqs, c.num_kv_heads);
    const AppendSrc src{k, v, cu_tokens, nullptr, nullptr, nullptr, r_v, clip, vprime_dbg};
    if (kprime_dbg || vprime_dbg)
        hipLaunchKernelGGL((append_kernel<true, APPEND_PLAIN, VAR_VROT>), grid, dim3(256), 0, s, c, src, t_k, page_table,
                           max_pages, kprime_dbg);
    else
        hipLaunchKernelGGL((append_kernel<false, APPEND_PLAIN, VAR_VROT>), grid, dim3(256), 0, s, c, src, t_k,
                           page_table, max_pages, kprime_dbg);
    return hipGetLastError();
}

hipError_t launch_append_tokgrid(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                                 int n_seqs, const int32_t *cu_tokens, const int32_t *page_table, int max_pages,
                                 float *kprime_dbg, hipStream_t s) {
    dim3 grid((max_pages + NPW - 1) / NPW, n_seqs, c.num_kv_heads);
    const AppendSrc src{k, v, cu_tokens, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr};
    if (kprime_dbg)
        hipLaunchKernelGGL((append_kernel<true, APPEND_PLAIN, VAR_TOKGRID>), grid, dim3(256), 0, s, c, src, t_k,
                           page_table, max_pages, kprime_dbg);
    else
        hipLaunchKernelGGL((append_kernel<false, APPEND_PLAIN, VAR_TOKGRID>), grid, dim3(256), 0, s, c, src, t_k,
                           page_table, max_pages, kprime_dbg);
    return hipGetLastError();
}

hipError_t launch_append_rope(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k,
                              const float *rope_cos, const float *rope_sin, int n_seqs, const int32_t *cu_tokens,
                              const int32_t *page_table, int max_pages, float *kprime_dbg, hipStream_t s) {
    dim3 grid((max_pages + NPW - 1) / NPW, n_seqs, c.num_kv_heads);
    AppendSrc src{k, v, cu_tokens, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr};
    src.rope_cos = rope_cos;
    src.rope_sin = rope_sin;
    if (kprime_dbg)
        hipLaunchKernelGGL((append_kernel<true, APPEND_PLAIN, VAR_ROPE>), grid, dim3(256), 0, s, c, src, t_k,
                           page_table, max_pages, kprime_dbg);
    else
        hipLaunchKernelGGL((append_kernel<false, APPEND_PLAIN, VAR_ROPE>), grid, dim3(256), 0, s, c, src, t_k,
                           page_table, max_pages, kprime_dbg);
    return hipGetLastError();
}

hipError_t launch_pack_tail(const dqk_cache &c, const dqk_tiers &t, const uint16_t *t_k, int batch,
                            const int32_t *lens_before, const int32_t *page_table, int max_pages, hipStream_t s) {
    dim3 grid(1, batch, c.num_kv_heads);
    const AppendSrc src{nullptr, nullptr, nullptr, lens_before, t.tail_kraw, t.tail_v, nullptr, 1.0f, nullptr};
    hipLaunchKernelGGL((append_kernel<false, APPEND_TAIL, VAR_PLAIN>), grid, dim3(256), 0, s, c, src, t_k, page_table,
                       max_pages, nullptr);
    return hipGetLastError();
}

}  // namespace dqk
