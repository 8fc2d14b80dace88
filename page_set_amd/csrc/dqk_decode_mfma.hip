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

#include <utility>

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

// ---------------------------------------------------------------- staging through LDS
// Direct global -> LDS loads (16 or 4 bytes per lane, written at M0 + lane * size).
// They are issued from asm so that the compiler's conservative wait-for-all
// before every LDS read does not apply; completion is awaited explicitly with
// s_waitcnt vmcnt(N), N = DMA instructions this wave issued afterwards (any
// other vector memory op only makes that wait stricter).
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %0" ::"s"(sbase), "v"(voff), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_v(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4_v(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "s"(lds) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_dma() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that waits only for this wave's LDS operations.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

template <int KSM>
struct Lay {
    static constexpr int NCH = 8 * KSM;            // compacted channel slots
    static constexpr int KHR = 2 * NCH;            // 16-byte key half rows per page
    static constexpr int KPS = 32 * NCH + 32;      // key page stride: row groups of the 4 pages start 8 banks apart
    static constexpr int KINS = (KHR + 63) / 64;   // DMA instructions per key page
    static constexpr int KMI = (4 * NCH + 63) / 64;  // 4-byte DMA instructions for key metadata
    static constexpr int VBS = 32 * ROW_BYTES + 32;  // value block (32 tokens) stride, 8 banks apart
    static constexpr int VPS = 4 * VBS;
    static constexpr int OFF_K = 0;
    static constexpr int KAREA = 4 * KPS > 4 * GRP * PG * 2 ? 4 * KPS : 4 * GRP * PG * 2;  // key rows, later P
    static constexpr int OFF_KM = OFF_K + KAREA;       // u32 (scale | zero << 16) [4][NCH]
    static constexpr int OFF_K0 = OFF_KM + 16 * NCH;   // bf16 [4][128]
    static constexpr int OFF_VC = OFF_K0 + 4 * 256;    // value codes [4][4 blocks][32 rows][32 B]
    static constexpr int OFF_VM = OFF_VC + 4 * VPS;    // fp16 [4][2][4][128]
    static constexpr int QB = OFF_VM + 4 * 2048;       // one 4-page block
    static constexpr int NDMA = 4 * KINS + KMI + 1 + 16 + 8;
    static constexpr int NW = (NDMA + WAVES - 1) / WAVES;  // DMA instructions per wave per block
    static_assert(OFF_K0 % 16 == 0 && OFF_VC % 16 == 0 && OFF_VM % 16 == 0 && QB % 16 == 0, "alignment");
};

struct Quad {
    int64_t pg[4];  // physical page * hkv + g
    int nv[4];      // valid tokens (0 for slots past the range)
};

// Pages of logical pages lp0 .. lp0+3; slots past P1 reuse page lp0 (always valid).
__device__ __forceinline__ Quad quad_pages(const int32_t *__restrict__ ptab, int lp0, int P1, int L, int hkv, int g) {
    Quad q;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int lp = lp0 + p;
        const bool ok = lp < P1;
        q.pg[p] = (int64_t)ptab[ok ? lp : lp0] * hkv + g;
        q.nv[p] = ok ? min(PG, L - lp * PG) : 0;
    }
    return q;
}

__device__ __forceinline__ int64_t sel4l(const int64_t (&a)[4], int i) {
    const int64_t lo = (i & 1) ? a[1] : a[0];
    const int64_t hi = (i & 1) ? a[3] : a[2];
    return (i & 2) ? hi : lo;
}

// 16-byte chunks (row r of 4, chunk c of 16: tokens 8c .. 8c+7) of a 1 KB
// [4][128] fp16 table are stored at slot 16 (c & 3) + 4 (c >> 2) + r, so that
// the 16 chunks (r, 4G + k) read together for a k-step fall in distinct banks.
// LDS slot l of a DMA receives the chunk read from this byte offset:
__device__ __forceinline__ uint32_t vm_chunk(int l) {
    const int r = l & 3, c = 4 * ((l >> 2) & 3) + (l >> 4);
    return (uint32_t)(r * 256 + c * 16);
}
__device__ __forceinline__ constexpr int chunk_slot(int r, int c) { return 16 * (c & 3) + 4 * (c >> 2) + r; }

// One DMA instruction of a block fill; D_ is its compile-time index.
template <int KSM, int D_>
__device__ __forceinline__ void block_dma(const dqk_cache &c, const Quad &Q, uint32_t qb, int lane,
                                          const uint32_t (&kro)[Lay<KSM>::KINS],
                                          const uint32_t (&kmo)[Lay<KSM>::KMI], const int (&kmp)[Lay<KSM>::KMI]) {
    using Ly = Lay<KSM>;
    constexpr int NK = 4 * Ly::KINS, NKM = NK + Ly::KMI, NK0 = NKM + 1, NVC = NK0 + 16;
    constexpr int d = D_ < Ly::NDMA ? D_ : NKM;  // spare slots repeat the channel-0 load (same bytes)
    if constexpr (d < NK) {  // selected key rows of page p, 64 half rows per instruction
        constexpr int p = d / Ly::KINS, j = d % Ly::KINS;
        if (64 * j + lane < Ly::KHR)
            dma16_s(c.k_codes + Q.pg[p] * (D * ROW_BYTES), kro[j], qb + Ly::OFF_K + p * Ly::KPS + 64 * j * 16);
    } else if constexpr (d < NKM) {  // (scale, zero) of the selected channels of the 4 pages
        constexpr int t = d - NK;
        if (64 * t + lane < 4 * Ly::NCH)
            dma4_v(reinterpret_cast<const uint8_t *>(c.k_meta) + sel4l(Q.pg, kmp[t]) * (D * 4) + kmo[t],
                   qb + Ly::OFF_KM + 64 * t * 4);
    } else if constexpr (d < NK0) {  // channel 0 of the 4 pages
        dma16_v(reinterpret_cast<const uint8_t *>(c.k_ch0) + sel4l(Q.pg, lane >> 4) * (PG * 2) + (lane & 15) * 16,
                qb + Ly::OFF_K0);
    } else if constexpr (d < NVC) {  // value codes: page p, 32-token block bb
        constexpr int p = (d - NK0) >> 2, bb = (d - NK0) & 3;
        dma16_s(c.v_codes + Q.pg[p] * (PG * ROW_BYTES) + bb * 1024, (uint32_t)lane * 16u,
                qb + Ly::OFF_VC + p * Ly::VPS + bb * Ly::VBS);
    } else {  // value metadata: page p, half hf (scales / zeros), chunks permuted (see vm_chunk)
        constexpr int p = (d - NVC) >> 1, hf = (d - NVC) & 1;
        dma16_s(reinterpret_cast<const uint8_t *>(c.v_meta) + Q.pg[p] * (2 * VGROUPS * PG * 2) + hf * 1024,
                vm_chunk(lane), qb + Ly::OFF_VM + p * 2048 + hf * 1024);
    }
}

template <int KSM, int... Ds>
__device__ __forceinline__ void issue_all(const dqk_cache &c, const Quad &Q, uint32_t qb, int w, int lane,
                                          const uint32_t (&kro)[Lay<KSM>::KINS],
                                          const uint32_t (&kmo)[Lay<KSM>::KMI], const int (&kmp)[Lay<KSM>::KMI],
                                          std::integer_sequence<int, Ds...>) {
    ((w == (Ds & (WAVES - 1)) ? block_dma<KSM, Ds>(c, Q, qb, lane, kro, kmo, kmp) : (void)0), ...);
}

// Issue this wave's share (NW instructions) of the DMAs that fill one block buffer.
template <int KSM>
__device__ __forceinline__ void issue_block(const dqk_cache &c, const Quad &Q, uint32_t qb, int w, int lane,
                                            const uint32_t (&kro)[Lay<KSM>::KINS],
                                            const uint32_t (&kmo)[Lay<KSM>::KMI], const int (&kmp)[Lay<KSM>::KMI]) {
    issue_all<KSM>(c, Q, qb, w, lane, kro, kmo, kmp, std::make_integer_sequence<int, WAVES * Lay<KSM>::NW>{});
}

__device__ __forceinline__ uint32_t lds_u16(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t *>((uintptr_t)a);
}
__device__ __forceinline__ uint32_t lds_u32(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>((uintptr_t)a);
}
__device__ __forceinline__ u32x4 lds_u128(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((uintptr_t)a);
}
__device__ __forceinline__ void lds_st32(uint32_t a, uint32_t v) {
    *reinterpret_cast<__attribute__((address_space(3))) uint32_t *>((uintptr_t)a) = v;
}
__device__ __forceinline__ void lds_stf(uint32_t a, float v) {
    *reinterpret_cast<__attribute__((address_space(3))) float *>((uintptr_t)a) = v;
}
__device__ __forceinline__ float lds_f(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float *>((uintptr_t)a);
}

// Score tiles 2W, 2W+1 of one k-step (hi and lo halves of q~).
template <int W>
__device__ __forceinline__ void qk_step(f32x4 (&S)[2], const u32x4 &X, const half8 &Bh, const half8 &Bl) {
    Packed P;
    if (W == 0) P.L = X << 4;
    if (W == 2 || W == 3) P.R = X >> 6;
    P.X = X;
    const half8 a0 = as_half8(tile_codes<2 * W>(P));
    const half8 a1 = as_half8(tile_codes<2 * W + 1>(P));
    S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bh, S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bh, S[1], 0, 0, 0);
    S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bl, S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bl, S[1], 0, 0, 0);
}

template <int KSM>
__global__ __launch_bounds__(256) void decode_g4_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                        const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                        const int32_t *__restrict__ page_table, int max_pages,
                                                        const int32_t *__restrict__ seq_lens, float sm_scale,
                                                        int nsplit, float *__restrict__ partials) {
    using Ly = Lay<KSM>;
    constexpr int NCH = Ly::NCH;
    // two block buffers; the scores' probabilities reuse the key rows of the
    // current buffer once every wave is past its score MFMAs
    __shared__ __attribute__((aligned(16))) uint8_t blk[2][Ly::QB];
    __shared__ __attribute__((aligned(16))) _Float16 qt[2][4][GRP][NCH];  // q~ hi/lo [p][h][jj]
    __shared__ __attribute__((aligned(16))) float colmax[WAVES][16];
    __shared__ __attribute__((aligned(16))) float bias_lds[4][GRP];
    __shared__ __attribute__((aligned(16))) _Float16 zero16[8];
    static_assert(4 * GRP * PG * 2 <= Ly::KAREA, "probabilities fit in the key-row area");

    const int split = blockIdx.x, bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    const int b = bg / hkv, g = bg - b * hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform by construction
    const int G = lane >> 4, n = lane & 15;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    const int per = (((npages + nsplit - 1) / nsplit) + 15) & ~15;
    const int P0 = min(npages, split * per), P1 = min(npages, P0 + per);
    const int nq = (P1 - P0 + 3) >> 2;

    const float C = sm_scale * LOG2E;
    const int32_t *sel = sel_idx + ((size_t)b * hkv + g) * n_keep;
    const int has0 = sel[0] == 0;  // the list is ascending
    const int R = n_keep - has0;   // selected INT2 channels (R <= NCH)
    const int KS = (R + 7) >> 3;
    const float *qp = q_prime + ((size_t)b * hq + (size_t)g * GRP) * D;
    auto chan = [&](int jj) { return jj < R ? sel[jj + has0] : 0; };

    // per-lane DMA source offsets (fixed for the whole split)
    uint32_t kro[Ly::KINS];
#pragma unroll
    for (int j = 0; j < Ly::KINS; ++j) {
        const int hr = 64 * j + lane;
        kro[j] = hr < Ly::KHR ? (uint32_t)chan(hr >> 1) * ROW_BYTES + (hr & 1) * 16 : 0u;
    }
    uint32_t kmo[Ly::KMI];
    int kmp[Ly::KMI];
#pragma unroll
    for (int t = 0; t < Ly::KMI; ++t) {
        const int idx = min(64 * t + lane, 4 * NCH - 1);
        kmp[t] = idx / NCH;
        kmo[t] = (uint32_t)chan(idx - kmp[t] * NCH) * 4u;
    }
    // staging lane: channels 2*lane, 2*lane+1 of page slot w; C * q' of them for the 4 heads
    float qs[GRP][2];
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int jj = 2 * lane + e;
            qs[h][e] = jj < R ? qp[h * D + chan(jj)] * C : 0.0f;
        }
    const int pc = n >> 2, hc = n & 3;  // score lane: column (page slot, head)
    const int qv = n >> 2, hv = n & 3;  // value lane: row (group, head)
    const float q0c = has0 ? qp[hc * D] * C : 0.0f;
    if (tid < 8) zero16[tid] = (_Float16)0.0f;

    const uint32_t blk0 = lds_addr(&blk[0][0]);
    const int32_t *ptab = page_table + (size_t)b * max_pages;
    if (nq > 0) issue_block<KSM>(c, quad_pages(ptab, P0, P1, L, hkv, g), blk0, w, lane, kro, kmo, kmp);
    if (nq > 1) issue_block<KSM>(c, quad_pages(ptab, P0 + 4, P1, L, hkv, g), blk0 + Ly::QB, w, lane, kro, kmo, kmp);

    float m_lane = -__builtin_huge_valf();  // running max (log2 domain) of head n & 3
    float l_lane = 0.0f, z_lane = 0.0f;
    f32x4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = {0.f, 0.f, 0.f, 0.f};

    for (int u = 0; u < nq; ++u) {
        const uint32_t qb = blk0 + (uint32_t)(u & 1) * Ly::QB;
        if (u + 1 < nq)
            wait_dma<Ly::NW>();
        else
            wait_dma<0>();
        lds_barrier();

        // ---- stage q~ (fp16 hi/lo) for page slot w, channels 2 lane, 2 lane + 1; bias partials
        {
            float bp[GRP] = {0.f, 0.f, 0.f, 0.f};
            if (2 * lane < NCH) {
                const bool pv = P0 + 4 * u + w < P1;
                const uint32_t sz0 = lds_u32(qb + Ly::OFF_KM + (w * NCH + 2 * lane) * 4);
                const uint32_t sz1 = lds_u32(qb + Ly::OFF_KM + (w * NCH + 2 * lane + 1) * 4);
                const float s0 = pv ? h2f((uint16_t)sz0) : 0.f, z0 = pv ? h2f((uint16_t)(sz0 >> 16)) : 0.f;
                const float s1 = pv ? h2f((uint16_t)sz1) : 0.f, z1 = pv ? h2f((uint16_t)(sz1 >> 16)) : 0.f;
#pragma unroll
                for (int h = 0; h < GRP; ++h) {
                    const float t0 = qs[h][0] * s0, t1 = qs[h][1] * s1;
                    half2v hi, lo;
                    hi[0] = (_Float16)t0;
                    hi[1] = (_Float16)t1;
                    lo[0] = (_Float16)(t0 - (float)hi[0]);
                    lo[1] = (_Float16)(t1 - (float)hi[1]);
                    *reinterpret_cast<half2v *>(&qt[0][w][h][2 * lane]) = hi;
                    *reinterpret_cast<half2v *>(&qt[1][w][h][2 * lane]) = lo;
                    bp[h] = __builtin_fmaf(qs[h][1], z1, qs[h][0] * z0);
                }
            }
#pragma unroll
            for (int h = 0; h < GRP; ++h) {
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) bp[h] += __shfl_xor(bp[h], o);
            }
            if (lane == 0) {
#pragma unroll
                for (int h = 0; h < GRP; ++h) bias_lds[w][h] = bp[h];
            }
        }
        lds_barrier();

        // ---- scores: tiles 2w, 2w+1 of all 4 pages (block-diagonal over the page slots)
        f32x4 S[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        {
            const _Float16 *bhi = pc == G ? &qt[0][pc][hc][0] : &zero16[0];
            const _Float16 *blo = pc == G ? &qt[1][pc][hc][0] : &zero16[0];
            const int bstep = pc == G ? 8 : 0;
            const uint32_t krow = qb + Ly::OFF_K + G * Ly::KPS + 2 * n;
#pragma unroll
            for (int kk = 0; kk < KSM; ++kk) {
                if (kk < KS) {
                    const half8 Bh = *reinterpret_cast<const half8 *>(bhi + bstep * kk);
                    const half8 Bl = *reinterpret_cast<const half8 *>(blo + bstep * kk);
                    u32x4 X;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        X[e2] = lds_u16(krow + (8 * kk + 2 * e2) * ROW_BYTES) |
                                (lds_u16(krow + (8 * kk + 2 * e2 + 1) * ROW_BYTES) << 16);
                    switch (w) {
                        case 0: qk_step<0>(S, X, Bh, Bl); break;
                        case 1: qk_step<1>(S, X, Bh, Bl); break;
                        case 2: qk_step<2>(S, X, Bh, Bl); break;
                        default: qk_step<3>(S, X, Bh, Bl); break;
                    }
                }
            }
        }
        // ---- logits (log2 domain): tokens 32G + 8r + 2w + t of page slot pc, head hc
        const int lpc = P0 + 4 * u + pc;
        const int nvl = lpc < P1 ? min(PG, L - lpc * PG) : 0;
        const float bias = bias_lds[pc][hc];
        float x[2][4];
        {
            const float cmp0 = w == 0 ? tile_comp(0) : w == 1 ? tile_comp(2) : w == 2 ? tile_comp(4) : tile_comp(6);
            const float cmp1 = w == 0 ? tile_comp(1) : w == 1 ? tile_comp(3) : w == 2 ? tile_comp(5) : tile_comp(7);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 32 * G + 8 * r + 2 * w;
                const uint32_t k0p = has0 ? lds_u32(qb + Ly::OFF_K0 + (pc * PG + tok) * 2) : 0u;
                float v0 = __builtin_fmaf(S[0][r], cmp0, bias);
                float v1 = __builtin_fmaf(S[1][r], cmp1, bias);
                v0 = __builtin_fmaf(q0c, __uint_as_float(k0p << 16), v0);
                v1 = __builtin_fmaf(q0c, __uint_as_float(k0p & 0xFFFF0000u), v1);
                x[0][r] = tok < nvl ? v0 : -__builtin_huge_valf();
                x[1][r] = tok + 1 < nvl ? v1 : -__builtin_huge_valf();
            }
        }
        float xm = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        xm = fmaxf(xm, __shfl_xor(xm, 16));
        xm = fmaxf(xm, __shfl_xor(xm, 32));
        if (lane < 16) colmax[w][lane] = xm;
        lds_barrier();

        // ---- running max per head over the block (identical in every wave); each
        //      lane tracks the head n & 3 its score column and value row belong to
        float cm = lane < 16 ? fmaxf(fmaxf(colmax[0][n], colmax[1][n]), fmaxf(colmax[2][n], colmax[3][n]))
                             : -__builtin_huge_valf();
        cm = fmaxf(cm, __shfl_xor(cm, 4));
        cm = fmaxf(cm, __shfl_xor(cm, 8));  // lane h (< 4) holds the block max of head h
        const float m_new = fmaxf(m_lane, __shfl(cm, hc));
        const float alpha_lane = __builtin_amdgcn_exp2f(m_lane - m_new);
        if (__builtin_amdgcn_ballot_w64(m_new != m_lane)) {
            float alpha[GRP];
#pragma unroll
            for (int h = 0; h < GRP; ++h)
                alpha[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha_lane), h));
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[t][r] *= alpha[r];
            z_lane *= alpha_lane;
            l_lane *= alpha_lane;
        }
        m_lane = m_new;
        // probabilities to LDS (key-row area of this buffer): P[p][h][token] fp16
        {
            const float mh = m_lane;
            const uint32_t pbase = qb + Ly::OFF_K + pc * 1024;  // [p] 1 KB, chunks as in vm_chunk
            float ls = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pa = __builtin_amdgcn_exp2f(x[0][r] - mh);
                const float pb = __builtin_amdgcn_exp2f(x[1][r] - mh);
                ls += pa + pb;
                half2v hp;
                hp[0] = (_Float16)pa;
                hp[1] = (_Float16)pb;
                lds_st32(pbase + chunk_slot(hc, 4 * G + r) * 16 + 4 * w, as_u32(hp));
            }
            l_lane += ls;
        }
        lds_barrier();

        // ---- values of page slot w
        const int lpw = P0 + 4 * u + w;
        const int nvp = lpw < P1 ? min(PG, L - lpw * PG) : 0;
        if (nvp > 0) {
            const bool partial = nvp < PG;
            const uint32_t pb = qb + Ly::OFF_K + w * 1024 + chunk_slot(hv, 4 * G) * 16;   // + 256 per k-step
            const uint32_t sb = qb + Ly::OFF_VM + w * 2048 + chunk_slot(qv, 4 * G) * 16;
            const uint32_t vb = qb + Ly::OFF_VC + w * Ly::VPS + G * Ly::VBS + 2 * n;
            const half2v c15 = {(_Float16)1.5f, (_Float16)1.5f};
            const half2v m15 = {(_Float16)-1.5f, (_Float16)-1.5f};
#pragma unroll
            for (int kv = 0; kv < 4; ++kv) {
                u32x4 Pp = lds_u128(pb + 256 * kv);
                u32x4 sp = lds_u128(sb + 256 * kv);
                u32x4 zp = lds_u128(sb + 1024 + 256 * kv);
                if (partial) {
                    const int tok0 = 32 * G + 8 * kv;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const uint32_t keep = (tok0 + 2 * e2 < nvp ? 0x0000FFFFu : 0u) |
                                              (tok0 + 2 * e2 + 1 < nvp ? 0xFFFF0000u : 0u);
                        sp[e2] &= keep;
                        zp[e2] &= keep;
                        Pp[e2] &= keep;
                    }
                }
                u32x4 A;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const half2v a2 = as_half2(Pp[e2]) * as_half2(sp[e2]);
                    A[e2] = as_u32(a2);
                    // centred codes: v = (c - 1.5) s + (z + 1.5 s)
                    const half2v zc = __builtin_elementwise_fma(as_half2(sp[e2]), c15, as_half2(zp[e2]));
                    z_lane = __builtin_amdgcn_fdot2(as_half2(Pp[e2]), zc, z_lane, false);
                    z_lane = __builtin_amdgcn_fdot2(a2, m15, z_lane, false);
                }
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    X[e2] = lds_u16(vb + (8 * kv + 2 * e2) * ROW_BYTES) |
                            (lds_u16(vb + (8 * kv + 2 * e2 + 1) * ROW_BYTES) << 16);
                const half8 Ah = as_half8(A);
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
        lds_barrier();  // every wave is done with this buffer
        if (u + 2 < nq)
            issue_block<KSM>(c, quad_pages(ptab, P0 + 4 * (u + 2), P1, L, hkv, g), qb, w, lane, kro, kmo, kmp);
    }

    // ---- totals: each wave holds page slot w's value sums; all share m_run
    wait_dma<0>();
    l_lane += __shfl_xor(l_lane, 4);
    l_lane += __shfl_xor(l_lane, 8);
    l_lane += __shfl_xor(l_lane, 16);
    l_lane += __shfl_xor(l_lane, 32);  // lanes with hc = h: this wave's share of l of head h
    z_lane += __shfl_xor(z_lane, 16);
    z_lane += __shfl_xor(z_lane, 32);  // lane (., 4q + h): zero-point term of (q, h)
    float zq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) zq[r] = __shfl(z_lane, 16 * G + 4 * G + r);  // (q = G, h = r)
    float m_fin[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) m_fin[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_lane), h));
    float *comb = reinterpret_cast<float *>(&blk[0][0]);  // [WAVES][GRP][D + 1]
    lds_barrier();
    if ((n >> 2) == G) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                comb[(w * GRP + r) * (D + 1) + 8 * n + t] = __builtin_fmaf(O[t][r], tile_comp(t), zq[r]);
    }
    if (lane < GRP) comb[(w * GRP + lane) * (D + 1) + D] = l_lane;
    lds_barrier();
    for (int i = tid; i < GRP * D; i += 256) {
        const int h = i >> 7, ch = i & (D - 1);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) {
            acc += comb[(ww * GRP + h) * (D + 1) + ch];
            lsum += comb[(ww * GRP + h) * (D + 1) + D];
        }
        float *dst = partials + (((size_t)b * hq + (size_t)g * GRP + h) * nsplit + split) * PART_FLOATS;
        dst[ch] = nq > 0 ? acc : 0.0f;
        if (ch == 0) {
            dst[D] = nq > 0 ? m_fin[h] * LN2 : -__builtin_huge_valf();
            dst[D + 1] = nq > 0 ? lsum : 0.0f;
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

template <int KSM>
static hipError_t launch_ksm(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_g4_kernel<KSM>, grid, dim3(256), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    // key k-steps of 8 channels needed for n_keep selected channels
    const int ks = (a.n_keep + 7) / 8;
    if (ks <= 2) return launch_ksm<2>(a, s);
    if (ks <= 4) return launch_ksm<4>(a, s);
    if (ks <= 7) return launch_ksm<7>(a, s);
    if (ks <= 10) return launch_ksm<10>(a, s);
    if (ks <= 13) return launch_ksm<13>(a, s);
    return launch_ksm<16>(a, s);
}

}  // namespace dqk
