// Decode attention over the paged INT2 cache for 4 query heads per KV head
// (GQA 32/8-style), on MFMA (Dual-QK paper: masked scores over the selected
// channels with the full 1/sqrt(d) scale, §3.2; channel 0 from its bf16
// copy, INT2 channel-major key rows and token-major values, §3.3; one
// softmax over the context, §3.4).
//
// Every wave works on its own: a workgroup is one wave, which streams the
// page pairs of its split through two LDS stages filled by direct
// global -> LDS loads, keeps its own online softmax and writes one partial
// (no workgroup barriers anywhere).  Per page pair:
//
//  * Scores on v_mfma_f32_16x16x32_f16, block-diagonal over the two pages:
//    the 32-deep k dimension is (page, 16 selected channels), the 16 columns
//    are (page, head, limb), where the two limbs are the fp16 hi and lo parts
//    of q~ = log2(e)/sqrt(d) * q' * scale_j, so one MFMA yields both and a
//    DPP add of the neighbouring column joins them.  Token tile m, row i
//    holds token 8i + m: lane i reads the 16-bit word i of each selected
//    32-byte key row.  The zero points fold into one bias per (page, head).
//  * 2-bit codes enter MFMA as binary16 subnormals: one AND of a (possibly
//    shifted) packed word gives code * 2^(offset - 24) exactly for two codes
//    at once; the power of two is undone per tile after the MFMA.
//  * Online softmax in the log2 domain; the two lanes of a column pair
//    (the two limbs) split the 8 token tiles between them.
//  * Values: per page, O[(group q, head h)][channel] += (P*scale_q)[.][token]
//    x codes[token][channel] on MFMA (M = 4 groups x 4 heads); P moves to the
//    operand layout through LDS; the zero points (as sum_t P (z + 1.5 s) -
//    1.5 sum_t P s, centred codes) and the softmax denominator sum_t P
//    accumulate on two more MFMAs per 32 tokens.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int GRP = 4;  // query heads per KV head handled here
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

// ---------------------------------------------------------------- LDS access
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
__device__ __forceinline__ uint32_t lds_u16(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t *>((uintptr_t)a);
}
__device__ __forceinline__ u32x2 lds_u64(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x2 *>((uintptr_t)a);
}
__device__ __forceinline__ u32x4 lds_u128(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((uintptr_t)a);
}
__device__ __forceinline__ void lds_st64(uint32_t a, u32x2 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x2 *>((uintptr_t)a) = v;
}
// Two 16-bit LDS words -> one dword (lo, hi).
__device__ __forceinline__ uint32_t lds_pair(uint32_t a_lo, uint32_t a_hi) {
    return __builtin_amdgcn_perm(lds_u16(a_hi), lds_u16(a_lo), 0x05040100u);
}

// ---------------------------------------------------------------- direct global -> LDS loads
// 16 or 4 bytes per lane, written at M0 + lane * size.  Issued from asm so
// that the compiler's conservative wait-for-all before every LDS read does
// not apply; completion is awaited explicitly with s_waitcnt vmcnt(N), N =
// vector memory instructions this wave issued afterwards (any other vector
// memory op only makes that wait stricter).
// sbase must be wave-uniform (it is moved into SGPRs).
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds) {
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %0" ::"s"((const void *)(uintptr_t)u), "v"(voff),
                 "s"(lds)
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

// ---------------------------------------------------------------- cross-lane moves
__device__ __forceinline__ float bcast_lane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float dpp_xor1(float v) {  // quad_perm [1, 0, 3, 2]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor8(float v) {  // row_ror:8 within 16 lanes
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}
// v_permlane16_swap with both operands v leaves (row 0, row 0, row 2, row 2) in
// the first result and (row 1, row 1, row 3, row 3) in the second (rows of 16
// lanes); v_permlane32_swap does the same for the two halves.  Combining the
// two results reduces over lane ^ 16 (lane ^ 32), identically in both lanes.
__device__ __forceinline__ float sum_x16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------- stage layout
// Two stages per wave.  Stage u & 1 holds the keys of page pair u (needed by
// its scores) and the values of pair u (needed one step later, by its value
// products), so keys of pair u + 2 and values of pair u + 1 can be loaded
// while pair u is scored.  Key rows: 16 KS row slots per page (the selected
// INT2 channels in ascending order, padded with the all-zero row 0), slot s
// holding row s ^ ((s >> 3) & 1), page 1 starting 64 bytes later modulo 256,
// so that the four rows one k-step reads at a time fall in distinct banks.
template <int KS>
struct Stage {
    static constexpr int NR = 16 * KS;                  // key row slots per page
    static constexpr int KRP = NR * ROW_BYTES + 64;     // key page stride
    static constexpr int OFF_KM = 2 * KRP;              // (scale | zero << 16) [2][NR]
    static constexpr int OFF_K0 = OFF_KM + 2 * NR * 4;  // channel 0, bf16 [2][128]
    static constexpr int VBS = 32 * ROW_BYTES + 32;     // value block (32 tokens) stride
    static constexpr int VPS = 4 * VBS;                 // value page stride
    static constexpr int OFF_VC = OFF_K0 + 2 * PG * 2;  // value codes [2][4][32][32 B]
    static constexpr int OFF_VM = OFF_VC + 2 * VPS;     // value (scale, zero) [2][2][4][128]
    static constexpr int BYTES = OFF_VM + 2 * 2048;
    static constexpr int KRI = (2 * NR + 63) / 64;  // 16-byte key-row DMAs per page
    static constexpr int KMI = (2 * NR + 63) / 64;  // 4-byte key-metadata DMAs for the pair
    static constexpr int KN = 2 * KRI + KMI + 1;    // key DMAs of a pair
    static constexpr int VN = 8 + 4;                // value DMAs of a pair
    static_assert(OFF_KM % 16 == 0 && OFF_K0 % 16 == 0 && OFF_VC % 16 == 0 && OFF_VM % 16 == 0 &&
                      BYTES % 16 == 0,
                  "alignment");
    static_assert(2 * (KN + VN) <= 63, "vmcnt range");
};

struct Pair {
    int64_t pg0, pg1;  // physical page * hkv + g of the two slots (slot 1 repeats slot 0 when absent)
};

__device__ __forceinline__ Pair pair_pages(const int32_t *__restrict__ ptab, int lp0, int P1, int hkv, int g) {
    Pair p;
    p.pg0 = (int64_t)ptab[lp0] * hkv + g;
    p.pg1 = lp0 + 1 < P1 ? (int64_t)ptab[lp0 + 1] * hkv + g : p.pg0;
    return p;
}

// Per-lane DMA source offsets, fixed for the whole split.
template <int KS>
struct DmaPlan {
    uint32_t kro[Stage<KS>::KRI];  // key half-row source offsets within a page
    uint32_t kmo[Stage<KS>::KMI];  // key metadata offsets within a page
    uint32_t kmp;                  // bit t: key-metadata DMA t reads page slot 1
    uint32_t vmo;                  // value metadata chunk offset (permuted, see the plan)
};

// Keys of a page pair into stage st: exactly Stage<KS>::KN vector memory
// instructions, each with at least lane 0 active.
template <int KS>
__device__ __forceinline__ void issue_keys(const dqk_cache &c, const Pair &pr, uint32_t st, int lane,
                                           const DmaPlan<KS> &pl) {
    using S = Stage<KS>;
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // key rows, 64 half rows per instruction
        const uint8_t *base = c.k_codes + (p ? pr.pg1 : pr.pg0) * (D * ROW_BYTES);
#pragma unroll
        for (int j = 0; j < S::KRI; ++j)
            if (64 * j + lane < 2 * S::NR) dma16_s(base, pl.kro[j], st + p * S::KRP + 64 * j * 16);
    }
    // (scale, zero) of the selected channels, both pages
    const uint8_t *km0 = reinterpret_cast<const uint8_t *>(c.k_meta) + pr.pg0 * (D * 4);
    const uint8_t *km1 = reinterpret_cast<const uint8_t *>(c.k_meta) + pr.pg1 * (D * 4);
#pragma unroll
    for (int t = 0; t < S::KMI; ++t)
        if (64 * t + lane < 2 * S::NR) dma4_v(((pl.kmp >> t) & 1u ? km1 : km0) + pl.kmo[t], st + S::OFF_KM + 64 * t * 4);
    if (lane < 32) {  // channel 0 of both pages (32 lanes x 16 bytes)
        const uint8_t *k0 = reinterpret_cast<const uint8_t *>(c.k_ch0) + (lane < 16 ? pr.pg0 : pr.pg1) * (PG * 2);
        dma16_v(k0 + (lane & 15) * 16, st + S::OFF_K0);
    }
}

// Values of a page pair into stage st: exactly Stage<KS>::VN instructions.
template <int KS>
__device__ __forceinline__ void issue_vals(const dqk_cache &c, const Pair &pr, uint32_t st, int lane,
                                           const DmaPlan<KS> &pl) {
    using S = Stage<KS>;
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // value codes: page p, 32-token block bb
        const uint8_t *base = c.v_codes + (p ? pr.pg1 : pr.pg0) * (PG * ROW_BYTES);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
            dma16_s(base + bb * 1024, (uint32_t)lane * 16u, st + S::OFF_VC + p * S::VPS + bb * S::VBS);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // value metadata: page p, half hf (scales, zeros)
        const uint8_t *base =
            reinterpret_cast<const uint8_t *>(c.v_meta) + (p ? pr.pg1 : pr.pg0) * (2 * VGROUPS * PG * 2);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) dma16_s(base + hf * 1024, pl.vmo, st + S::OFF_VM + p * 2048 + hf * 1024);
    }
}

// ---------------------------------------------------------------- per-lane constants
template <int KS>
struct Lane {
    // score lanes: k range = page G >> 1, channels 16 ks + 8 (G & 1) + 0..7;
    // column n = (page pp, head hh, limb ll)
    int pp, hh, ll;
    uint32_t QH[KS][4], QL[KS][4];  // C q' fp16 pairs: limb-1 lanes (hi, lo), limb-0 lanes (0, hi)
    float q0c;                      // C q'_0 (0 when channel 0 is pruned)
    float comp[4];                  // tiles 4 ll + j after the limb split
    uint32_t kr_even, kr_odd, km, k0;
    uint32_t pw[4];  // P writes
    // value lanes: row (q, h) = (n >> 2, n & 3), tokens 32 G + 8 kv + 0..7
    uint32_t pr_ofs[4], vm_ofs[4], vc;
    half2v zc_s, zc_z, zc_c;
    half8 M15;
};

// One score k-step: 16 selected channels of each page of the pair.
template <int KS>
__device__ __forceinline__ void qk_step(int ks, uint32_t st, const Lane<KS> &ln, f32x4 (&Sc)[8], f32x4 &Sb) {
    const u32x4 d0 = lds_u128(st + ln.km + 64 * ks);
    const u32x4 d1 = lds_u128(st + ln.km + 64 * ks + 16);
    const uint32_t dd[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    u32x4 Bv, Zv, QLv;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        const half2v s2 = as_half2(__builtin_amdgcn_perm(dd[2 * e2 + 1], dd[2 * e2], 0x05040100u));
        Zv[e2] = __builtin_amdgcn_perm(dd[2 * e2 + 1], dd[2 * e2], 0x07060302u);
        const half2v qh = as_half2(ln.QH[ks][e2]), ql = as_half2(ln.QL[ks][e2]);
        const half2v t1 = qh * s2;
        const half2v t2 = __builtin_elementwise_fma(qh, s2, -t1);
        Bv[e2] = as_u32(__builtin_elementwise_fma(ql, s2, t2));
        QLv[e2] = ln.QL[ks][e2];
    }
    const half8 Bh = as_half8(Bv);
    // rows of A all equal z_k (k = this lane's channels), B = the lane's limb of C q'
    Sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(Zv), as_half8(QLv), Sb, 0, 0, 0);
    u32x4 X;
    const uint32_t kb = st + 16 * ks * ROW_BYTES;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) X[e2] = lds_pair(kb + ln.kr_even + 64 * e2, kb + ln.kr_odd + 64 * e2 + ROW_BYTES);
    const Packed XP = pack_shifts(X);
    Sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<0>(XP)), Bh, Sc[0], 0, 0, 0);
    Sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<1>(XP)), Bh, Sc[1], 0, 0, 0);
    Sc[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<2>(XP)), Bh, Sc[2], 0, 0, 0);
    Sc[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<3>(XP)), Bh, Sc[3], 0, 0, 0);
    Sc[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<4>(XP)), Bh, Sc[4], 0, 0, 0);
    Sc[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<5>(XP)), Bh, Sc[5], 0, 0, 0);
    Sc[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<6>(XP)), Bh, Sc[6], 0, 0, 0);
    Sc[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(tile_codes<7>(XP)), Bh, Sc[7], 0, 0, 0);
}

// One value step: 32 tokens (32 G + 8 kv + 0..7) of page vp; P from pbase.
template <int KS>
__device__ __forceinline__ void pv_step(int vp, int kv, uint32_t st, uint32_t pbase, const Lane<KS> &ln,
                                        f32x4 (&O)[8], f32x4 &Oz) {
    using S = Stage<KS>;
    const u32x4 Pp = lds_u128(pbase + vp * 1024 + ln.pr_ofs[kv]);
    const u32x4 sp = lds_u128(st + vp * 2048 + ln.vm_ofs[kv]);
    const u32x4 zp = lds_u128(st + vp * 2048 + ln.vm_ofs[kv] + 1024);
    // centred codes: v = (c - 1.5) s + (z + 1.5 s)
    u32x4 A, Bz;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        A[e2] = as_u32(as_half2(Pp[e2]) * as_half2(sp[e2]));
        Bz[e2] = as_u32(__builtin_elementwise_fma(as_half2(sp[e2]), ln.zc_s,
                                                  __builtin_elementwise_fma(as_half2(zp[e2]), ln.zc_z, ln.zc_c)));
    }
    u32x4 X;
    const uint32_t vb = st + ln.vc + vp * S::VPS + 8 * kv * ROW_BYTES;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) X[e2] = lds_pair(vb + 64 * e2, vb + 64 * e2 + ROW_BYTES);
    const half8 Ah = as_half8(A);
    Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(Pp), as_half8(Bz), Oz, 0, 0, 0);
    Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, ln.M15, Oz, 0, 0, 0);
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

// Value scales and zero points of tokens at or past nv (0 <= nv < 128) of a page
// set to zero, so that unspecified bytes past the end of a sequence cannot
// reach the products (their probabilities are already zero).
__device__ __forceinline__ void clear_tail_meta(uint32_t vm_page, int nv, int lane) {
    // entry (hf, q, t) of the page sits in chunk t >> 3 of group q, at slot (t >> 3) ^ q
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = 64 * i + lane;  // 1024 entries: hf (1), q (2), t (7)
        const int hf = e >> 9, q = (e >> 7) & 3, t = e & 127;
        if (t >= nv) {
            const uint32_t a = vm_page + hf * 1024 + q * 256 + 16 * ((t >> 3) ^ q) + 2 * (t & 7);
            *reinterpret_cast<__attribute__((address_space(3))) uint16_t *>((uintptr_t)a) = 0;
        }
    }
}

template <int KS>
__global__ __launch_bounds__(64) void decode_g4_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                       const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                       const int32_t *__restrict__ page_table, int max_pages,
                                                       const int32_t *__restrict__ seq_lens, float sm_scale,
                                                       int nsplit, float *__restrict__ partials) {
    using S = Stage<KS>;
    constexpr int NR = S::NR;
    __shared__ __attribute__((aligned(16))) uint8_t stg[2][S::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * GRP * PG * 2];  // P [2][4][128] fp16

    const int split = blockIdx.x, bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    const int b = bg / hkv, g = bg - b * hkv;
    const int lane = threadIdx.x;
    const int G = lane >> 4, n = lane & 15;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    const int per = (((npages + nsplit - 1) / nsplit) + 1) & ~1;
    const int P0 = min(npages, split * per), P1 = min(npages, P0 + per);
    const int npairs = (P1 - P0 + 1) >> 1;
    const int32_t *ptab = page_table + (size_t)b * max_pages;
    const uint32_t st0 = lds_addr(&stg[0][0]);
    const uint32_t pb = lds_addr(&pbuf[0]);
    auto stage = [&](int u) { return st0 + (uint32_t)(u & 1) * S::BYTES; };
    auto nvalid = [&](int lp) { return lp < P1 ? min(PG, L - lp * PG) : 0; };

    DmaPlan<KS> pl;
    // value metadata: LDS slot l of each 1 KB half holds chunk (l & 15) ^ (l >> 4) of group l >> 4
    pl.vmo = (uint32_t)((lane >> 4) * 256 + 16 * ((lane & 15) ^ (lane >> 4)));
    // values of pair 0 do not depend on the selection: in flight first
    Pair pr_v = {0, 0};  // pages whose values load next
    if (npairs > 0) {
        pr_v = pair_pages(ptab, P0, P1, hkv, g);
        issue_vals<KS>(c, pr_v, stage(0), lane, pl);
    }

    const float C = sm_scale * LOG2E;
    static_assert(GRP * D * 4 + D * 4 <= S::BYTES, "q' and the selection fit in one stage");
    // q' of the 4 heads and the selected channels go through LDS (stage 1, before its
    // first fill) with one round of loads
    {
        const float4 *qsrc = reinterpret_cast<const float4 *>(q_prime + ((size_t)b * hq + (size_t)g * GRP) * D);
        const int32_t *ssrc = sel_idx + ((size_t)b * hkv + g) * n_keep;
        const float4 qa = qsrc[lane], qb = qsrc[lane + 64];
        const int sa = ssrc[min(lane, n_keep - 1)], sb = ssrc[min(lane + 64, n_keep - 1)];
        float4 *qd = reinterpret_cast<float4 *>(&stg[1][0]);
        int32_t *sd = reinterpret_cast<int32_t *>(&stg[1][GRP * D * 4]);
        qd[lane] = qa;
        qd[lane + 64] = qb;
        sd[lane] = sa;
        sd[lane + 64] = sb;
    }
    __syncthreads();
    const float *q_l = reinterpret_cast<const float *>(&stg[1][0]);                  // [4][128]
    const int32_t *sel_l = reinterpret_cast<const int32_t *>(&stg[1][GRP * D * 4]);  // [n_keep]
    const int has0 = sel_l[0] == 0;  // the list is ascending
    const int R = n_keep - has0;     // selected INT2 channels (R <= NR)
    // selected INT2 channel of key row r; rows past R read the all-zero row 0
    auto chan = [&](int r) {
        const int v = sel_l[min(r + has0, n_keep - 1)];
        return r < R ? v : 0;
    };

    // ---- key DMA plan
#pragma unroll
    for (int j = 0; j < S::KRI; ++j) {
        const int x = 64 * j + lane, s = x >> 1;
        const int r = s ^ ((s >> 3) & 1);
        pl.kro[j] = x < 2 * NR ? (uint32_t)chan(r) * ROW_BYTES + (x & 1) * 16 : 0u;
    }
    pl.kmp = 0;
#pragma unroll
    for (int t = 0; t < S::KMI; ++t) {
        const int x = min(64 * t + lane, 2 * NR - 1);
        const int p = x >= NR;
        pl.kmp |= (uint32_t)p << t;
        pl.kmo[t] = (uint32_t)chan(x - p * NR) * 4u;
    }

    // ---- per-lane constants
    Lane<KS> ln;
    ln.pp = n >> 3;
    ln.hh = (n >> 1) & 3;
    ln.ll = n & 1;
    const int kpage = G >> 1, kh = G & 1;
    // limb-1 lanes hold (hi, lo), limb-0 lanes (0, hi), so fma(QL, s, fma(QH, s, -QH s))
    // is the lane's limb of C q' s either way
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            half2v h, l;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int jj = 16 * ks + 8 * kh + 2 * e2 + u;
                const float qj = q_l[ln.hh * D + chan(jj)];
                const float v = (ln.pp == kpage && jj < R) ? qj * C : 0.0f;
                const _Float16 vh = (_Float16)v;
                const _Float16 vl = (_Float16)(v - (float)vh);
                h[u] = ln.ll ? vh : (_Float16)0.0f;
                l[u] = ln.ll ? vl : vh;
            }
            ln.QH[ks][e2] = as_u32(h);
            ln.QL[ks][e2] = as_u32(l);
        }
    {
        const float q0 = q_l[ln.hh * D];
        ln.q0c = has0 ? q0 * C : 0.0f;
    }
    // stage 1 is free again once every LDS read above has returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    Pair pr_k = {0, 0};  // pages whose keys load next
    if (npairs > 0) issue_keys<KS>(c, pr_v, stage(0), lane, pl);
    if (npairs > 1) {
        pr_k = pair_pages(ptab, P0 + 2, P1, hkv, g);
        issue_keys<KS>(c, pr_k, stage(1), lane, pl);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ln.comp[j] = ln.ll ? tile_comp(4 + j) : tile_comp(j);
    // key row 16 ks + 8 kh + e sits in slot 16 ks + 8 kh + (e ^ kh)
    ln.kr_even = kpage * S::KRP + (9 * kh) * ROW_BYTES + 2 * n;  // e even: slot e + kh
    ln.kr_odd = kpage * S::KRP + (7 * kh) * ROW_BYTES + 2 * n;   // e odd: slot e - kh
    ln.km = S::OFF_KM + (kpage * NR + 8 * kh) * 4;
    ln.k0 = S::OFF_K0 + ln.pp * 256 + 64 * G + 8 * ln.ll;
#pragma unroll
    for (int r = 0; r < 4; ++r)  // chunk 4G + r of (pp, hh) at slot (4G + r) ^ hh, half ll
        ln.pw[r] = ln.pp * 1024 + ln.hh * 256 + 16 * ((4 * G + r) ^ ln.hh) + 8 * ln.ll;
    const int qv = n >> 2, hv = n & 3;
#pragma unroll
    for (int kv = 0; kv < 4; ++kv) {
        ln.pr_ofs[kv] = hv * 256 + 16 * ((4 * G + kv) ^ hv);
        ln.vm_ofs[kv] = S::OFF_VM + qv * 256 + 16 * ((4 * G + kv) ^ qv);
    }
    ln.vc = S::OFF_VC + G * S::VBS + 2 * n;
    // zero-point MFMA B operand: z + 1.5 s of group n >> 2 in columns 4q (its row
    // (q, h) sum is sum_t P (z + 1.5 s)), 1 in columns 4q + 1 (sum_t P, the softmax
    // denominator), 0 elsewhere; -1.5 in columns 4q of the second one adds -1.5 sum_t P s
    {
        const int zcol = n & 3;
        const _Float16 a = (_Float16)(zcol == 0 ? 1.5f : 0.f), o = (_Float16)(zcol == 0 ? 1.f : 0.f);
        const _Float16 cc = (_Float16)(zcol == 1 ? 1.f : 0.f), m = (_Float16)(zcol == 0 ? -1.5f : 0.f);
        ln.zc_s = half2v{a, a};
        ln.zc_z = half2v{o, o};
        ln.zc_c = half2v{cc, cc};
        ln.M15 = half8{m, m, m, m, m, m, m, m};
    }

    float m_run = -__builtin_huge_valf();  // running max (log2 domain) of head hh
    f32x4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = {0.f, 0.f, 0.f, 0.f};
    f32x4 Oz = {0.f, 0.f, 0.f, 0.f};  // zero-point terms (columns 4q) and denominators (4q + 1)

    // Step u scores pair u (u < npairs) and multiplies the values of pair u - 1
    // (u >= 1).  At its start the loads issued two steps back have to be
    // complete: keys of pair u and values of pair u - 1.
    int issued = 0;  // vector memory instructions issued by the previous step
    if (npairs > 1) issued = S::KN;  // keys of pair 1 behind those of pair 0
    for (int u = 0; u <= npairs; ++u) {
        if (issued == S::KN + S::VN)
            wait_dma<S::KN + S::VN>();
        else if (issued == S::KN)
            wait_dma<S::KN>();
        else if (issued == S::VN)
            wait_dma<S::VN>();
        else
            wait_dma<0>();
        const bool score = u < npairs, mult = u >= 1;
        const uint32_t stq = stage(u), stv = stage(u - 1);
        if (mult) {  // unspecified metadata past the end of a sequence must not reach the products
            const int lp = P0 + 2 * (u - 1);
            const int v0 = nvalid(lp), v1 = nvalid(lp + 1);
            if (v0 < PG) clear_tail_meta(stv + S::OFF_VM, v0, lane);
            if (v1 < PG) clear_tail_meta(stv + S::OFF_VM + 2048, v1, lane);  // an absent page too
        }
        // next loads: keys of pair u + 2 (into this stage, once scored), values of
        // pair u + 1 (into the other stage, once multiplied)
        const bool ld_k = u + 2 < npairs, ld_v = u + 1 < npairs;
        Pair nk = {0, 0}, nv = {0, 0};
        if (ld_k) nk = pair_pages(ptab, P0 + 2 * (u + 2), P1, hkv, g);
        if (ld_v) nv = pr_k;  // keys of pair u + 1 were loaded last step with these pages

        // channel 0 of pair u, read before this stage's key area is refilled below
        u32x2 k0v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) k0v[r] = score ? lds_u64(stq + ln.k0 + 16 * r) : u32x2{0u, 0u};
        f32x4 Sc[8], Sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 8; ++t) Sc[t] = {0.f, 0.f, 0.f, 0.f};
        if (score && mult) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                pv_step<KS>(i >> 2, i & 3, stv, pb, ln, O, Oz);
                if (i < KS) qk_step<KS>(i, stq, ln, Sc, Sb);
            }
        } else if (score) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qk_step<KS>(ks, stq, ln, Sc, Sb);
        } else if (mult) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pv_step<KS>(i >> 2, i & 3, stv, pb, ln, O, Oz);
        }
        // every LDS read of the two stages has returned: refill them
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issued = 0;
        if (ld_k) {
            issue_keys<KS>(c, nk, stq, lane, pl);
            issued += S::KN;
        }
        if (ld_v) {
            issue_vals<KS>(c, nv, stage(u + 1), lane, pl);
            issued += S::VN;
        }
        if (ld_k) pr_k = nk;
        if (!score) break;

        // ---- logits (log2 domain) of pair u: lane keeps tiles 4 ll + j of its
        //      column, rows r: token 32 G + 8 r + 4 ll + j of page pp, head hh
        const int lp0 = P0 + 2 * u;
        const int nv0 = nvalid(lp0), nv1 = nvalid(lp0 + 1);
        const float bias = Sb[0] + dpp_xor1(Sb[0]);  // both limbs
        const uint32_t llmask = ln.ll ? 0xFFFFFFFFu : 0u;
        float x[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u32x2 k0 = k0v[r];  // q0c = 0 when channel 0 is pruned
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // bitwise selects: a conditional pick between the two tiles would be
                // turned into an indexed access of the accumulator array
                const uint32_t lo = __float_as_uint(Sc[j][r]), hi = __float_as_uint(Sc[4 + j][r]);
                const float mine = __uint_as_float((hi & llmask) | (lo & ~llmask));
                const float give = __uint_as_float((lo & llmask) | (hi & ~llmask));
                float v = __builtin_fmaf(mine + dpp_xor1(give), ln.comp[j], bias);
                const uint32_t kw = k0[j >> 1];
                v = __builtin_fmaf(ln.q0c, __uint_as_float((j & 1) ? (kw & 0xFFFF0000u) : (kw << 16)), v);
                x[r][j] = v;
            }
        }
        if (nv0 < PG || nv1 < PG) {
            const int nvp = ln.pp ? nv1 : nv0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (32 * G + 8 * r + 4 * ln.ll + j >= nvp) x[r][j] = -__builtin_huge_valf();
        }
        // ---- running max of head hh over the pair
        float bm = -__builtin_huge_valf();
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, fmaxf(fmaxf(x[r][0], x[r][1]), fmaxf(x[r][2], x[r][3])));
        bm = fmaxf(bm, dpp_xor1(bm));
        bm = fmaxf(bm, dpp_xor8(bm));
        bm = max_x32(max_x16(bm));
        const float m_new = fmaxf(m_run, bm);
        if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {  // O already holds pair u - 1
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // head hh
            float a[GRP];
#pragma unroll
            for (int h = 0; h < GRP; ++h) a[h] = bcast_lane(alpha, 2 * h);  // lane 2h: column (0, h, 0)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[t][r] *= a[r];
#pragma unroll
            for (int r = 0; r < 4; ++r) Oz[r] *= a[r];
        }
        m_run = m_new;
        // ---- probabilities -> fp16 -> LDS (read by the next step's value products)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[r][j] - m_new);
            half2v h01, h23;
            h01[0] = (_Float16)p[0];
            h01[1] = (_Float16)p[1];
            h23[0] = (_Float16)p[2];
            h23[1] = (_Float16)p[3];
            lds_st64(pb + ln.pw[r], u32x2{as_u32(h01), as_u32(h23)});
        }
    }
    wait_dma<0>();

    // ---- totals: row (q = G, h = r) of Oz holds the zero-point term in column 4G
    //      (broadcast over the quad of lanes 4G..4G+3) and l_h in column 4q + 1
    float zq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        zq[r] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Oz[r]), 0x00, 0xF, 0xF, false));
    float l_h[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) l_h[h] = bcast_lane(Oz[h], 1);  // lane 1: column 1, rows (0, h)
    float *dst0 = partials + (((size_t)b * hq + (size_t)g * GRP) * nsplit + split) * PART_FLOATS;
    const size_t hstride = (size_t)nsplit * PART_FLOATS;
    if ((n >> 2) == G) {  // channel 8n + t belongs to group q = G
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst0[r * hstride + 8 * n + t] = npairs > 0 ? __builtin_fmaf(O[t][r], tile_comp(t), zq[r]) : 0.0f;
    }
    if (lane < 8 && (lane & 1) == 0) {  // lane 2h: column (0, h, 0)
        const int h = lane >> 1;
        const float lh = (h & 2) ? ((h & 1) ? l_h[3] : l_h[2]) : ((h & 1) ? l_h[1] : l_h[0]);
        dst0[h * hstride + D] = npairs > 0 ? m_run * LN2 : -__builtin_huge_valf();
        dst0[h * hstride + D + 1] = npairs > 0 ? lh : 0.0f;
    }
}

}  // namespace

bool use_mfma_decode(int hq, int hkv) { return hkv > 0 && hq == GRP * hkv; }

template <int KS>
static constexpr int wave_lds_bytes() {
    return 2 * Stage<KS>::BYTES + 2 * GRP * PG * 2;
}

int decode_splits_mfma(int batch, int hkv, int max_pages, int n_keep) {
    // enough single-wave workgroups to fill every CU once (256 CUs, as many
    // per CU as fit in 160 KB of LDS), at least 8 pages each; n_keep = 0 asks
    // for the largest count any n_keep can use (workspace sizing)
    static constexpr int lds[9] = {0,
                                   wave_lds_bytes<1>(), wave_lds_bytes<2>(), wave_lds_bytes<3>(), wave_lds_bytes<4>(),
                                   wave_lds_bytes<5>(), wave_lds_bytes<6>(), wave_lds_bytes<7>(), wave_lds_bytes<8>()};
    const int ks = n_keep > 0 ? (n_keep + 15) / 16 : 1;
    const int per_cu = (160 * 1024) / lds[ks < 1 ? 1 : ks > 8 ? 8 : ks];
    const int units = batch * hkv;
    int s = (256 * per_cu + units - 1) / units;
    const int cap = (max_pages + 7) / 8;
    if (s > cap) s = cap;
    return s < 1 ? 1 : s;
}

template <int KS>
static hipError_t launch_ks(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_g4_kernel<KS>, grid, dim3(64), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    // 16-channel k-steps per page for up to n_keep INT2 channels
    switch ((a.n_keep + 15) / 16) {
        case 1: return launch_ks<1>(a, s);
        case 2: return launch_ks<2>(a, s);
        case 3: return launch_ks<3>(a, s);
        case 4: return launch_ks<4>(a, s);
        case 5: return launch_ks<5>(a, s);
        case 6: return launch_ks<6>(a, s);
        case 7: return launch_ks<7>(a, s);
        default: return launch_ks<8>(a, s);
    }
}

}  // namespace dqk
