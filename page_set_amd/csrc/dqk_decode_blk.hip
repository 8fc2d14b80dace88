// Decode attention over the paged INT2 cache for four query heads per KV head
// (the GQA 32/8 shape), on MFMA.  Dual-QK paper: scores over the KV head's
// selected channels with the full 1/sqrt(d) scale (§3.2); channel 0 from its
// bf16 copy, channel-major INT2 key rows and token-major values with separate
// metadata (§3.3); one softmax over the whole context (§3.4).
//
// Work decomposition.  A workgroup (12 waves, one per CU) owns one split (a run
// of 8-page blocks) of one (sequence, KV head) and walks it in steps of four
// pages.  Loads go straight from HBM to LDS: the selected key rows of a whole
// 8-page block (one 256-byte run per channel), its key metadata and channel 0
// into one of two key stages, the value codes and value metadata of each
// 4-page half into one of three value stages, two steps ahead, every wave
// issuing a fixed share.  Waves 0-3 score: at step u wave w takes page w of
// half u (all 128 tokens, four heads), keeps the online softmax of that page
// stream and leaves the fp16 probabilities and the per-head rescale factor in
// LDS.  Waves 4-11 multiply: waves 4 + w and 8 + w take the values of page w
// of half u - 1, tokens 0-63 and 64-127.  Each SIMD thus runs one scoring and
// two multiplying waves.  The four page streams (two token halves each) are
// combined in LDS at the end of the split.
//
// Scores (v_mfma_f32_16x16x32_f16).  The 32-deep k dimension is (token group
// tg, 16 selected channels): A row i of tile m holds token 64 tg + 4 i + m,
// so a lane reads one byte (four tokens) of each of its eight channel rows
// and one AND per dword and tile yields two codes as binary16 subnormals
// code * 2^(2m - 24).  The 16 columns are (tg, head, limb), block diagonal in
// tg; the limbs are the fp16 hi and lo parts of q~ = log2(e)/sqrt(d) * q' *
// scale, computed once per page into LDS.  The zero points enter through an
// fp32 bias per head and page.
//
// Values.  O[(group q, head h)][channel] += (P * scale')[.][token] x
// code[token][channel] on the same MFMA, with P * scale' in fp16 where
// P = 2^(x - m + 14) (m an integer running maximum) and scale' = scale *
// 2^-E (E a running maximum exponent of the value scales): both stay in the
// normal fp16 range whatever the softmax sharpness or the value magnitude.
// Zero points, the softmax denominator and the centring term accumulate on
// two more MFMAs per 32 tokens.
#include "dqk_internal.h"

namespace dqk {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int GRP = 4;          // query heads per KV head handled here
constexpr int NW = 12;          // waves per workgroup: 4 scoring, 8 multiplying (two per page)
constexpr int NTHR = 64 * NW;
constexpr int PBOOST = 14;      // probabilities are kept as 2^(x - m + 14)
constexpr int EMIN = -15, EMAX = 15;  // clamp of the value-scale exponent
constexpr int TABN = 64;        // blocks of a split whose alignment is tabulated up front
constexpr int MAX_KS = 8;       // 16-channel k-steps: up to 128 selected channels
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
static_assert(KBLK == 8, "the kernel walks 8-page blocks in halves of four pages");

// ---------------------------------------------------------------- LDS layout
// KSX = KS + 16 KG + 32 RB: KS 16-channel k-steps; KG = 1 for one key grid per
// token (the block's key metadata then is [8 pages][128 tokens] pairs, 4 KB);
// RB = 1 for bucket-relative RoPE (a query and a channel list per 2048-token
// bucket, all of a split's buckets kept in LDS past the usual layout).
template <int KSX>
struct Lay {
    static constexpr int KS = KSX & 15;
    static constexpr bool KG = ((KSX >> 4) & 1) != 0;
    static constexpr bool RB = ((KSX >> 5) & 1) != 0;
    static constexpr int NR = 16 * KS;              // key row slots (selected INT2 channels, padded)
    static constexpr int NMR = (NR + 31) / 32 * 32;  // key metadata rows (whole load instructions)
    // key stage: rows [NR][256 B] (16-byte chunk c of row r at c ^ (2 ((r >> 3) & 1))),
    // metadata [NMR][8 pages] (scale | zero << 16) or, KG, [8 pages][128 tokens],
    // channel 0 [8 pages][128] bf16
    static constexpr int KMB = KG ? KBLK * PG * 4 : NMR * 32;
    static constexpr int KC = 0;
    static constexpr int KM = KC + NR * 256;
    static constexpr int K0 = KM + KMB;
    static constexpr int KST = K0 + 2048;
    // value stage: codes [token group G 4][32-token step 4][4 pages][8 tokens][32 B], each
    // group followed by 64 bytes of padding (the four groups read together fall in
    // different banks); metadata [4 pages][2 planes][4 groups q][128] fp16 with
    // 16-byte chunk c of (page, plane, q) at c ^ 4q
    static constexpr int VS = 2 * KST;
    static constexpr int VC = 0;
    static constexpr int VM = 16384 + 3 * 64;
    static constexpr int VST = VM + 8192;
    static constexpr int PBROW = 320;               // P of one head: 128 fp16 + 64 B of padding
    static constexpr int PBPAGE = 4 * PBROW;
    static constexpr int PBBUF = 4 * PBPAGE;
    // three value stages (values two steps ahead); two when the key stages leave no room
    // for a third (values then one step ahead) or, with buckets, for eight buckets' queries
    static constexpr int NV = KS <= (RB ? 6 : 7) ? 3 : 2;
    static constexpr int PB = VS + NV * VST;        // [2 buffers][4 pages][4 heads][PBROW]
    static constexpr int AL = PB + 2 * PBBUF;       // [2 buffers][4 pages][4 heads] float rescale factors
    static constexpr int QT = AL + 2 * 16 * 4;      // [4 scoring waves][KS][256 B] q~ B fragments
    static constexpr int ZERO = QT + 4 * KS * 256;  // KS * 256 bytes of zeros
    static constexpr int ONES = ZERO + KS * 256;    // 256 bytes of fp16 1.0
    static constexpr int TOTAL = ONES + 256;
    // buckets (RB): per bucket of the split q' of the four heads [4][128] fp32
    // and the ascending channel list [128] int32 (the layout of the scratch
    // below), up to MAXB buckets (a split covers at most 2 MAXB blocks)
    static constexpr int RBB = GRP * D * 4 + D * 4;
    static constexpr int RBA = TOTAL;
    static constexpr int MAXB_ROOM = (160 * 1024 - TOTAL) / RBB;
    static constexpr int MAXB = MAXB_ROOM < 8 ? MAXB_ROOM : 8;
    static constexpr int TOTAL_ALL = RB ? RBA + MAXB * RBB : TOTAL;
    // the selection run inside the decode (prologue only): T_Q of the KV head
    // [128][128] fp32 at 0, the four heads' q in fp32, then room for the
    // pooled energies and a mask word (kept in the layout; the energies now
    // stay in wave 0's registers); q' and the selected channels go to the
    // usual scratch in the last value stage, which lies past all of them
    static constexpr int SCR = VS + (NV - 1) * VST;
    static constexpr int FT = 0;
    static constexpr int FQ = D * D * 4;
    static constexpr int FS = FQ + GRP * D * 4;
    static constexpr int FM = FS + D * 4;
    static constexpr bool FUSABLE = FM + 16 <= SCR && FM + 16 <= TOTAL;
    // the values of the first half can load during the selection (their stage lies past it)
    static constexpr bool EARLY_V = NV == 3 && FM + 16 <= VS + VST;
    // global -> LDS loads: a key block is NRI row, NMI metadata and 2 channel-0
    // instructions; a value half is 16 code and 8 metadata instructions
    static constexpr int NRI = NR / 4;
    static constexpr int NMI = KMB / 1024;
    static constexpr int NKI = NRI + NMI + 2;
    static constexpr int KN = (NKI + NW - 1) / NW;  // key instructions per wave per block
    static constexpr int VN = 24 / NW;              // value instructions per wave per half
    static_assert(24 % NW == 0, "value loads split evenly");
    static_assert(TOTAL <= 160 * 1024 && TOTAL_ALL <= 160 * 1024, "LDS");
    static_assert(!RB || (MAXB >= 1 && !KG), "bucket area");
    static_assert(KST % 16 == 0 && KM % 16 == 0 && K0 % 16 == 0 && VS % 16 == 0 && PB % 16 == 0 &&
                      QT % 16 == 0 && ZERO % 16 == 0 && ONES % 16 == 0,
                  "align");
    static_assert(KN + VN <= 63, "vmcnt range");
    static_assert(8 * GRP * PART_FLOATS * 4 <= PB, "exchange area");
    static_assert(GRP * D * 4 + D * 4 <= VST, "prologue scratch");
};

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ half2v as_half2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// An LDS address computed once per step: the empty asm keeps the compiler from
// re-associating (step base + per-lane constant) + immediate, so that every
// access below folds the immediate into the instruction's offset field.
__device__ __forceinline__ uint32_t pinned(uint32_t a) {
    __asm__ volatile("" : "+v"(a));
    return a;
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T *>((uintptr_t)a);
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t a, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T *>((uintptr_t)a) = v;
}

// Direct global -> LDS loads: 16 or 4 bytes per lane written at M0 + lane * size.
// Issued from asm so that the compiler's wait-for-all before LDS reads does
// not apply; completion is awaited with s_waitcnt vmcnt(N), N = vector memory
// instructions this wave issued afterwards.  The scalar base must be
// wave-uniform.
__device__ __forceinline__ uint64_t uniform64(uint64_t a) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
}
__device__ __forceinline__ void dma16_s(uint64_t sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %0" ::"s"((const void *)(uintptr_t)sbase),
                 "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
// Own global->LDS loads down to N outstanding and own LDS accesses done,
// then the workgroup barrier, as one statement so that no LDS access can be
// scheduled between the wait and the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float bcast_lane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
template <int CTL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTL, 0xF, 0xF, false));
}
template <int CTL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROR4 = 0x124;  // row_ror:4 (rotate within 16 lanes)
constexpr int DPP_HMIRROR = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8
constexpr int DPP_ROR8 = 0x128;  // row_ror:8
template <int C>
constexpr int DPP_QB = C * 0x55;  // quad_perm [C, C, C, C]

// v_permlane16/32_swap with both operands v: combining the two results
// reduces over lane ^ 16 (lane ^ 32), identically in both lanes.
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
__device__ __forceinline__ uint32_t umax_x16(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t umax_x32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(r[0], r[1]);
}

// 2^e as binary16 bits, -15 <= e <= 15 (2^-15 is subnormal).
__device__ __forceinline__ uint32_t pow2_h(int e) {
    return e >= -14 ? (uint32_t)(e + 15) << 10 : 0x0200u;
}


// ---------------------------------------------------------------- load plan
// Key instruction idx of an 8-page block: 0 .. NRI-1 rows 4 idx .. 4 idx + 3
// (16 lanes a row; LDS chunk c of row r receives the row's global chunk
// c ^ (2 ((r >> 3) & 1)), i.e. page slot (chunk >> 1), half (chunk & 1));
// NRI .. NRI+NMI-1 metadata rows 32 j .. 32 j + 31 (two lanes a row, pages
// 4 h .. 4 h + 3 each); NRI + NMI + {0, 1} channel 0 of pages 4 i .. 4 i + 3.
// Value instruction idx of a 4-page half: 0 .. 15 codes of page idx >> 2,
// token rows 32 (idx & 3) .. + 31; 16 .. 23 metadata of page (idx - 16) >> 1,
// plane (idx - 16) & 1 (LDS chunk c of group q receives chunk c ^ q).
// Regions: 0 key rows, 1 key metadata, 2 channel 0, 3 value codes, 4 value metadata.
template <int KS>
__device__ __forceinline__ int key_region(int idx) {
    using Ly = Lay<KS>;
    return idx < Ly::NRI ? 0 : idx < Ly::NRI + Ly::NMI ? 1 : 2;
}
template <int KS>
__device__ __forceinline__ uint32_t key_lds(int idx) {
    using Ly = Lay<KS>;
    return idx < Ly::NRI ? Ly::KC + idx * 1024 : idx < Ly::NRI + Ly::NMI ? Ly::KM + (idx - Ly::NRI) * 1024
                                                                        : Ly::K0 + (idx - Ly::NRI - Ly::NMI) * 1024;
}
template <int KS>
__device__ __forceinline__ int key_row(int idx, int lane) {
    using Ly = Lay<KS>;
    return idx < Ly::NRI                            ? 4 * idx + (lane >> 4)
           : idx < Ly::NRI + Ly::NMI && !Ly::KG ? 32 * (idx - Ly::NRI) + (lane >> 1)
                                                  : 0;
}
// Per-lane byte offset of key instruction idx from the base of an aligned block.
template <int KS>
__device__ __forceinline__ uint32_t key_aoff(int idx, int lane, int chan, int hkv) {
    using Ly = Lay<KS>;
    if (idx < Ly::NRI) {
        const int r = 4 * idx + (lane >> 4);
        const int cd = (lane & 15) ^ (2 * ((r >> 3) & 1));
        return (uint32_t)(chan * (KBLK * ROW_BYTES) + cd * 16);
    }
    if (idx < Ly::NRI + Ly::NMI)  // per channel: two lanes a row; per token: 1 KB of the block's 4 KB
        return Ly::KG ? (uint32_t)((idx - Ly::NRI) * 1024 + lane * 16) : (uint32_t)(chan * (KBLK * 4) + (lane & 1) * 16);
    const int i = idx - Ly::NRI - Ly::NMI;
    return (uint32_t)(4 * i + (lane >> 4)) * (uint32_t)(hkv * PG * 2) + (uint32_t)((lane & 15) * 16);
}
__device__ __forceinline__ int val_region(int idx) { return idx < 16 ? 3 : 4; }
// Value code instruction idx = 4 G + s: tokens 32 s + 8 G .. + 7 of the half's
// four pages (16 lanes a page); metadata instruction 16 + j: page j >> 1,
// plane j & 1.
template <int KS>
__device__ __forceinline__ uint32_t val_lds(int idx) {
    using Ly = Lay<KS>;
    return idx < 16 ? Ly::VC + idx * 1024 + 64 * (idx >> 2) : Ly::VM + (idx - 16) * 1024;
}
__device__ __forceinline__ uint32_t vcode_off(int idx, int lane) {  // within the page
    return (uint32_t)((32 * (idx & 3) + 8 * (idx >> 2)) * ROW_BYTES + (lane & 15) * 16);
}
__device__ __forceinline__ uint32_t vmeta_off(int j, int lane) {  // within the page
    const int q = lane >> 4;
    return (uint32_t)((j & 1) * 1024 + q * 256 + (((lane & 15) ^ (4 * q)) * 16));
}
// Per-lane byte offset of value instruction idx from the base of an aligned half.
__device__ __forceinline__ uint32_t val_aoff(int idx, int lane, int hkv) {
    if (idx < 16) return (uint32_t)(lane >> 4) * (uint32_t)(hkv * PG * ROW_BYTES) + vcode_off(idx, lane);
    const int j = idx - 16;
    return (uint32_t)(j >> 1) * (uint32_t)(hkv * 2 * VGROUPS * PG * 2) + vmeta_off(j, lane);
}

// Base of KV head g's data in region r for aligned block (half) 0, and the
// stride from one aligned block (key regions) or half (value regions) to the next.
// (selects, not a switch: the region is wave-uniform and no indexed access
// to the cache descriptor is wanted)
__device__ __forceinline__ uint64_t region_base(const dqk_cache &c, int r, int g) {
    const uint64_t kc = (uint64_t)(uintptr_t)c.k_codes + (uint64_t)g * (D * KBLK * ROW_BYTES);
    const uint64_t km = (uint64_t)(uintptr_t)c.k_meta + (uint64_t)g * (D * KBLK * 4);
    const uint64_t k0 = (uint64_t)(uintptr_t)c.k_ch0 + (uint64_t)g * (PG * 2);
    const uint64_t vc = (uint64_t)(uintptr_t)c.v_codes + (uint64_t)g * (PG * ROW_BYTES);
    const uint64_t vm = (uint64_t)(uintptr_t)c.v_meta + (uint64_t)g * (2 * VGROUPS * PG * 2);
    return r == 0 ? kc : r == 1 ? km : r == 2 ? k0 : r == 3 ? vc : vm;
}
__device__ __forceinline__ uint64_t region_stride(int r, int hkv) {
    const uint32_t e = r == 0 ? D * KBLK * ROW_BYTES
                     : r == 1 ? D * KBLK * 4
                     : r == 2 ? KBLK * PG * 2
                     : r == 3 ? 4 * PG * ROW_BYTES
                              : 4 * 2 * VGROUPS * PG * 2;
    return (uint64_t)hkv * e;
}

// Aligned-block index of block bi of a sequence (its valid pages are physical
// pages 8k .. 8k + nvalid - 1 in slot order), or -1.
__device__ __forceinline__ int block_aligned(const int32_t *__restrict__ ptab, int bi, int npages) {
    const int lp = KBLK * bi, nv = min(KBLK, npages - lp);
    const int p0 = ptab[lp];
    bool al = (p0 & (KBLK - 1)) == 0;
#pragma unroll
    for (int j = 1; j < KBLK; ++j)
        if (j < nv) al = al && ptab[lp + j] == p0 + j;
    return al ? p0 / KBLK : -1;
}

// Physical page of slot s of block bi (slot 0's page for slots past the end).
struct BlockPages {
    const int32_t *pt;  // the block's page-table entries
    int nv;             // valid slots
    __device__ __forceinline__ int operator()(int s) const { return pt[s < nv ? s : 0]; }
};
__device__ __forceinline__ BlockPages block_pages(const int32_t *__restrict__ ptab, int bi, int npages) {
    return BlockPages{ptab + KBLK * bi, min(KBLK, npages - KBLK * bi)};
}

// Loads of a block whose pages are not an aligned group: each lane fetches
// its 16 bytes from its own page through registers and stores them where the
// direct load would have put them.
template <int KS>
__device__ __forceinline__ void slow_key(int idx, int lane, int chan, const BlockPages &p, const dqk_cache &c, int g,
                                         int hkv, uint32_t lds) {
    using Ly = Lay<KS>;
    u32x4 v;
    if (idx < Ly::NRI) {
        const int r = 4 * idx + (lane >> 4);
        const int cd = (lane & 15) ^ (2 * ((r >> 3) & 1));
        const int pp = p(cd >> 1);
        v = *reinterpret_cast<const u32x4 *>(c.k_codes + krow(pp, g, hkv, chan) * ROW_BYTES + (cd & 1) * 16);
    } else if (idx < Ly::NRI + Ly::NMI) {
        if constexpr (Ly::KG) {  // bytes 1024 j + 16 lane of the block: page slot 2 j + lane / 32, 4 tokens
            const int j = idx - Ly::NRI;
            v = *reinterpret_cast<const u32x4 *>(c.k_meta + ktok(p(2 * j + (lane >> 5)), g, hkv, (lane & 31) * 4) * 2);
        } else {
            const int h = lane & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = *reinterpret_cast<const uint32_t *>(c.k_meta + krow(p(4 * h + i), g, hkv, chan) * 2);
        }
    } else {
        const int i = idx - Ly::NRI - Ly::NMI;
        const int pp = p(4 * i + (lane >> 4));
        v = *reinterpret_cast<const u32x4 *>(c.k_ch0 + ((size_t)pp * hkv + g) * PG + (lane & 15) * 8);
    }
    lds_st<u32x4>(lds + lane * 16, v);
}

__device__ __forceinline__ void slow_val(int idx, int lane, const BlockPages &p, int hb, const dqk_cache &c, int g,
                                         int hkv, uint32_t lds) {
    u32x4 v;
    if (idx < 16) {
        const int pp = p(4 * hb + (lane >> 4));
        v = *reinterpret_cast<const u32x4 *>(c.v_codes + ((size_t)pp * hkv + g) * (PG * ROW_BYTES) + vcode_off(idx, lane));
    } else {
        const int j = idx - 16;
        const int pp = p(4 * hb + (j >> 1));
        v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint8_t *>(c.v_meta) +
                                             ((size_t)pp * hkv + g) * (2 * VGROUPS * PG * 2) + vmeta_off(j, lane));
    }
    lds_st<u32x4>(lds + lane * 16, v);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    half2v h;
    h[0] = (_Float16)a;
    h[1] = (_Float16)b;
    return as_u32(h);
}
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// The loads of one split: which instructions this wave issues for every block
// (the same plan each time), the alignment table, and the pipeline's wait.
template <int KS>
struct Feeder {
    using Ly = Lay<KS>;
    uint32_t S;
    const dqk_cache *c;
    const int32_t *ptab;
    int g, hkv, lane, wv, npages, B0, nb, nst;
    int tab;   // lane j: aligned index of block B0 + j (j < TABN), or -1
    int pend;  // loads of this wave issued at the previous step (the ones allowed in flight)
    uint32_t rba;  // buckets (RB): LDS address of bucket B0 / 2's query and channel list
    int n_keep;
    int kidx[Ly::KN], kchan[Ly::KN];
    uint32_t kaoff[Ly::KN], vaoff[Ly::VN];
    uint64_t kbase[Ly::KN], kstr[Ly::KN], vbase[Ly::VN], vstr[Ly::VN];

    __device__ __forceinline__ uint32_t kstage(int j) const { return S + (uint32_t)(j & 1) * Ly::KST; }
    // half u -> value stage (u + 1) % 3 (half 0 in stage 1, clear of the prologue's scratch
    // areas), or u % 2 with two stages
    __device__ __forceinline__ uint32_t vstage(int u) const {
        return S + Ly::VS + (uint32_t)((u + (Ly::NV == 3 ? 1 : 0)) % Ly::NV) * Ly::VST;
    }
    __device__ __forceinline__ int blk_of(int j) const {
        return j < TABN ? __builtin_amdgcn_readlane(tab, j)
                        : __builtin_amdgcn_readfirstlane(block_aligned(ptab, B0 + j, npages));
    }
    // Value plans and the alignment table (independent of the selected channels).
    __device__ __forceinline__ void plan_vals() {
#pragma unroll
        for (int k = 0; k < Ly::VN; ++k) {
            const int idx = wv + NW * k;
            vaoff[k] = val_aoff(idx, lane, hkv);
            vbase[k] = uniform64(region_base(*c, val_region(idx), g));
            vstr[k] = uniform64(region_stride(val_region(idx), hkv));
        }
        tab = -1;
        if (lane < min(nb, TABN)) tab = block_aligned(ptab, B0 + lane, npages);
        pend = 0;
    }
    // Key plans from the selected channels (chan_of: key row slot -> channel).
    template <typename ChanOf>
    __device__ __forceinline__ void plan_keys(ChanOf chan_of) {
#pragma unroll
        for (int k = 0; k < Ly::KN; ++k) {
            kidx[k] = __builtin_amdgcn_readfirstlane((wv + NW * k) % Ly::NKI);
            kchan[k] = chan_of(key_row<KS>(kidx[k], lane));
            kaoff[k] = key_aoff<KS>(kidx[k], lane, kchan[k], hkv);
            kbase[k] = uniform64(region_base(*c, key_region<KS>(kidx[k]), g));
            kstr[k] = uniform64(region_stride(key_region<KS>(kidx[k]), hkv));
        }
    }
    // Key plans of bucket kl of the split (RB): its channel list in the bucket area.
    __device__ __forceinline__ void plan_bucket(int kl) {
        const uint32_t lst = rba + (uint32_t)kl * Ly::RBB + GRP * D * 4;
        const int has0 = lds_ld<int32_t>(lst) == 0;  // the list is ascending
        const int R = n_keep - has0;
        plan_keys([&](int r) { return r < R ? lds_ld<int32_t>(lst + (r + has0) * 4) : 0; });
    }
    // Loads of block j's keys / half u's values; true when the block took the
    // register path (which leaves no load of this wave in flight).
    __device__ __forceinline__ bool issue_keys(int j) const {
        const uint32_t st = kstage(j);
        const int k = blk_of(j);
        if (k >= 0) {
#pragma unroll
            for (int i = 0; i < Ly::KN; ++i)
                dma16_s(uniform64(kbase[i] + (uint64_t)(uint32_t)k * kstr[i]), kaoff[i], st + key_lds<KS>(kidx[i]));
            return false;
        }
        const BlockPages p = block_pages(ptab, B0 + j, npages);
#pragma unroll
        for (int i = 0; i < Ly::KN; ++i) slow_key<KS>(kidx[i], lane, kchan[i], p, *c, g, hkv, st + key_lds<KS>(kidx[i]));
        return true;
    }
    __device__ __forceinline__ bool issue_vals(int u) const {
        const uint32_t st = vstage(u);
        const int j = u >> 1, hb = u & 1;
        const int k = blk_of(j);
        if (k >= 0) {
            const uint32_t hx = 2 * (uint32_t)k + (uint32_t)hb;
#pragma unroll
            for (int i = 0; i < Ly::VN; ++i)
                dma16_s(uniform64(vbase[i] + (uint64_t)hx * vstr[i]), vaoff[i], st + val_lds<KS>(wv + NW * i));
            return false;
        }
        const BlockPages p = block_pages(ptab, B0 + j, npages);
#pragma unroll
        for (int i = 0; i < Ly::VN; ++i) slow_val(wv + NW * i, lane, p, hb, *c, g, hkv, st + val_lds<KS>(wv + NW * i));
        return true;
    }
    // Start of step u: this wave's loads older than the previous step (with two
    // value stages: all but the previous step's key loads) are done, then the
    // workgroup barrier; then the loads of half u + 1's values (half u's) and,
    // at even steps, block u/2 + 1's keys.  halfpages(u): whether half u holds a page.
    template <typename HalfPages>
    __device__ __forceinline__ void top(int u, HalfPages halfpages) {
        if (u > 0 && pend == Ly::KN + Ly::VN)
            wait_vm_barrier<Ly::KN + Ly::VN>();
        else if (u > 0 && pend == Ly::KN)
            wait_vm_barrier<Ly::KN>();
        else if (u > 0 && pend == Ly::VN)
            wait_vm_barrier<Ly::VN>();
        else
            wait_vm_barrier<0>();
        int np = 0;
        if constexpr (Ly::NV == 3) {  // values of half u + 1: needed two steps later
            if (u + 1 < nst && halfpages(u + 1)) np = issue_vals(u + 1) ? 0 : np + Ly::VN;
        } else {  // values of half u: needed at the next step, so never left in flight
            if (u < nst && halfpages(u)) issue_vals(u);
        }
        if (!(u & 1) && (u >> 1) + 1 < nb) {
            // with buckets, an even block (B0 is even) starts the next bucket: its channels first
            if constexpr (Ly::RB)
                if (!(((u >> 1) + 1) & 1)) plan_bucket(((u >> 1) + 1) >> 1);
            np = issue_keys((u >> 1) + 1) ? 0 : np + Ly::KN;
        }
        pend = np;
    }
};

// ---------------------------------------------------------------- the kernel
// The channel selection of one (sequence, KV head), as dqk_select_channels
// computes it (the same fp32 fma chains in the same order, the same kept
// set), into the LDS scratch the decode prologue reads: q' [4][128] at scr,
// the ascending channel list after it.  qp_out / sel_out (may be null)
// receive the same values in global memory.  wsel (may be null): the KV
// head's selection scales, as dqk_select_channels_base applies them.
template <int KS>
__device__ __forceinline__ void select_into_lds(uint32_t S, uint32_t scr, const uint16_t *__restrict__ q_bf16,
                                                const float *__restrict__ t_q, const float *__restrict__ wsel, int b,
                                                int g, int hq, int hkv, int n_keep, float *__restrict__ qp_out,
                                                int32_t *__restrict__ sel_out) {
    using Ly = Lay<KS>;
    const int tid = threadIdx.x;
    // every load of the transform is issued before any is stored
    const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(t_q + (size_t)g * D * D);
    constexpr int NT = (D * D / 4 + NTHR - 1) / NTHR;
    u32x4 tv[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int i = tid + k * NTHR;
        if (i < D * D / 4) tv[k] = tsrc[i];
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int i = tid + k * NTHR;
        if (i < D * D / 4) lds_st<u32x4>(S + Ly::FT + i * 16, tv[k]);
    }
    const uint16_t *qg = q_bf16 + ((size_t)b * hq + (size_t)g * GRP) * D;
    for (int i = tid; i < GRP * D; i += NTHR) lds_st<float>(S + Ly::FQ + i * 4, bf2f(qg[i]));
    if (tid < D) lds_st<int32_t>(scr + GRP * D * 4 + tid * 4, 0);
    __syncthreads();
    // q'_{h,j}: fma chain over ascending input channel i
    if (tid < GRP * D) {
        const int h = tid >> 7, j = tid & (D - 1);
        float acc = 0.0f;
#pragma unroll 4
        for (int i = 0; i < D; i += 4) {
            const f32x4 qv4 = lds_ld<f32x4>(S + Ly::FQ + (h * D + i) * 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(qv4[k], lds_ld<float>(S + Ly::FT + ((i + k) * D + j) * 4), acc);
        }
        lds_st<float>(scr + (h * D + j) * 4, acc);
        if (qp_out) qp_out[((size_t)b * hq + (size_t)g * GRP + h) * D + j] = acc;
    }
    __syncthreads();
    // wave 0: pooled energies of channels lane and lane + 64 (fma chains over
    // ascending head), then the mask (top_k_wave) and the ascending list
    if (tid < 64) {
        const float wa = wsel ? wsel[tid] : 1.0f, wb = wsel ? wsel[tid + 64] : 1.0f;  // x * 1 is x exactly
        float ea = 0.0f, eb = 0.0f;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
            const float va = __fmul_rn(lds_ld<float>(scr + (h * D + tid) * 4), wa);
            const float vb = __fmul_rn(lds_ld<float>(scr + (h * D + tid + 64) * 4), wb);
            ea = __builtin_fmaf(va, va, ea);
            eb = __builtin_fmaf(vb, vb, eb);
        }
        const KeptPair kp = top_k_wave(ea, eb, n_keep);
        int32_t *so = sel_out ? sel_out + ((size_t)b * hkv + g) * n_keep : nullptr;
        if (kp.ka && kp.pa < n_keep) {
            lds_st<int32_t>(scr + GRP * D * 4 + kp.pa * 4, tid);
            if (so) so[kp.pa] = tid;
        }
        if (kp.kb && kp.pb < n_keep) {
            lds_st<int32_t>(scr + GRP * D * 4 + kp.pb * 4, tid + 64);
            if (so) so[kp.pb] = tid + 64;
        }
    }
}

template <int KSX, bool FUSED>
__global__ __launch_bounds__(NTHR) void decode_blk_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                          const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                          const int32_t *__restrict__ page_table, int max_pages,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          int nsplit, float *__restrict__ partials,
                                                          const uint16_t *__restrict__ q_bf16,
                                                          const float *__restrict__ t_q,
                                                          const float *__restrict__ sel_scale,
                                                          float *__restrict__ qp_out,
                                                          int32_t *__restrict__ sel_out, int nbk) {
    using Ly = Lay<KSX>;
    constexpr int KS = Ly::KS;
    constexpr bool KG = Ly::KG;
    static_assert(!(Ly::RB && FUSED), "buckets take their selection from memory");
    __shared__ __attribute__((aligned(16))) uint8_t smem[Ly::TOTAL_ALL];
    const uint32_t S = lds_addr(smem);

    const int split = blockIdx.x, bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    // grid.y runs over (sequence, KV head, set of up to four of its query
    // heads): a KV head with grp query heads takes ceil(grp / 4) workgroups
    // per split, each reading the KV head's pages for its heads h0 .. h0+nh-1
    // (a set of fewer than four leaves the rest of the tile at q' = 0)
    const int grp = hq / hkv, nsub = (grp + GRP - 1) / GRP;
    const int b = bg / (hkv * nsub), gs = bg - b * (hkv * nsub), g = gs / nsub, sub = gs - g * nsub;
    const int h0 = g * grp + sub * GRP, nh = min(GRP, grp - sub * GRP);
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // page of the half this wave scores (waves 0-3) or multiplies (waves 4-11, token half th)
    const int w = wv < 4 ? wv : (wv - 4) & 3;
    const int th = wv < 4 ? 0 : (wv - 4) >> 2;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    const int nblk = (npages + KBLK - 1) / KBLK;
    // with buckets (two blocks each) a split holds whole buckets, at most MAXB
    // of them (the launch picks enough splits; a larger split is left empty)
    int per = (nblk + nsplit - 1) / nsplit;
    if constexpr (Ly::RB) per = (per + 1) & ~1;
    const bool fits = !Ly::RB || per <= 2 * Ly::MAXB;
    const int B0 = fits ? min(nblk, split * per) : nblk, B1 = min(nblk, B0 + per);
    const int nb = B1 - B0;   // 8-page blocks of this split
    const int nst = 2 * nb;   // 4-page halves
    const int32_t *ptab = page_table + (size_t)b * max_pages;
    float *part_base = partials + (((size_t)b * hq + (size_t)h0) * nsplit + split) * PART_FLOATS;
    const size_t hstride = (size_t)nsplit * PART_FLOATS;

    if (FUSED && nb <= 0 && split == 0) {  // still deliver the selection of this (sequence, KV head)
        select_into_lds<KSX>(S, S + Ly::SCR, q_bf16, t_q, sel_scale ? sel_scale + (size_t)g * D : nullptr, b, g, hq,
                            hkv, n_keep, qp_out, sel_out);
    }
    if (nb <= 0) {  // nothing of this sequence falls in this split: an empty partial
        if (tid >= nh * D) return;
        const int h = tid >> 7, ch = tid & (D - 1);
        part_base[h * hstride + ch] = 0.0f;
        if (ch == 0) {
            part_base[h * hstride + D] = -__builtin_huge_valf();
            part_base[h * hstride + D + 1] = 0.0f;
            part_base[h * hstride + D + 2] = 0.0f;
        }
        return;
    }
    // valid tokens of page slot ps of block j (relative to B0)
    auto page_valid = [&](int j, int ps) { return min(PG, max(0, L - PG * (KBLK * (B0 + j) + ps))); };

    // ---- the loader: value plans first (they do not depend on the selection)
    Feeder<KSX> fd;
    fd.S = S;
    fd.c = &c;
    fd.ptab = ptab;
    fd.g = g;
    fd.hkv = hkv;
    fd.lane = lane;
    fd.wv = wv;
    fd.npages = npages;
    fd.B0 = B0;
    fd.nb = nb;
    fd.nst = nst;
    fd.rba = S + Ly::RBA;
    fd.n_keep = n_keep;
    fd.plan_vals();
    // in flight while the selection runs (or q' and the channel list are staged)
    constexpr bool early_v = Ly::NV == 3 && (!FUSED || Ly::EARLY_V);
    if constexpr (early_v) fd.issue_vals(0);

    // ---- q' of the four heads and the selected channels into LDS (value stage 2)
    const uint32_t scr = S + Ly::SCR;
    if constexpr (FUSED) {
        static_assert(Ly::FUSABLE, "selection scratch");
        select_into_lds<KSX>(S, scr, q_bf16, t_q, sel_scale ? sel_scale + (size_t)g * D : nullptr, b, g, hq, hkv,
                            n_keep, split == 0 ? qp_out : nullptr, split == 0 ? sel_out : nullptr);
        for (int i = tid; i < KS * 64; i += NTHR) lds_st<uint32_t>(S + Ly::ZERO + i * 4, 0u);
        if (tid < 64) lds_st<uint32_t>(S + Ly::ONES + tid * 4, 0x3C003C00u);
    } else if constexpr (Ly::RB) {
        // q' of the four heads and the channel list of every bucket of the split
        // (bucket kb0 + kl at RBA + kl RBB, laid out as the scratch below)
        const int kb0 = B0 >> 1, nbl = ((B1 + 1) >> 1) - kb0;
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(q_prime);
        for (int i = tid; i < nbl * 128; i += NTHR) {
            const int kl = i >> 7, r = i & 127, hr = r >> 5;
            const size_t row = ((size_t)b * nbk + kb0 + kl) * hq + h0 + hr;
            lds_st<u32x4>(S + Ly::RBA + kl * Ly::RBB + r * 16,
                          hr < nh ? qsrc[row * (D / 4) + (r & 31)] : u32x4{0u, 0u, 0u, 0u});
        }
        for (int i = tid; i < nbl * 128; i += NTHR) {
            const int kl = i >> 7, r = i & 127;
            const int32_t *ssrc = sel_idx + (((size_t)b * nbk + kb0 + kl) * hkv + g) * n_keep;
            lds_st<int32_t>(S + Ly::RBA + kl * Ly::RBB + GRP * D * 4 + r * 4, r < n_keep ? ssrc[r] : 0);
        }
        for (int i = tid; i < KS * 64; i += NTHR) lds_st<uint32_t>(S + Ly::ZERO + i * 4, 0u);
        if (tid < 64) lds_st<uint32_t>(S + Ly::ONES + tid * 4, 0x3C003C00u);
    } else {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(q_prime + ((size_t)b * hq + (size_t)h0) * D);
        const int32_t *ssrc = sel_idx + ((size_t)b * hkv + g) * n_keep;
        if (tid < 128) lds_st<u32x4>(scr + tid * 16, tid < 32 * nh ? qsrc[tid] : u32x4{0u, 0u, 0u, 0u});
        if (tid < 128) lds_st<int32_t>(scr + GRP * D * 4 + tid * 4, tid < n_keep ? ssrc[tid] : 0);
        for (int i = tid; i < KS * 64; i += NTHR) lds_st<uint32_t>(S + Ly::ZERO + i * 4, 0u);
        if (tid < 64) lds_st<uint32_t>(S + Ly::ONES + tid * 4, 0x3C003C00u);
    }
    __syncthreads();
    // q' and the channel list in force (with buckets: those of the split's first bucket)
    const uint32_t qsel = Ly::RB ? S + Ly::RBA : scr;
    auto qv = [&](int h, int j) { return lds_ld<float>(qsel + (h * D + j) * 4); };
    const int has0 = lds_ld<int32_t>(qsel + GRP * D * 4) == 0;  // the list is ascending
    const int R = n_keep - has0;                                 // selected INT2 channels
    // channel of key row slot r (slots past R read channel 0's all-zero row)
    auto chan_of = [&](int r) { return r < R ? lds_ld<int32_t>(qsel + GRP * D * 4 + (r + has0) * 4) : 0; };
    // key load plans, the same for every block: key instructions wv + 12k (a
    // wave past the end repeats a real load: same bytes, same place)
    fd.plan_keys(chan_of);
    auto halfpages = [&](int u) { return page_valid(u >> 1, 4 * (u & 1)) > 0; };

    // ---- per-lane constants of both roles (q' products from the scratch)
    const float C = sm_scale * LOG2E;
    const int ar = lane & 15, Gk = lane >> 4;
    constexpr int NPI = (KS + 1) / 2;  // channel pairs per lane in the q~ precompute
    float QC[NPI][2];
    const int hp = lane >> 4, j16 = lane & 15;  // q~ precompute: head, pair index
#pragma unroll
    for (int i = 0; i < NPI; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int slot = 2 * (j16 + 16 * i) + e;
            QC[i][e] = (slot < 16 * KS && slot < R) ? qv(hp, chan_of(slot)) * C : 0.0f;
        }
    const int hh = (ar >> 1) & 3;  // score column head
    float q0c = has0 ? qv(hh, 0) * C : 0.0f;
    // with buckets: the same constants from bucket kl's q' and channel list
    auto bucket_qc = [&](int kl) {
        const uint32_t qb = S + Ly::RBA + (uint32_t)kl * Ly::RBB, lst = qb + GRP * D * 4;
        const int h0s = lds_ld<int32_t>(lst) == 0;
        const int Rb = n_keep - h0s;
#pragma unroll
        for (int i = 0; i < NPI; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int slot = 2 * (j16 + 16 * i) + e;
                QC[i][e] = (slot < 16 * KS && slot < Rb)
                               ? lds_ld<float>(qb + (hp * D + lds_ld<int32_t>(lst + (slot + h0s) * 4)) * 4) * C
                               : 0.0f;
            }
        q0c = h0s ? lds_ld<float>(qb + hh * D * 4) * C : 0.0f;
    };
    __syncthreads();  // scratch read by every wave

    // ---- prologue loads: keys of block 0, values of half 0 (with two value stages, at step 0)
    fd.issue_keys(0);
    if constexpr (!early_v && Ly::NV == 3) fd.issue_vals(0);

    // exchange slots [4 page streams][2 token halves][4 heads][PART_FLOATS]
    const uint32_t xw = S + (uint32_t)(2 * w + th) * (GRP * PART_FLOATS * 4);
    if (wv < 4) {
        // ================= scoring waves: page w of every half
        const int tga = Gk >> 1, cs8 = Gk & 1;        // A: token group and channel half of the k-chunk
        const int tgc = ar >> 3, ll = ar & 1;         // B / output column (tg, head hh, limb)
        const uint32_t qt_w = S + Ly::QT + (uint32_t)w * (KS * 256);
        const uint32_t qb_lane = (tga == tgc ? qt_w : S + Ly::ZERO) + cs8 * 128 + hh * 32 + ll * 16;
        const int tok0 = 64 * tgc + 16 * Gk + 2 * ll;       // this lane's tokens: tok0 + 4 r + mm
        float m_run = -__builtin_huge_valf();  // integer running maximum (log2 units) of head hh
        float l32 = 0.0f;                      // fp32 sum of 2^(x - m) over this lane's tokens
        // ---- per-token key grids: the q~ limbs (q~_j = C q'_j, scaled by 2^kq as
        //      below) and the bias sum_j C q'_j, once per split; each token then
        //      scales its dot product by s_t and the bias by z_t.  The per-channel
        //      form in the loop is the same computation with the page's scales and
        //      zero points.
        auto prep_qt = [&](float &bias, float &comp0, float &comp1) {
            float bacc = 0.0f, vmax = 0.0f;
            float vq[NPI][2];
#pragma unroll
            for (int i = 0; i < NPI; ++i) {
                const int c0 = 2 * (j16 + 16 * i);
                vq[i][0] = vq[i][1] = 0.0f;
                if (c0 < 16 * KS) {
                    vq[i][0] = QC[i][0];
                    vq[i][1] = QC[i][1];
                    vmax = fmaxf(vmax, fmaxf(__builtin_fabsf(vq[i][0]), __builtin_fabsf(vq[i][1])));
                    bacc += QC[i][0];
                    bacc += QC[i][1];
                }
            }
            vmax = fmaxf(vmax, dpp<DPP_XOR1>(vmax));
            vmax = fmaxf(vmax, dpp<DPP_XOR2>(vmax));
            vmax = fmaxf(vmax, dpp<DPP_ROR4>(vmax));
            vmax = fmaxf(vmax, dpp<DPP_ROR8>(vmax));
            vmax = max_x32(max_x16(vmax));
            const int ev = (int)((__float_as_uint(vmax) >> 23) & 255u) - 127;  // floor(log2 vmax)
            const int kq = vmax > 0.0f ? min(100, max(-100, 14 - ev)) : 0;
            const float sq = __uint_as_float((uint32_t)(127 + kq) << 23);
#pragma unroll
            for (int i = 0; i < NPI; ++i) {
                const int c0 = 2 * (j16 + 16 * i);
                if (c0 < 16 * KS) {
                    const float v0 = vq[i][0] * sq, v1 = vq[i][1] * sq;
                    const _Float16 hi0 = (_Float16)v0, hi1 = (_Float16)v1;
                    const uint32_t off = (c0 >> 4) * 256 + ((c0 >> 3) & 1) * 128 + hp * 32 + (c0 & 7) * 2;
                    half2v hi;
                    hi[0] = hi0;
                    hi[1] = hi1;
                    lds_st<uint32_t>(qt_w + off, as_u32(hi));
                    lds_st<uint32_t>(qt_w + off + 16, pack_h2(v0 - (float)hi0, v1 - (float)hi1));
                }
            }
            // code units: tiles 0, 2 at 2^-20, tiles 1, 3 at 2^-18; undo them and 2^kq
            comp0 = __uint_as_float((uint32_t)(127 + 20 - kq) << 23);
            comp1 = __uint_as_float((uint32_t)(127 + 18 - kq) << 23);
            bacc += dpp<DPP_XOR1>(bacc);
            bacc += dpp<DPP_XOR2>(bacc);
            bacc += dpp<DPP_ROR4>(bacc);
            bacc += dpp<DPP_ROR8>(bacc);  // every lane of row h holds head h's bias
            const float b0 = bcast_lane(bacc, 0), b1 = bcast_lane(bacc, 16), b2 = bcast_lane(bacc, 32),
                        b3 = bcast_lane(bacc, 48);
            bias = hh == 0 ? b0 : hh == 1 ? b1 : hh == 2 ? b2 : b3;
        };
        float bias_t = 0.0f, comp0_t = 0.0f, comp1_t = 0.0f;  // per-token key grids: fixed for the split
        if constexpr (KG) prep_qt(bias_t, comp0_t, comp1_t);


        for (int u = 0; u <= nst; ++u) {
            fd.top(u, halfpages);
            if (u >= nst) continue;
            if constexpr (Ly::RB)
                if (u > 0 && (u & 3) == 0) bucket_qc(u >> 2);  // an even block (B0 is even) starts a bucket
            const int ps = 4 * (u & 1) + w;
            const int nv = page_valid(u >> 1, ps);
            if (nv <= 0) continue;
            const uint32_t kst = fd.kstage(u >> 1);

            float bias, comp0, comp1;
            if constexpr (KG) {
                bias = bias_t;
                comp0 = comp0_t;
                comp1 = comp1_t;
            } else {
                // ---- q~ limbs of the page into this wave's fragments, bias sum_j z_j C q'_j in fp32.
                //      q~ is scaled by 2^kq (largest |q~| of the page near 2^14) so that its
                //      products with the codes stay far above the binary16 subnormal range.
                float bacc = 0.0f, vmax = 0.0f;
                float vq[NPI][2];
    #pragma unroll
                for (int i = 0; i < NPI; ++i) {
                    const int c0 = 2 * (j16 + 16 * i);
                    vq[i][0] = vq[i][1] = 0.0f;
                    if (c0 < 16 * KS) {
                        const uint32_t d0 = lds_ld<uint32_t>(kst + Ly::KM + c0 * 32 + ps * 4);
                        const uint32_t d1 = lds_ld<uint32_t>(kst + Ly::KM + (c0 + 1) * 32 + ps * 4);
                        vq[i][0] = QC[i][0] * h2f(d0 & 0xFFFFu);
                        vq[i][1] = QC[i][1] * h2f(d1 & 0xFFFFu);
                        vmax = fmaxf(vmax, fmaxf(__builtin_fabsf(vq[i][0]), __builtin_fabsf(vq[i][1])));
                        bacc = __builtin_fmaf(QC[i][0], h2f(d0 >> 16), bacc);
                        bacc = __builtin_fmaf(QC[i][1], h2f(d1 >> 16), bacc);
                    }
                }
                vmax = fmaxf(vmax, dpp<DPP_XOR1>(vmax));
                vmax = fmaxf(vmax, dpp<DPP_XOR2>(vmax));
                vmax = fmaxf(vmax, dpp<DPP_ROR4>(vmax));
                vmax = fmaxf(vmax, dpp<DPP_ROR8>(vmax));
                vmax = max_x32(max_x16(vmax));
                const int ev = (int)((__float_as_uint(vmax) >> 23) & 255u) - 127;  // floor(log2 vmax)
                const int kq = vmax > 0.0f ? min(100, max(-100, 14 - ev)) : 0;
                const float sq = __uint_as_float((uint32_t)(127 + kq) << 23);
    #pragma unroll
                for (int i = 0; i < NPI; ++i) {
                    const int c0 = 2 * (j16 + 16 * i);
                    if (c0 < 16 * KS) {
                        const float v0 = vq[i][0] * sq, v1 = vq[i][1] * sq;
                        const _Float16 hi0 = (_Float16)v0, hi1 = (_Float16)v1;
                        const uint32_t off = (c0 >> 4) * 256 + ((c0 >> 3) & 1) * 128 + hp * 32 + (c0 & 7) * 2;
                        half2v hi;
                        hi[0] = hi0;
                        hi[1] = hi1;
                        lds_st<uint32_t>(qt_w + off, as_u32(hi));
                        lds_st<uint32_t>(qt_w + off + 16, pack_h2(v0 - (float)hi0, v1 - (float)hi1));
                    }
                }
                // code units: tiles 0, 2 at 2^-20, tiles 1, 3 at 2^-18; undo them and 2^kq
                comp0 = __uint_as_float((uint32_t)(127 + 20 - kq) << 23);
                comp1 = __uint_as_float((uint32_t)(127 + 18 - kq) << 23);
                bacc += dpp<DPP_XOR1>(bacc);
                bacc += dpp<DPP_XOR2>(bacc);
                bacc += dpp<DPP_ROR4>(bacc);
                bacc += dpp<DPP_ROR8>(bacc);  // every lane of row h holds head h's bias
                const float b0 = bcast_lane(bacc, 0), b1 = bcast_lane(bacc, 16), b2 = bcast_lane(bacc, 32),
                            b3 = bcast_lane(bacc, 48);
                bias = hh == 0 ? b0 : hh == 1 ? b1 : hh == 2 ? b2 : b3;
            }

            // ---- scores: four token tiles
            f32x4 Sc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) Sc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint32_t ab = kst + Ly::KC + cs8 * (8 * 256) + ((((2 * ps + tga) ^ (2 * cs8))) * 16) + ar;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint32_t lo = lds_ld<uint8_t>(ab + (16 * ks + 2 * e2) * 256);
                    const uint32_t hi = lds_ld<uint8_t>(ab + (16 * ks + 2 * e2 + 1) * 256);
                    X[e2] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u);  // lo byte -> byte 0, hi byte -> byte 2
                }
                const u32x4 Bq = lds_ld<u32x4>(qb_lane + ks * 256);
                // codes at bits 4..7 of each half (tiles 0, 1 shifted up): units 2^-20, 2^-18
                const u32x4 XS = X << 4;
                Sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(XS & 0x00300030u), as_half8(Bq), Sc[0], 0, 0, 0);
                Sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(XS & 0x00C000C0u), as_half8(Bq), Sc[1], 0, 0, 0);
                Sc[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(X & 0x00300030u), as_half8(Bq), Sc[2], 0, 0, 0);
                Sc[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(X & 0x00C000C0u), as_half8(Bq), Sc[3], 0, 0, 0);
            }

            // ---- logits (log2 units) of this lane's 8 tokens: tiles 2 ll, 2 ll + 1 joined with the other limb
            float x[4][2];
            const uint32_t k0a = kst + Ly::K0 + ps * 256 + tok0 * 2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t kw = lds_ld<uint32_t>(k0a + r * 8);
                u32x2 szt = {0u, 0u};  // per-token key grids: (scale, zero) of tokens tok0 + 4 r + {0, 1}
                if constexpr (KG) szt = lds_ld<u32x2>(kst + Ly::KM + (uint32_t)(ps * PG + tok0 + 4 * r) * 4);
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const float mine = ll ? Sc[2 + mm][r] : Sc[mm][r];
                    const float give = ll ? Sc[mm][r] : Sc[2 + mm][r];
                    float cm = mm ? comp1 : comp0, bz = bias;
                    if constexpr (KG) {
                        cm *= h2f(szt[mm] & 0xFFFFu);
                        bz *= h2f(szt[mm] >> 16);
                    }
                    float v = __builtin_fmaf(mine + dpp<DPP_XOR1>(give), cm, bz);
                    v = __builtin_fmaf(q0c, __uint_as_float(mm ? (kw & 0xFFFF0000u) : (kw << 16)), v);
                    x[r][mm] = v;
                }
            }
            if (nv < PG) {  // tokens past the sequence end (their bytes are unspecified) get no weight
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int mm = 0; mm < 2; ++mm)
                        if (tok0 + 4 * r + mm >= nv) x[r][mm] = -__builtin_huge_valf();
            }
            // ---- integer running maximum of head hh, rescale factor for the multiplying wave
            float bm = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[1][0], x[1][1])),
                             fmaxf(fmaxf(x[2][0], x[2][1]), fmaxf(x[3][0], x[3][1])));
            bm = fmaxf(bm, dpp<DPP_XOR1>(bm));
            bm = fmaxf(bm, dpp<DPP_ROR8>(bm));
            bm = max_x32(max_x16(bm));
            const float m_new = fmaxf(m_run, ceilf(bm));
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf, 1 when unchanged
            m_run = m_new;
            l32 *= alpha;
            // ---- probabilities 2^(x - m + 14) -> fp16 -> the P buffer of this half
            const uint32_t pbw = S + Ly::PB + (uint32_t)(u & 1) * Ly::PBBUF + (uint32_t)w * Ly::PBPAGE + hh * Ly::PBROW +
                                 tok0 * 2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p0 = __builtin_amdgcn_exp2f(x[r][0] - m_new + (float)PBOOST);
                const float p1 = __builtin_amdgcn_exp2f(x[r][1] - m_new + (float)PBOOST);
                l32 += p0 + p1;
                lds_st<uint32_t>(pbw + r * 8, pack_h2(p0, p1));
            }
            if (lane < 8 && ll == 0)  // lane 2h: column (0, h, 0)
                lds_st<float>(S + Ly::AL + (uint32_t)(((u & 1) * 16 + w * 4 + hh) * 4), alpha);
        }
        // ---- this stream's m and l32 per head
        float l32h = l32 + dpp<DPP_XOR1>(l32);
        l32h += dpp<DPP_ROR8>(l32h);
        l32h = sum_x32(sum_x16(l32h));
        __syncthreads();  // every wave is done with the stages: the exchange reuses them
        if (lane < 8 && ll == 0) {
            lds_st<float>(xw + (hh * PART_FLOATS + D) * 4, m_run);
            lds_st<float>(xw + (hh * PART_FLOATS + D + 2) * 4, l32h);
        }
    } else {
        // ================= multiplying waves: tokens 64 th .. 64 th + 63 of page w of every
        //                   half, one step behind (32-token steps ps = 2 th, 2 th + 1)
        const int q = ar >> 2, hv = ar & 3, cz = ar & 3;  // A row (group q, head hv); Oz column (q, cz)
        const uint32_t pr_lane = S + Ly::PB + (uint32_t)w * Ly::PBPAGE + hv * Ly::PBROW + 16 * Gk + 128 * th;
        // scales of group q, tokens 32 ps + 8 Gk .. + 7: chunk 4 ps + Gk stored at (4 ps + Gk) ^ 4 q
        uint32_t sp_lane[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sp_lane[j] = Ly::VM + (uint32_t)w * 2048 + q * 256 + 16 * (4 * ((2 * th + j) ^ q) + Gk);
        const uint32_t bz_plane = cz == 0 ? 1024u : 0u;  // zero points / scales
        const uint32_t bz_const = S + (cz == 1 ? Ly::ONES : Ly::ZERO);
        const bool bz_var = (cz & 1) == 0;
        const uint32_t vc_lane = Ly::VC + 4160u * Gk + 256u * w + 2 * ar + 2048u * th;  // + 1024 j + 32 e
        half8 M15;
        {
            const _Float16 m = (_Float16)(cz == 3 ? -1.5f : 0.0f);
            M15 = half8{m, m, m, m, m, m, m, m};
        }
        int e_run = EMIN;  // running exponent of the value scales
        f32x4 O[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 Oz = {0.f, 0.f, 0.f, 0.f};

        for (int u = 0; u <= nst; ++u) {
            fd.top(u, halfpages);
            if (u < 1) continue;
            const int uu = u - 1;
            const int nvp = page_valid(uu >> 1, 4 * (uu & 1) + w);  // valid tokens of the page
            if (nvp <= 0) continue;                                    // not scored either
            const int buf = uu & 1;
            // ---- softmax rescale of what this stream holds (also when this half holds
            //      no token of the page: the scoring wave may have raised the maximum)
            const f32x4 al = lds_ld<f32x4>(S + Ly::AL + (uint32_t)((buf * 16 + w * 4) * 4));
            if (al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f) {  // wave-uniform
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) O[t][r] *= al[r];
#pragma unroll
                for (int r = 0; r < 4; ++r) Oz[r] *= al[r];
            }
            const int nv = nvp - 64 * th;  // valid tokens of this half
            if (nv <= 0) continue;
            const uint32_t vst = fd.vstage(uu);
            // ---- value-scale exponent of these tokens; rescale O when it grows
            u32x4 spv[2], keep[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) spv[j] = lds_ld<u32x4>(vst + sp_lane[j]);
            if (nv < 64) {  // metadata past the sequence end is unspecified: keep it out of everything
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int t = 32 * j + 8 * Gk + 2 * e2;
                        keep[j][e2] = (t < nv ? 0x0000FFFFu : 0u) | (t + 1 < nv ? 0xFFFF0000u : 0u);
                    }
                    spv[j] &= keep[j];
                }
            }
            // largest scale: packed 16-bit maxima (scales are >= 0, so their bit
            // patterns order like their values), as a tree
            u16x2 m2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) m2[e] = __builtin_elementwise_max(as_u16x2(spv[0][e]), as_u16x2(spv[1][e]));
            m2[0] = __builtin_elementwise_max(m2[0], m2[1]);
            m2[2] = __builtin_elementwise_max(m2[2], m2[3]);
            m2[0] = __builtin_elementwise_max(m2[0], m2[2]);
            uint32_t mx = max((uint32_t)m2[0][0], (uint32_t)m2[0][1]);
            mx = max(mx, dpp_u<DPP_ROR4>(mx));
            mx = max(mx, dpp_u<DPP_ROR8>(mx));
            mx = umax_x32(umax_x16(mx));
            const int ex = __builtin_amdgcn_readfirstlane((int)((mx >> 10) & 31u));
            const int e_pg = min(EMAX, max(EMIN, ex == 0 ? EMIN : ex - 15));
            if (e_pg > e_run) {  // wave-uniform
                const float f = __uint_as_float((uint32_t)(127 + e_run - e_pg) << 23);
#pragma unroll
                for (int t = 0; t < 8; ++t) O[t] *= f;
                if (cz == 3) Oz *= f;
                e_run = e_pg;
            }
            // scale' = scale * 2^-E (skipped when E = 0)
            if (e_run != 0) {  // wave-uniform
                const uint32_t sc_h = pow2_h(-e_run);
                const half2v sc2 = as_half2(sc_h | (sc_h << 16));
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) spv[j][e2] = as_u32(as_half2(spv[j][e2]) * sc2);
            }
            // ---- value products, 32 tokens per step
            const uint32_t prb = pr_lane + (uint32_t)buf * Ly::PBBUF;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4 Pp = lds_ld<u32x4>(prb + 64 * j);
                u32x4 Bz = lds_ld<u32x4>(bz_var ? vst + sp_lane[j] + bz_plane : bz_const + 64 * j);
                if (nv < 64) Bz &= keep[j];
                u32x4 A;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) A[e2] = as_u32(as_half2(Pp[e2]) * as_half2(spv[j][e2]));
                const uint32_t vb = pinned(vst + vc_lane + 1024 * j);
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint32_t lo = lds_ld<uint16_t>(vb + (2 * e2) * 32);
                    const uint32_t hi = lds_ld<uint16_t>(vb + (2 * e2 + 1) * 32);
                    X[e2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
                const half8 Ah = as_half8(A);
                Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(Pp), as_half8(Bz), Oz, 0, 0, 0);
                Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, M15, Oz, 0, 0, 0);
                // channel t of each 16-bit word moved to bit 4, 6 or 8 (units 2^-20, 2^-18, 2^-16):
                // the lowest subnormal positions lose product bits in the MFMA
                const u32x4 XL = X << 4, XM = X >> 2, XH = X >> 8;
                O[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XL & 0x00300030u), O[0], 0, 0, 0);
                O[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XL & 0x00C000C0u), O[1], 0, 0, 0);
                O[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XL & 0x03000300u), O[2], 0, 0, 0);
                O[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XM & 0x00300030u), O[3], 0, 0, 0);
                O[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XM & 0x00C000C0u), O[4], 0, 0, 0);
                O[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XM & 0x03000300u), O[5], 0, 0, 0);
                O[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XH & 0x00300030u), O[6], 0, 0, 0);
                O[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XH & 0x00C000C0u), O[7], 0, 0, 0);
            }
        }
        // ---- this stream's o and l: lanes with ar >> 2 == Gk hold channels 8 ar + t of
        //      group Gk for heads r = 0..3; columns 4 Gk + c of Oz hold the group's sums
        float col[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            col[0][r] = dpp<DPP_QB<0>>(Oz[r]);
            col[1][r] = dpp<DPP_QB<1>>(Oz[r]);
            col[2][r] = dpp<DPP_QB<2>>(Oz[r]);
            col[3][r] = dpp<DPP_QB<3>>(Oz[r]);
        }
        const float escale = __uint_as_float((uint32_t)(127 + e_run) << 23);
        __syncthreads();  // every wave is done with the stages: the exchange reuses them
        if ((ar >> 2) == Gk) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float comp = t % 3 == 0 ? 1048576.0f : t % 3 == 1 ? 262144.0f : 65536.0f;  // 2^20, 2^18, 2^16
                    const float o = __builtin_fmaf(escale, __builtin_fmaf(O[t][r], comp, col[3][r]),
                                                   __builtin_fmaf(1.5f, col[2][r], col[0][r]));
                    lds_st<float>(xw + (r * PART_FLOATS + 8 * ar + t) * 4, o);
                }
            if (ar == 4 * Gk) {  // l of head Gk: column (Gk, 1), row (Gk, Gk)
                const float lg = Gk == 0 ? col[1][0] : Gk == 1 ? col[1][1] : Gk == 2 ? col[1][2] : col[1][3];
                lds_st<float>(xw + (Gk * PART_FLOATS + D + 1) * 4, lg);
            }
        }
    }
    __syncthreads();
    // ---- combine the four page streams (two token halves each): thread (h, ch)
    if (tid < nh * D) {
        const int h = tid >> 7, ch = tid & (D - 1);
        auto slot = [&](int v, int half) { return S + (uint32_t)(((2 * v + half) * GRP + h) * PART_FLOATS) * 4; };
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, lds_ld<float>(slot(v, 0) + D * 4));
        float o = 0.0f, l = 0.0f, l3 = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float mv = lds_ld<float>(slot(v, 0) + D * 4);
            const float f = mv == -__builtin_huge_valf() ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
            o = __builtin_fmaf(lds_ld<float>(slot(v, 0) + ch * 4) + lds_ld<float>(slot(v, 1) + ch * 4), f, o);
            if (ch == 0) {
                l = __builtin_fmaf(lds_ld<float>(slot(v, 0) + (D + 1) * 4) + lds_ld<float>(slot(v, 1) + (D + 1) * 4), f,
                                   l);
                l3 = __builtin_fmaf(lds_ld<float>(slot(v, 0) + (D + 2) * 4), f, l3);
            }
        }
        float *dst = part_base + (size_t)h * hstride;
        const bool any = M != -__builtin_huge_valf();
        dst[ch] = any ? o : 0.0f;
        if (ch == 0) {
            dst[D] = any ? (M - (float)PBOOST) * LN2 : -__builtin_huge_valf();
            dst[D + 1] = any ? l : 0.0f;
            dst[D + 2] = any ? l3 : 0.0f;
        }
    }
}

}  // namespace

bool use_mfma_decode(int hq, int hkv, int n_keep) {
    return hkv > 0 && hq % hkv == 0 && hq / hkv <= MAX_GROUP && n_keep <= 16 * MAX_KS;
}

int mfma_head_sets(int hq, int hkv) { return (hq / hkv + GRP - 1) / GRP; }

static int ks_of(int n_keep) {
    const int k = (n_keep + 15) / 16;
    return k < 1 ? 1 : k > MAX_KS ? MAX_KS : k;
}

// units_per_seq: workgroups of one split and sequence (KV heads x head sets)
int decode_splits_mfma(int batch, int units_per_seq, int max_pages, int n_keep) {
    (void)n_keep;
    // one workgroup per CU (LDS-bound): enough splits to give each of the 256
    // CUs one (down to one 8-page block per split: a short batch is latency-
    // bound, and more workgroups in flight beat a longer pipeline in each);
    // long contexts split so that no split exceeds 16 blocks (ragged batches
    // stay balanced)
    const int units = batch * units_per_seq;
    const int nblk = (max_pages + KBLK - 1) / KBLK;
    int s = (256 + units - 1) / units;
    const int need = (nblk + 15) / 16;
    if (s < need) s = need;
    if (s > nblk) s = nblk;
    return s < 1 ? 1 : s;
}

// n_keep 0: the most any n_keep needs (workspace sizing)
int decode_splits_rope(int max_pages, int n_keep) {
    int maxb = 8;
    switch (n_keep > 0 ? ks_of(n_keep) : 0) {
        case 0: {
            const int m[8] = {Lay<33>::MAXB, Lay<34>::MAXB, Lay<35>::MAXB, Lay<36>::MAXB,
                              Lay<37>::MAXB, Lay<38>::MAXB, Lay<39>::MAXB, Lay<40>::MAXB};
            for (int i = 0; i < 8; ++i) maxb = m[i] < maxb ? m[i] : maxb;
            break;
        }
        case 1: maxb = Lay<1 + 32>::MAXB; break;
        case 2: maxb = Lay<2 + 32>::MAXB; break;
        case 3: maxb = Lay<3 + 32>::MAXB; break;
        case 4: maxb = Lay<4 + 32>::MAXB; break;
        case 5: maxb = Lay<5 + 32>::MAXB; break;
        case 6: maxb = Lay<6 + 32>::MAXB; break;
        case 7: maxb = Lay<7 + 32>::MAXB; break;
        default: maxb = Lay<8 + 32>::MAXB; break;
    }
    const int nblk = (max_pages + KBLK - 1) / KBLK;
    return (nblk + 2 * maxb - 1) / (2 * maxb);
}

bool fused_select_ok(int hq, int hkv, int n_keep, bool token_grid) {
    if (!use_mfma_decode(hq, hkv, n_keep) || hq != GRP * hkv) return false;  // the prologue pools four heads
    const int g = token_grid ? 16 : 0;
    switch (ks_of(n_keep) + g) {
        case 1: return Lay<1>::FUSABLE;
        case 2: return Lay<2>::FUSABLE;
        case 3: return Lay<3>::FUSABLE;
        case 4: return Lay<4>::FUSABLE;
        case 5: return Lay<5>::FUSABLE;
        case 6: return Lay<6>::FUSABLE;
        case 7: return Lay<7>::FUSABLE;
        case 8: return Lay<8>::FUSABLE;
        case 17: return Lay<17>::FUSABLE;
        case 18: return Lay<18>::FUSABLE;
        case 19: return Lay<19>::FUSABLE;
        case 20: return Lay<20>::FUSABLE;
        case 21: return Lay<21>::FUSABLE;
        case 22: return Lay<22>::FUSABLE;
        case 23: return Lay<23>::FUSABLE;
        default: return Lay<24>::FUSABLE;
    }
}

template <int KSX, bool FUSED>
static hipError_t launch_ks2(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv * mfma_head_sets(a.hq, a.hkv));
    hipLaunchKernelGGL((decode_blk_kernel<KSX, FUSED>), grid, dim3(NTHR), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep,
                       a.hq, a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials, a.q_bf16,
                       a.t_q, a.sel_scale, a.qp_out, a.sel_out, a.n_buckets);
    return hipGetLastError();
}

template <int KS>
static hipError_t launch_ks(const DecodeArgs &a, hipStream_t s) {
    if (a.n_buckets > 0) {  // bucket-relative RoPE (KSX = KS + 32), the selection from memory
        if (a.q_bf16 || a.token_grid) return hipErrorInvalidValue;
        return launch_ks2<KS + 32, false>(a, s);
    }
    if (a.token_grid) {  // per-token key grids (KSX = KS + 16)
        if constexpr (Lay<KS + 16>::FUSABLE) {
            if (a.q_bf16) return launch_ks2<KS + 16, true>(a, s);
        } else {
            if (a.q_bf16) return hipErrorInvalidValue;
        }
        return launch_ks2<KS + 16, false>(a, s);
    }
    if constexpr (Lay<KS>::FUSABLE) {
        if (a.q_bf16) return launch_ks2<KS, true>(a, s);
    } else {
        if (a.q_bf16) return hipErrorInvalidValue;
    }
    return launch_ks2<KS, false>(a, s);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    // 16-channel k-steps for the selected INT2 channels
    switch (ks_of(a.n_keep)) {
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
