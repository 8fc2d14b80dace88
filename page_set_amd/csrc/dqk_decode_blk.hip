// Decode attention over the paged INT2 cache for four query heads per KV head
// (the GQA 32/8 shape), on MFMA.  Dual-QK paper: scores over the KV head's
// selected channels with the full 1/sqrt(d) scale (§3.2); channel 0 from its
// bf16 copy, channel-major INT2 key rows and token-major values with separate
// metadata (§3.3); one softmax over the whole context (§3.4).
//
// Work decomposition.  A workgroup is 8 waves and owns one split (a run of
// aligned 4-page blocks) of one (sequence, KV head).  The block is the unit of
// staging: its selected key rows (one 128-byte run per channel: the four
// pages' 32-byte rows side by side), key metadata, channel 0, value codes and
// value metadata go through LDS by direct global->LDS loads, three blocks in
// flight.  Wave (w, hf) handles tokens 64hf..64hf+63 of page w of every block
// and keeps its own online softmax; the eight partials are combined in LDS at
// the end of the split.  Step u scores block u and multiplies the values of
// block u - 1 in one instruction stream; the keys of block u + 2 and the
// values of block u + 1 load meanwhile.
//
// Scores (v_mfma_f32_16x16x32_f16).  The 32-deep k dimension is (token group
// tg, 16 selected channels): A row i holds token 32tg + 8(i >> 2) + 4m + (i & 3)
// of tile m, so a lane reads one 16-bit word (8 tokens) of each of its eight
// channel rows and one AND per dword gives two codes as binary16 subnormals
// code * 2^(2(i & 3) - 24).  The 16 columns are (tg, head, limb), block
// diagonal in tg; the limbs are the fp16 hi and lo parts of
// q~ = log2(e)/sqrt(d) * q' * scale, computed once per page into LDS.
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

constexpr int GRP = 4;          // query heads per KV head handled here
constexpr int NW = 8;           // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int NSTAGE = 3;
constexpr int PBOOST = 14;      // probabilities are kept as 2^(x - m + 14)
constexpr int EMIN = -15, EMAX = 15;  // clamp of the value-scale exponent
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- LDS layout
template <int KS>
struct Lay {
    static constexpr int NR = 16 * KS;         // key row slots (selected INT2 channels, padded)
    static constexpr int KC = 0;               // [NR][128 B]; 16-byte chunk c of row r at c ^ ((r >> 3) & 1)
    static constexpr int KM = KC + NR * 128;   // [NR][4 pages] (scale | zero << 16)
    static constexpr int K0 = KM + NR * 16;    // [4 pages][128] bf16 channel 0
    static constexpr int VC = K0 + 1024;       // [4 pages][128 tokens][32 B]
    static constexpr int VM = VC + 16384;      // [4 pages][2 planes][4 groups][128] fp16; chunk c of (., q) at c ^ q
    static constexpr int STAGE = VM + 8192;
    static constexpr int PBW = 4 * 144;        // per wave: P [4 heads][64 tokens] fp16, rows padded to 144 B
    static constexpr int PB = NSTAGE * STAGE;
    static constexpr int QT = PB + NW * PBW;   // per wave: q~ B fragments [KS][256 B]
    static constexpr int ZERO = QT + NW * KS * 256;  // KS * 256 B of zeros
    static constexpr int ONES = ZERO + KS * 256;     // 16 B of fp16 ones, then 16 B of zeros
    static constexpr int TOTAL = ONES + 32;
    // global -> LDS loads of one block: key rows (2 KS x 1 KB), key metadata
    // (KS x 64 dwords), channel 0 (1 KB); value codes (16 x 1 KB), value metadata (8 x 1 KB)
    static constexpr int NKI = 3 * KS + 1;
    static constexpr int KN = (NKI + NW - 1) / NW;   // key instructions per wave per block
    static constexpr int VN = 3;                     // value instructions per wave per block
    static_assert(TOTAL <= 160 * 1024, "LDS");
    static_assert(STAGE % 16 == 0 && KM % 16 == 0 && K0 % 16 == 0 && VC % 16 == 0 && VM % 16 == 0, "align");
    static_assert(2 * (KN + VN) <= 63, "vmcnt range");
};

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ half2v as_half2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

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
// Two 16-bit LDS words -> one dword (lo, hi).
__device__ __forceinline__ uint32_t lds_pair(uint32_t a_lo, uint32_t a_hi) {
    return __builtin_amdgcn_perm(lds_ld<uint16_t>(a_hi), lds_ld<uint16_t>(a_lo), 0x05040100u);
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
                 "v"(voff), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(uint64_t sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, %0" ::"s"((const void *)(uintptr_t)sbase),
                 "v"(voff), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_v(uint64_t addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"((const void *)(uintptr_t)addr),
                 "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_v(uint64_t addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"((const void *)(uintptr_t)addr), "s"(lds)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Own loads down to N outstanding, then the workgroup barrier, as one
// statement so that no LDS access can be scheduled between the two.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
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

// ---------------------------------------------------------------- block addressing
// Base addresses of one 4-page block of one KV head in the five buffers, for
// the aligned case (the block's pages are physical pages 4k .. 4k+3).
struct BlockBase {
    uint64_t kc, km, k0, vc, vm;
};

__device__ __forceinline__ BlockBase block_base(const dqk_cache &c, int64_t k, int g, int hkv) {
    BlockBase bb;
    const uint64_t kb = (uint64_t)k * hkv + g;         // key block index
    const uint64_t pg = (uint64_t)(4 * k) * hkv + g;   // first page of the block
    bb.kc = uniform64((uint64_t)(uintptr_t)c.k_codes + kb * (D * KBLK * ROW_BYTES));
    bb.km = uniform64((uint64_t)(uintptr_t)c.k_meta + kb * (D * KBLK * 4));
    bb.k0 = uniform64((uint64_t)(uintptr_t)c.k_ch0 + pg * (PG * 2));
    bb.vc = uniform64((uint64_t)(uintptr_t)c.v_codes + pg * (PG * ROW_BYTES));
    bb.vm = uniform64((uint64_t)(uintptr_t)c.v_meta + pg * (2 * VGROUPS * PG * 2));
    return bb;
}

// Physical pages of block `blk` of a sequence: pages[j] for its valid slots,
// slot 0's page repeated for the others; aligned iff page 4k + j sits in slot j.
struct BlockPages {
    int64_t p[4];
    bool aligned;
    int nvalid;  // valid pages in the block
};

__device__ __forceinline__ BlockPages block_pages(const int32_t *__restrict__ ptab, int blk, int npages) {
    BlockPages bp;
    const int lp = 4 * blk;
    bp.nvalid = min(4, npages - lp);
    bp.p[0] = ptab[lp];
    bool al = (bp.p[0] & 3) == 0;
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        bp.p[j] = j < bp.nvalid ? (int64_t)ptab[lp + j] : bp.p[0];
        al = al && (j >= bp.nvalid || bp.p[j] == bp.p[0] + j);
    }
    bp.aligned = al;
    return bp;
}

// Global -> LDS load instructions of one block, numbered 0 .. NKI-1 (keys) and
// 0 .. 23 (values).  Key instruction idx: 0 .. 2KS-1 key rows 8 idx .. 8 idx + 7
// (8 lanes per row: 16-byte chunk cd of the row's 128-byte run at LDS chunk
// cd ^ (idx & 1)); 2KS .. 3KS-1 key metadata rows 16 j .. 16 j + 15 (a dword per
// page); 3KS channel 0 of the four pages.  Value instruction idx: 0 .. 15 value
// codes of page idx >> 2, token rows 32 (idx & 3) .. + 31; 16 .. 23 value
// metadata of page (idx - 16) >> 1, plane (idx - 16) & 1 (chunk cd of group q
// at LDS chunk cd ^ q).
//
// Per lane, the page slot of its chunk and its byte offset within that page's
// data (key rows / metadata: within the channel's run, the slot excluded).
struct LanePart {
    uint32_t slot, off;
};

template <int KS>
__device__ __forceinline__ int key_row(int idx, int lane) {
    return idx < 2 * KS ? 8 * idx + (lane >> 3) : idx < 3 * KS ? 16 * (idx - 2 * KS) + (lane >> 2) : 0;
}

template <int KS>
__device__ __forceinline__ LanePart key_part(int idx, int lane, int chan_r) {
    if (idx < 2 * KS) {
        const int cs = (lane & 7) ^ (idx & 1);
        return {(uint32_t)(cs >> 1), (uint32_t)(chan_r * (KBLK * ROW_BYTES) + (cs & 1) * 16)};
    }
    if (idx < 3 * KS) return {(uint32_t)(lane & 3), (uint32_t)(chan_r * (KBLK * 4))};
    return {(uint32_t)(lane >> 4), (uint32_t)((lane & 15) * 16)};
}

__device__ __forceinline__ LanePart val_part(int idx, int lane) {
    if (idx < 16) return {(uint32_t)(idx >> 2), (uint32_t)((idx & 3) * 1024 + lane * 16)};
    const int j = idx - 16, q = lane >> 4, cd = lane & 15;
    return {(uint32_t)(j >> 1), (uint32_t)((j & 1) * 1024 + q * 256 + ((cd ^ q) * 16))};
}

template <int KS>
__device__ __forceinline__ int key_region(int idx) {
    return idx < 2 * KS ? 0 : idx < 3 * KS ? 1 : 2;
}
__device__ __forceinline__ int val_region(int idx) { return idx < 16 ? 3 : 4; }

template <int KS>
__device__ __forceinline__ uint32_t key_lds(int idx) {
    using Ly = Lay<KS>;
    return idx < 2 * KS ? Ly::KC + idx * 1024 : idx < 3 * KS ? Ly::KM + (idx - 2 * KS) * 256 : Ly::K0;
}
template <int KS>
__device__ __forceinline__ uint32_t val_lds(int idx) {
    using Ly = Lay<KS>;
    return idx < 16 ? Ly::VC + idx * 1024 : Ly::VM + (idx - 16) * 1024;
}

// Offset of a lane's chunk from the aligned block's base in its region.
__device__ __forceinline__ uint32_t aligned_off(int region, LanePart lp, int hkv) {
    switch (region) {
        case 0: return lp.off + lp.slot * ROW_BYTES;
        case 1: return lp.off + lp.slot * 4;
        case 2: return lp.off + lp.slot * (uint32_t)(hkv * PG * 2);
        case 3: return lp.off + lp.slot * (uint32_t)(hkv * PG * ROW_BYTES);
        default: return lp.off + lp.slot * (uint32_t)(hkv * 2 * VGROUPS * PG * 2);
    }
}

// Issue one planned load of a block into stage `st` (LDS byte address):
// region and lds are wave-uniform; aoff is the lane's aligned offset and lp its
// (slot, offset) for a block whose pages are not an aligned group.
__device__ __forceinline__ void issue(int region, uint32_t lds_rel, uint32_t aoff, LanePart lp, const BlockPages &bp,
                                      const BlockBase &bb, const dqk_cache &c, int g, int hkv, uint32_t st) {
    const uint32_t lds = st + lds_rel;
    if (bp.aligned) {  // wave-uniform
        switch (region) {
            case 0: dma16_s(bb.kc, aoff, lds); break;
            case 1: dma4_s(bb.km, aoff, lds); break;
            case 2: dma16_s(bb.k0, aoff, lds); break;
            case 3: dma16_s(bb.vc, aoff, lds); break;
            default: dma16_s(bb.vm, aoff, lds); break;
        }
        return;
    }
    const int64_t p = lp.slot == 0 ? bp.p[0] : lp.slot == 1 ? bp.p[1] : lp.slot == 2 ? bp.p[2] : bp.p[3];
    const uint64_t pg = (uint64_t)p * hkv + g;
    const uint64_t kr = (uint64_t)((p >> 2) * hkv + g) * (D * KBLK) + (uint64_t)(p & 3);  // key row index, channel 0
    switch (region) {
        case 0: dma16_v((uint64_t)(uintptr_t)c.k_codes + kr * ROW_BYTES + lp.off, lds); break;
        case 1: dma4_v((uint64_t)(uintptr_t)c.k_meta + kr * 4 + lp.off, lds); break;
        case 2: dma16_v((uint64_t)(uintptr_t)c.k_ch0 + pg * (PG * 2) + lp.off, lds); break;
        case 3: dma16_v((uint64_t)(uintptr_t)c.v_codes + pg * (PG * ROW_BYTES) + lp.off, lds); break;
        default: dma16_v((uint64_t)(uintptr_t)c.v_meta + pg * (2 * VGROUPS * PG * 2) + lp.off, lds); break;
    }
}

// ---------------------------------------------------------------- the kernel
template <int KS>
__global__ __launch_bounds__(NTHR) void decode_blk_kernel(dqk_cache c, const float *__restrict__ q_prime,
                                                          const int32_t *__restrict__ sel_idx, int n_keep, int hq,
                                                          const int32_t *__restrict__ page_table, int max_pages,
                                                          const int32_t *__restrict__ seq_lens, float sm_scale,
                                                          int nsplit, float *__restrict__ partials) {
    using Ly = Lay<KS>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Ly::TOTAL];
    const uint32_t S = lds_addr(smem);

    const int split = blockIdx.x, bg = blockIdx.y;
    const int hkv = c.num_kv_heads;
    const int b = bg / hkv, g = bg - b * hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wv & 3, hf = wv >> 2;  // page slot and token half of this wave
    const int G = lane >> 4, n = lane & 15;
    const int L = seq_lens[b];
    const int npages = (L + PG - 1) / PG;
    const int nblk = (npages + 3) >> 2;
    const int per = (nblk + nsplit - 1) / nsplit;
    const int B0 = min(nblk, split * per), B1 = min(nblk, B0 + per);
    const int nst = B1 - B0;
    const int32_t *ptab = page_table + (size_t)b * max_pages;
    auto stage = [&](int u) { return S + (uint32_t)(u % NSTAGE) * Ly::STAGE; };
    float *part_base = partials + (((size_t)b * hq + (size_t)g * GRP) * nsplit + split) * PART_FLOATS;
    const size_t hstride = (size_t)nsplit * PART_FLOATS;

    if (nst <= 0) {  // nothing of this sequence falls in this split: an empty partial
        const int h = tid >> 7, ch = tid & (D - 1);
        part_base[h * hstride + ch] = 0.0f;
        if (ch == 0) {
            part_base[h * hstride + D] = -__builtin_huge_valf();
            part_base[h * hstride + D + 1] = 0.0f;
            part_base[h * hstride + D + 2] = 0.0f;
        }
        return;
    }

    // ---- q' of the four heads and the selected channels into LDS (stage 2, free until step 0)
    const uint32_t scr = stage(2);
    {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(q_prime + ((size_t)b * hq + (size_t)g * GRP) * D);
        const int32_t *ssrc = sel_idx + ((size_t)b * hkv + g) * n_keep;
        if (tid < 128) lds_st<u32x4>(scr + tid * 16, qsrc[tid]);
        if (tid < 128) lds_st<int32_t>(scr + GRP * D * 4 + tid * 4, tid < n_keep ? ssrc[tid] : 0);
        // constant areas: zeros for the off-diagonal q~ fragments, fp16 ones / zeros
        for (int i = tid; i < KS * 64; i += NTHR) lds_st<uint32_t>(S + Ly::ZERO + i * 4, 0u);
        if (tid < 8) lds_st<uint32_t>(S + Ly::ONES + tid * 4, tid < 4 ? 0x3C003C00u : 0u);
    }
    __syncthreads();
    auto qv = [&](int h, int j) { return lds_ld<float>(scr + (h * D + j) * 4); };
    const int has0 = lds_ld<int32_t>(scr + GRP * D * 4) == 0;  // the list is ascending
    const int R = n_keep - has0;                                 // selected INT2 channels
    // channel of key row slot r (rows past R read row 0, which is zero)
    auto chan_of = [&](int r) { return r < R ? lds_ld<int32_t>(scr + GRP * D * 4 + (r + has0) * 4) : 0; };

    // ---- load plans (the same for every block): this wave issues key
    //      instructions wv + 8k (a wave past the end repeats a real load: same
    //      bytes, same place) and value instructions wv + 8k
    uint32_t kaoff[Ly::KN], kchan[Ly::KN], vaoff[Ly::VN];
#pragma unroll
    for (int k = 0; k < Ly::KN; ++k) {
        const int idx = (wv + NW * k) % Ly::NKI;
        kchan[k] = (uint32_t)chan_of(key_row<KS>(idx, lane));
        kaoff[k] = aligned_off(key_region<KS>(idx), key_part<KS>(idx, lane, (int)kchan[k]), hkv);
    }
#pragma unroll
    for (int k = 0; k < Ly::VN; ++k) {
        const int idx = wv + NW * k;
        vaoff[k] = aligned_off(val_region(idx), val_part(idx, lane), hkv);
    }
    auto issue_keys = [&](const BlockPages &bp, const BlockBase &bb, uint32_t st) {
#pragma unroll
        for (int k = 0; k < Ly::KN; ++k) {
            const int idx = (wv + NW * k) % Ly::NKI;
            issue(key_region<KS>(idx), key_lds<KS>(idx), kaoff[k], bp.aligned ? LanePart{0, 0} : key_part<KS>(idx, lane, (int)kchan[k]),
                  bp, bb, c, g, hkv, st);
        }
    };
    auto issue_vals = [&](const BlockPages &bp, const BlockBase &bb, uint32_t st) {
#pragma unroll
        for (int k = 0; k < Ly::VN; ++k) {
            const int idx = wv + NW * k;
            issue(val_region(idx), val_lds<KS>(idx), vaoff[k], bp.aligned ? LanePart{0, 0} : val_part(idx, lane), bp,
                  bb, c, g, hkv, st);
        }
    };

    // ---- per-lane constants of the q~ precompute: lane l owns dword l of every
    //      k-step: channel slots 16 ks + 8 G1 + 2 ep + {0, 1}, head hq_, limb ll_q
    const float C = sm_scale * LOG2E;
    const int G1 = lane >> 5, hq_ = (lane >> 3) & 3, llq = (lane >> 2) & 1, ep = lane & 3;
    uint32_t QH[KS], QL[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        half2v h, l;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 16 * ks + 8 * G1 + 2 * ep + u;
            const float v = r < R ? qv(hq_, chan_of(r)) * C : 0.0f;
            const _Float16 vh = (_Float16)v;
            const _Float16 vl = (_Float16)(v - (float)vh);
            h[u] = llq ? vh : (_Float16)0.0f;
            l[u] = llq ? vl : vh;
        }
        QH[ks] = as_u32(h);
        QL[ks] = as_u32(l);
    }
    // score lanes: column n = (tg, head hh, limb ll); rows 4G + r
    const int tg = n >> 3, hh = (n >> 1) & 3, ll = n & 1;
    const float q0c = has0 ? qv(hh, 0) * C : 0.0f;
    __syncthreads();  // every wave is done with the scratch in stage 2

    // score A reads: word 4 tg_a + (n >> 2) of the wave's 16 bytes of each row
    const int tga = G >> 1;
    const uint32_t ka_base = Ly::KC + (8 * (G & 1)) * 128 + (((2 * w + hf) ^ (G & 1)) * 16) +
                             2 * (4 * tga + (n >> 2));
    const uint32_t amask = 0x00030003u << (2 * (n & 3));
    // score B reads: the q~ fragment (or zeros off the token-group diagonal)
    const uint32_t qt_w = S + Ly::QT + wv * (KS * 256);
    const uint32_t qb_lane = (tga == tg ? qt_w : S + Ly::ZERO) + ((G & 1) * 8 + (n & 7)) * 16;
    // ch0 / P write: tokens 32 tg + 8 G + 4 ll + r of the wave's 64
    const int tok4 = 32 * tg + 8 * G + 4 * ll;
    const uint32_t pb_w = S + Ly::PB + wv * Ly::PBW;
    // value lanes: row (q, h) = (n >> 2, n & 3); k = tokens 32 ps + 8 G + e of the wave's 64
    const int qv_ = n >> 2, hv = n & 3;
    const uint32_t pr_lane = pb_w + hv * 144 + 16 * G;                               // + 64 ps
    const uint32_t sp_lane = Ly::VM + w * 2048 + qv_ * 256 + (((8 * hf + G) ^ qv_) * 16);  // + 64 ps
    const int cz = n & 3;
    const uint32_t bz_lane = cz == 0 ? sp_lane + 1024 : cz == 2 ? sp_lane : 0u;       // stage-relative (0: constant)
    const uint32_t bz_const = S + Ly::ONES + (cz == 1 ? 0u : 16u);
    const uint32_t vc_lane = Ly::VC + w * 4096 + (64 * hf + 8 * G) * 32 + 2 * n;      // + 1024 ps + 32 e
    half8 M15;
    {
        const _Float16 m = (_Float16)(cz == 3 ? -1.5f : 0.0f);
        M15 = half8{m, m, m, m, m, m, m, m};
    }

    // ---- state
    float m_run = -__builtin_huge_valf();  // integer running maximum (log2 units) of head hh
    float l32 = 0.0f;                      // fp32 sum of 2^(x - m) over this lane's tokens of head hh
    int e_run = EMIN;                      // running exponent of the value scales
    f32x4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 Oz = {0.f, 0.f, 0.f, 0.f};

    // ---- prologue loads: keys of block 0, values of block 0, keys of block 1
    auto blk_info = [&](int u, BlockPages &bp, BlockBase &bb) {
        bp = block_pages(ptab, B0 + u, npages);
        bb = block_base(c, bp.p[0] >> 2, g, hkv);
    };
    {
        BlockPages bp;
        BlockBase bb;
        blk_info(0, bp, bb);
        issue_keys(bp, bb, stage(0));
        issue_vals(bp, bb, stage(0));
        if (nst > 1) {
            blk_info(1, bp, bb);
            issue_keys(bp, bb, stage(1));
        }
    }

    const float comp[4] = {16777216.0f, 4194304.0f, 1048576.0f, 262144.0f};  // 2^(24 - 2r)

    for (int u = 0; u <= nst; ++u) {
        // loads issued at the previous step may stay in flight
        const int pend = (u + 1 < nst ? Ly::KN : 0) + (u < nst ? Ly::VN : 0);
        if (pend == Ly::KN + Ly::VN)
            wait_vm_barrier<Ly::KN + Ly::VN>();
        else if (pend == Ly::VN)
            wait_vm_barrier<Ly::VN>();
        else
            wait_vm_barrier<0>();
        // keys of block u + 2, values of block u + 1
        if (u + 2 < nst) {
            BlockPages bp;
            BlockBase bb;
            blk_info(u + 2, bp, bb);
            issue_keys(bp, bb, stage(u + 2));
        }
        if (u + 1 < nst) {
            BlockPages bp;
            BlockBase bb;
            blk_info(u + 1, bp, bb);
            issue_vals(bp, bb, stage(u + 1));
        }

        const uint32_t sk = stage(u), sv = stage(u + NSTAGE - 1);  // keys of block u, values of block u - 1
        // valid tokens of this wave in the scored block and in the multiplied block
        const int nv_s = u < nst ? min(64, max(0, L - PG * (4 * (B0 + u) + w) - 64 * hf)) : 0;
        const int nv_v = u >= 1 ? min(64, max(0, L - PG * (4 * (B0 + u - 1) + w) - 64 * hf)) : 0;

        // ---- q~ of the scored page into this wave's LDS area, and the bias sum_j z_j C q'_j
        float bias = 0.0f;
        if (nv_s > 0) {
            float zsum = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int r0 = 16 * ks + 8 * G1 + 2 * ep;
                const uint32_t d0 = lds_ld<uint32_t>(sk + Ly::KM + r0 * 16 + w * 4);
                const uint32_t d1 = lds_ld<uint32_t>(sk + Ly::KM + (r0 + 1) * 16 + w * 4);
                const half2v s2 = as_half2(__builtin_amdgcn_perm(d1, d0, 0x05040100u));
                const half2v qh = as_half2(QH[ks]), ql = as_half2(QL[ks]);
                const half2v t1 = qh * s2;
                const half2v t2 = __builtin_elementwise_fma(qh, s2, -t1);
                lds_st<uint32_t>(qt_w + ks * 256 + lane * 4, as_u32(__builtin_elementwise_fma(ql, s2, t2)));
                // z . (hi + lo) of the two channels, exact products, fp32 sums
                const half2v z2 = as_half2(__builtin_amdgcn_perm(d1, d0, 0x07060302u));
                zsum = __builtin_amdgcn_fdot2(z2, ql, __builtin_amdgcn_fdot2(z2, qh, zsum, false), false);
            }
            if (!llq) zsum = 0.0f;  // limb-0 lanes hold (0, hi) only
            // sum over the lanes of head hq_: bits 0, 1 (ep), 2 (limb), 5 (G1)
            zsum += dpp<DPP_XOR1>(zsum);
            zsum += dpp<DPP_XOR2>(zsum);      // every lane of a quad holds the quad's sum
            zsum += dpp<DPP_HMIRROR>(zsum);   // plus the other quad of its 8
            zsum = sum_x32(zsum);
            // lane 8h holds head h's bias
            const float b0 = bcast_lane(zsum, 0), b1 = bcast_lane(zsum, 8), b2 = bcast_lane(zsum, 16),
                        b3 = bcast_lane(zsum, 24);
            bias = hh == 0 ? b0 : hh == 1 ? b1 : hh == 2 ? b2 : b3;
        }
        wait_lgkm0();  // q~ written (and the previous step's P stores done)

        // ---- value-scale exponent of the multiplied page; rescale O when it grows
        u32x4 spv[2], keep[2];
        if (nv_v > 0) {
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                spv[ps] = lds_ld<u32x4>(sv + sp_lane + 64 * ps);
                keep[ps] = u32x4{~0u, ~0u, ~0u, ~0u};
            }
            if (nv_v < 64) {  // metadata past the sequence end is unspecified: keep it out of everything
#pragma unroll
                for (int ps = 0; ps < 2; ++ps)
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int t = 32 * ps + 8 * G + 2 * e2;
                        keep[ps][e2] = (t < nv_v ? 0x0000FFFFu : 0u) | (t + 1 < nv_v ? 0xFFFF0000u : 0u);
                    }
#pragma unroll
                for (int ps = 0; ps < 2; ++ps) spv[ps] &= keep[ps];
            }
            uint32_t mx = 0;
#pragma unroll
            for (int ps = 0; ps < 2; ++ps)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = spv[ps][e];
                    mx = max(mx, max(x & 0xFFFFu, x >> 16));
                }
            mx = max(mx, dpp_u<DPP_ROR4>(mx));
            mx = max(mx, dpp_u<DPP_ROR8>(mx));
            mx = umax_x32(umax_x16(mx));
            const int ex = (int)((mx >> 10) & 31u);
            const int e_pg = min(EMAX, max(EMIN, ex == 0 ? EMIN : ex - 15));
            if (e_pg > e_run) {  // wave-uniform
                const float f = __uint_as_float((uint32_t)(127 + e_run - e_pg) << 23);
#pragma unroll
                for (int t = 0; t < 8; ++t) O[t] *= f;
                if (cz == 3) Oz *= f;
                e_run = e_pg;
            }
        }
        const uint32_t sc_h = pow2_h(-e_run);
        const half2v sc2 = as_half2(sc_h | (sc_h << 16));

        // ---- scores of the scored page and value products of the multiplied page
        f32x4 Sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (nv_s > 0) {
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                const uint32_t ka = sk + ka_base + (16 * i) * 128;
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) X[e2] = lds_pair(ka + (2 * e2) * 128, ka + (2 * e2 + 1) * 128);
                const u32x4 Bq = lds_ld<u32x4>(qb_lane + i * 256);
                const u32x4 A0 = X & amask, A1 = (X >> 8) & amask;
                Sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(A0), as_half8(Bq), Sc[0], 0, 0, 0);
                Sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(A1), as_half8(Bq), Sc[1], 0, 0, 0);
            }
        }
        if (nv_v > 0) {
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const u32x4 Pp = lds_ld<u32x4>(pr_lane + 64 * ps);
                const u32x4 sp = spv[ps];
                u32x4 Bz = lds_ld<u32x4>(bz_lane ? sv + bz_lane + 64 * ps : bz_const);
                if (nv_v < 64) Bz &= keep[ps];
                u32x4 A;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) A[e2] = as_u32(as_half2(Pp[e2]) * (as_half2(sp[e2]) * sc2));
                const uint32_t vb = sv + vc_lane + 1024 * ps;
                u32x4 X;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) X[e2] = lds_pair(vb + (2 * e2) * 32, vb + (2 * e2 + 1) * 32);
                const half8 Ah = as_half8(A);
                Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(Pp), as_half8(Bz), Oz, 0, 0, 0);
                Oz = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, M15, Oz, 0, 0, 0);
                const u32x4 XR = X >> 6;
                O[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(X & 0x00030003u), O[0], 0, 0, 0);
                O[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(X & 0x000C000Cu), O[1], 0, 0, 0);
                O[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(X & 0x00300030u), O[2], 0, 0, 0);
                O[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(X & 0x00C000C0u), O[3], 0, 0, 0);
                O[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(X & 0x03000300u), O[4], 0, 0, 0);
                O[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XR & 0x00300030u), O[5], 0, 0, 0);
                O[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XR & 0x00C000C0u), O[6], 0, 0, 0);
                O[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, as_half8(XR & 0x03000300u), O[7], 0, 0, 0);
            }
        }
        if (nv_s <= 0) continue;

        // ---- logits (log2 units) of 4 tokens: tile ll of this lane, joined with the other limb
        float x[4];
        {
            const u32x2 k0 = lds_ld<u32x2>(sk + Ly::K0 + w * 256 + (64 * hf + tok4) * 2);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mine = ll ? Sc[1][r] : Sc[0][r];
                const float give = ll ? Sc[0][r] : Sc[1][r];
                float v = __builtin_fmaf(mine + dpp<DPP_XOR1>(give), comp[r], bias);
                const uint32_t kw = k0[r >> 1];
                v = __builtin_fmaf(q0c, __uint_as_float((r & 1) ? (kw & 0xFFFF0000u) : (kw << 16)), v);
                x[r] = (tok4 + r < nv_s) ? v : -__builtin_huge_valf();
            }
        }
        // ---- integer running maximum of head hh
        float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        bm = fmaxf(bm, dpp<DPP_XOR1>(bm));
        bm = fmaxf(bm, dpp<DPP_ROR8>(bm));
        bm = max_x32(max_x16(bm));
        const float m_new = fmaxf(m_run, ceilf(bm));
        if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {  // O holds pages up to u - 1
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // head hh; 0 when m_run = -inf
            float a[GRP];
#pragma unroll
            for (int h = 0; h < GRP; ++h) a[h] = bcast_lane(alpha, 2 * h);  // lane 2h: column (0, h, 0)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[t][r] *= a[r];
#pragma unroll
            for (int r = 0; r < 4; ++r) Oz[r] *= a[r];
            l32 *= alpha;
        }
        m_run = m_new;
        // ---- probabilities 2^(x - m + 14) -> fp16 -> this wave's P buffer
        {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - m_new + (float)PBOOST);
            l32 += (p[0] + p[1]) + (p[2] + p[3]);
            half2v h01, h23;
            h01[0] = (_Float16)p[0];
            h01[1] = (_Float16)p[1];
            h23[0] = (_Float16)p[2];
            h23[1] = (_Float16)p[3];
            lds_st<u32x2>(pb_w + hh * 144 + tok4 * 2, u32x2{as_u32(h01), as_u32(h23)});
        }
    }

    // ---- this wave's partials: lanes with n >> 2 == G hold channels 8n + t of group G
    //      for heads r = 0..3; columns 4G + c of Oz hold the group's sums
    float col[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        col[0][r] = dpp<DPP_QB<0>>(Oz[r]);
        col[1][r] = dpp<DPP_QB<1>>(Oz[r]);
        col[2][r] = dpp<DPP_QB<2>>(Oz[r]);
        col[3][r] = dpp<DPP_QB<3>>(Oz[r]);
    }
    // l32 of head hh: sum over its 16 lanes (G, tg, ll)
    float l32h = l32 + dpp<DPP_XOR1>(l32);
    l32h += dpp<DPP_ROR8>(l32h);
    l32h = sum_x32(sum_x16(l32h));
    const float escale = __uint_as_float((uint32_t)(127 + e_run) << 23);
    __syncthreads();  // every wave is done with the stages: reuse stage 0 for the exchange
    // exchange: [wave][head][o[128], m, l, l32, pad] floats
    const uint32_t xw = S + (uint32_t)wv * (GRP * PART_FLOATS * 4);
    if ((n >> 2) == G) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float o = __builtin_fmaf(escale, __builtin_fmaf(O[t][r], t < 5 ? (16777216.0f / (float)(1u << (2 * t))) : (16777216.0f / (float)(1u << (2 * t - 6))), col[3][r]),
                                               __builtin_fmaf(1.5f, col[2][r], col[0][r]));
                lds_st<float>(xw + (r * PART_FLOATS + 8 * n + t) * 4, o);
            }
        if (n == 4 * G) {  // one lane per row block: l = sum P (column 1)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r == G) lds_st<float>(xw + (r * PART_FLOATS + D + 1) * 4, col[1][r]);
        }
    }
    if (lane < 8 && (lane & 1) == 0) {  // lane 2h: column (0, h, 0): m and l32 of head h
        const int h = lane >> 1;
        lds_st<float>(xw + (h * PART_FLOATS + D) * 4, m_run);
        lds_st<float>(xw + (h * PART_FLOATS + D + 2) * 4, l32h);
    }
    __syncthreads();
    // combine the eight waves: thread (h, ch)
    {
        const int h = tid >> 7, ch = tid & (D - 1);
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, lds_ld<float>(S + ((v * GRP + h) * PART_FLOATS + D) * 4));
        float o = 0.0f, l = 0.0f, l3 = 0.0f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const uint32_t base = S + (uint32_t)((v * GRP + h) * PART_FLOATS) * 4;
            const float mv = lds_ld<float>(base + D * 4);
            const float f = mv == -__builtin_huge_valf() ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
            o = __builtin_fmaf(lds_ld<float>(base + ch * 4), f, o);
            if (ch == 0) {
                l = __builtin_fmaf(lds_ld<float>(base + (D + 1) * 4), f, l);
                l3 = __builtin_fmaf(lds_ld<float>(base + (D + 2) * 4), f, l3);
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

bool use_mfma_decode(int hq, int hkv) { return hkv > 0 && hq == GRP * hkv; }

static int ks_of(int n_keep) {
    const int k = (n_keep + 15) / 16;
    return k < 1 ? 1 : k > 8 ? 8 : k;
}

int decode_splits_mfma(int batch, int hkv, int max_pages, int n_keep) {
    (void)n_keep;
    // one 8-wave workgroup per CU (LDS-bound): enough splits to give each of the
    // 256 CUs one, at least 8 blocks per split; long contexts split so that no
    // split exceeds 32 blocks (ragged batches stay balanced)
    const int units = batch * hkv;
    const int nblk = (max_pages + 3) / 4;
    int s = (256 + units - 1) / units;
    const int cap = (nblk + 7) / 8;
    if (s > cap) s = cap;
    const int need = (nblk + 31) / 32;
    if (s < need) s = need;
    if (s > nblk) s = nblk;
    return s < 1 ? 1 : s;
}

template <int KS>
static hipError_t launch_ks(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(a.num_splits, a.batch * a.hkv);
    hipLaunchKernelGGL(decode_blk_kernel<KS>, grid, dim3(NTHR), 0, s, *a.c, a.q_prime, a.sel_idx, a.n_keep, a.hq,
                       a.page_table, a.max_pages, a.seq_lens, a.sm_scale, a.num_splits, a.partials);
    return hipGetLastError();
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
