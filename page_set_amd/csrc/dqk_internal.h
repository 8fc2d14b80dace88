// Internal declarations shared by libdqk's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqk.h"

namespace dqk {

constexpr int D = DQK_HEAD_DIM;
constexpr int PG = DQK_PAGE;
constexpr int ROW_BYTES = 32;     // 128 two-bit codes
constexpr int VGROUPS = 4;        // value groups of 32 channels

// Partial of one (b, h, split): o[128] (unnormalised, relative to m), m, l.
constexpr int PART_FLOATS = D + 2;

// ---------------------------------------------------------------- formats
// binary16 bits -> fp32 (exact).
__device__ __forceinline__ float h2f(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf_rne(float x) {
    uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// |x| onto the binary16 grid toward zero: bits of the magnitude, and whether
// the value was inexact.  Magnitudes above 65504 saturate to 65504 (inexact).
__device__ __forceinline__ uint32_t f16_mag_trunc(uint32_t ua, bool &inexact) {
    // ua: fp32 bits with the sign cleared
    if (ua > 0x477FE000u) {  // 65504.0f
        inexact = true;
        return 0x7BFFu;
    }
    int e = (int)(ua >> 23) - 127;
    if (e >= -14) {
        uint32_t m = ua & 0x7FFFFFu;
        inexact = (m & 0x1FFFu) != 0;
        return ((uint32_t)(e + 15) << 10) | (m >> 13);
    }
    // below the binary16 normal range: multiples of 2^-24
    float a = __uint_as_float(ua) * 16777216.0f;  // exact power-of-two scaling
    float fl = floorf(a);
    inexact = fl != a;
    return (uint32_t)fl;
}

// Largest binary16 <= x, and smallest binary16 >= x.  Sign of zero follows x.
__device__ __forceinline__ uint16_t f16_round_down(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 16) & 0x8000u;
    bool inexact;
    uint32_t m = f16_mag_trunc(u & 0x7FFFFFFFu, inexact);
    if (s && inexact) m += 1;  // negative: move the magnitude up
    return (uint16_t)(s | m);
}

__device__ __forceinline__ uint16_t f16_round_up(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 16) & 0x8000u;
    bool inexact;
    uint32_t m = f16_mag_trunc(u & 0x7FFFFFFFu, inexact);
    if (!s && inexact) m += 1;
    return (uint16_t)(s | m);
}

// INT2 grid of a group from its min and max (signed zeros taken as +0).
struct Grid {
    float s, z;
    uint16_t sb, zb;
};

__device__ __forceinline__ Grid make_grid(float mn, float mx) {
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    Grid g;
    g.zb = f16_round_down(mn);
    g.z = h2f(g.zb);
    float d = __fsub_rn(mx, g.z);
    float t = __fdiv_rn(d, 3.0f);
    g.sb = f16_round_up(t);
    g.s = h2f(g.sb);
    return g;
}

struct Thresholds {
    float t0, t1, t2;
};

__device__ __forceinline__ Thresholds thresholds(const Grid &g) {
    return {__builtin_fmaf(0.5f, g.s, g.z), __builtin_fmaf(1.5f, g.s, g.z), __builtin_fmaf(2.5f, g.s, g.z)};
}

__device__ __forceinline__ uint32_t code2(float x, const Thresholds &t) {
    return (uint32_t)(x >= t.t0) + (uint32_t)(x >= t.t1) + (uint32_t)(x >= t.t2);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_select(const uint16_t *q, const float *t_q, int batch, int hq, int hkv, int n_keep, float *q_prime,
                         int32_t *sel_idx, hipStream_t s);

hipError_t launch_append(const dqk_cache &c, const uint16_t *k, const uint16_t *v, const uint16_t *t_k, int n_seqs,
                         const int32_t *cu_tokens, const int32_t *page_table, int max_pages, float *kprime_dbg,
                         hipStream_t s);

struct DecodeArgs {
    const dqk_cache *c;
    const float *q_prime;
    const int32_t *sel_idx;
    int n_keep, batch, hq, hkv;
    const int32_t *page_table;
    int max_pages;
    const int32_t *seq_lens;
    float sm_scale;
    int num_splits;
    float *partials;
    float *out, *lse;
};

// Generic path: any group size up to 16.
constexpr int GENERIC_MAX_GROUP = 16;
int decode_splits_generic(int batch, int hkv, int max_pages);
hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s);

// MFMA path (group size 4, the GQA 32/8 shape).
bool use_mfma_decode(int hq, int hkv);
int decode_splits_mfma(int batch, int hkv, int max_pages, int n_keep);  // n_keep 0: the largest
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s);

struct DecodeBf16Args {
    const uint16_t *k_pages, *v_pages;
    int hkv;
    const uint16_t *q;
    int batch, hq;
    const int32_t *page_table;
    int max_pages;
    const int32_t *seq_lens;
    float sm_scale;
    int num_splits;
    float *partials;
    float *out, *lse;
};

hipError_t launch_decode_bf16(const DecodeBf16Args &a, hipStream_t s);

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);

hipError_t launch_merge(const float *partials, int batch, int hq, int num_splits, float *out, float *lse,
                        hipStream_t s);

}  // namespace dqk
