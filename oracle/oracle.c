/*
 * oracle.c -- plain CPU reference for Dual-QK decode attention over a 2-bit
 * KV cache, written from "Dual-QK: Sharp Queries and Flat Keys for Prunable
 * 2-bit KV Caches" (Whang, Oh, Kim, Seo).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the HIP library; both follow the same written format
 * specification independently.
 *
 * Built with -O2 -std=c99 -ffp-contract=off and no intrinsics, so every
 * float operation rounds exactly as written: fmaf only where the format says
 * fma, fp64 wherever the method leaves the precision open.
 *
 * Conventions (row vectors, as in Eq. 1 of §3.1): q' = q T_Q, k' = k T_K,
 * T[i][j] with i the input and j the output channel.  d = 128, pages of 128
 * tokens.  Query head h uses KV head h / (Hq/Hkv).
 *
 * Cache format (all little-endian).  Physical pages come in aligned blocks
 * of eight (page p is slot p & 7 of block p >> 3); per block B, KV head g:
 *   k_codes u8   [P/8][Hkv][128 ch][8 slot][32]  channel-major rows (§3.3: one
 *                                       channel of one page per contiguous
 *                                       32-byte row); the eight pages' rows of
 *                                       a channel are adjacent.  Token t at
 *                                       byte t>>2, bits 2*(t&3).  Row 0 zero.
 *   k_meta  f16  [P/8][Hkv][128 ch][8 slot][2]  (scale, zero) per channel and
 *                                       page; channel 0 entries zero.
 * and per physical page p:
 *   k_ch0   bf16 [P][Hkv][128 tok]     channel 0 of k' kept in bf16 (§3.3).
 *   v_codes u8   [P][Hkv][128 tok][32] token-major (§3.3); channel c at byte
 *                                       c>>2, bits 2*(c&3).
 *   v_meta  f16  [P][Hkv][2][4][128]   [0][grp][tok] = scale, [1][grp][tok] =
 *                                       zero, per token and 32-channel group.
 *
 * Parity status of each function is listed in the oracle's Python header.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HD 128
#define PG 128
#define VGROUP 32

/* Index of the 32-byte key row (and of the 2-entry key metadata) of channel j
 * of physical page p, KV head g: block p >> 3, slot p & 7. */
static size_t krow(int64_t p, int g, int hkv, int j)
{
    return ((((size_t)(p >> 3) * (size_t)hkv + (size_t)g) * HD + (size_t)j) * 8) + (size_t)(p & 7);
}

/* Per-token key grid (§3.3 as the paper states it, one grid per token and KV
 * head over channels 1..127): the (scale, zero) pair of token s of page p in
 * k_meta, laid out [P/8][Hkv][8 slot][128 tok][2] -- the same bytes as the
 * per-channel metadata of the block, token-major. */
static size_t ktok(int64_t p, int g, int hkv, int s)
{
    return (((size_t)(p >> 3) * (size_t)hkv + (size_t)g) * 8 + (size_t)(p & 7)) * PG + (size_t)s;
}

/* ------------------------------------------------------------------------ */
/* Number formats, from their IEEE 754 definitions (binary16; bfloat16 is the
 * top half of binary32).  Values are handled as exact doubles.              */

double orc_f16_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* Encode a double that is exactly a binary16 value (or +-inf). */
static uint16_t f16_encode(double v)
{
    uint16_t s = 0;
    if (signbit(v)) {
        s = 0x8000;
        v = -v;
    }
    if (isinf(v))
        return s | 0x7C00;
    if (v == 0.0)
        return s;
    if (v < ldexp(1.0, -14))
        return s | (uint16_t)(v * ldexp(1.0, 24));
    int e;
    double fr = frexp(v, &e); /* v = fr * 2^e, fr in [0.5, 1) */
    uint16_t m = (uint16_t)((fr * 2.0 - 1.0) * 1024.0);
    return s | (uint16_t)((e - 1 + 15) << 10) | m;
}

/* Spacing of the binary16 grid at magnitude a (0 <= a <= 65504). */
static double f16_spacing(double a)
{
    if (a < ldexp(1.0, -14))
        return ldexp(1.0, -24);
    int e;
    frexp(a, &e);
    return ldexp(1.0, e - 1 - 10);
}

static double f16_mag_down(double a)
{
    if (a > 65504.0)
        return 65504.0;
    double u = f16_spacing(a);
    return floor(a / u) * u;
}

static double f16_mag_up(double a)
{
    if (a > 65504.0)
        return INFINITY;
    double t = f16_mag_down(a);
    return t == a ? a : t + f16_spacing(a);
}

/* Largest binary16 <= x (sign of zero follows x). */
uint16_t orc_f16_round_down(float x)
{
    double a = (double)x;
    return f16_encode(signbit(a) ? -f16_mag_up(-a) : f16_mag_down(a));
}

/* Smallest binary16 >= x (sign of zero follows x). */
uint16_t orc_f16_round_up(float x)
{
    double a = (double)x;
    return f16_encode(signbit(a) ? -f16_mag_down(-a) : f16_mag_up(a));
}

float orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Nearest bfloat16 (8 significant bits, binary32 exponent range), ties to
 * even significand. */
uint16_t orc_bf16_round_nearest(float x)
{
    double a = fabs((double)x);
    uint16_t s = signbit(x) ? 0x8000 : 0;
    if (a == 0.0)
        return s;
    double u;
    if (a < ldexp(1.0, -126)) {
        u = ldexp(1.0, -133);
    } else {
        int e;
        frexp(a, &e);
        u = ldexp(1.0, e - 1 - 7);
    }
    double q = a / u, r = floor(q), f = q - r;
    if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) == 1.0))
        r += 1.0;
    double v = r * u;
    if (v > 3.3895313892515355e38) /* largest finite bfloat16 */
        return s | 0x7F80;
    float fv = (float)v; /* exact: v is a bfloat16 value */
    uint32_t bits;
    memcpy(&bits, &fv, 4);
    return s | (uint16_t)((bits >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------------------ */
/* Asymmetric INT2 grid (§3.3 and App. B.2: one asymmetric 2-bit grid per
 * group, keys not clipped).  Levels z + c*s, c = 0..3.  z is the group
 * minimum rounded down to binary16 and s = fp32((max - z)/3) rounded up to
 * binary16, so [min, max] lies inside [z, z + 3s] up to fp32 rounding.  The
 * code is the number of thresholds fmaf(c + 0.5, s, z), c = 0..2, that the
 * value reaches (a value on a threshold takes the upper level).            */

typedef struct {
    uint16_t s_bits, z_bits;
    float s, z;
} grid_t;

/* clip scales both ends of the group range toward zero before the grid is
 * fitted (1.0f leaves them as they are; values outside the clipped range take
 * code 0 or 3 by the threshold rule). */
static grid_t make_grid_clip(const float *x, int n, int stride, float clip)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        float v = x[(size_t)i * stride];
        if (v < mn)
            mn = v;
        if (v > mx)
            mx = v;
    }
    mn = clip * mn;
    mx = clip * mx;
    if (mn == 0.0f)
        mn = 0.0f; /* canonical +0 */
    if (mx == 0.0f)
        mx = 0.0f;
    grid_t g;
    g.z_bits = orc_f16_round_down(mn);
    g.z = (float)orc_f16_value(g.z_bits);
    float d = mx - g.z;
    float t = d / 3.0f;
    g.s_bits = orc_f16_round_up(t);
    g.s = (float)orc_f16_value(g.s_bits);
    return g;
}

static grid_t make_grid(const float *x, int n, int stride) { return make_grid_clip(x, n, stride, 1.0f); }

static int code_of(float x, const grid_t *g)
{
    return (x >= fmaf(0.5f, g->s, g->z)) + (x >= fmaf(1.5f, g->s, g->z)) + (x >= fmaf(2.5f, g->s, g->z));
}

/* Exposed for tests: grid and codes of one group of n fp32 values. */
void orc_quantize_group_clip(const float *x, int n, float clip, uint16_t *s_bits, uint16_t *z_bits, uint8_t *codes)
{
    grid_t g = make_grid_clip(x, n, 1, clip);
    *s_bits = g.s_bits;
    *z_bits = g.z_bits;
    for (int i = 0; i < n; ++i)
        codes[i] = (uint8_t)code_of(x[i], &g);
}

void orc_quantize_group(const float *x, int n, uint16_t *s_bits, uint16_t *z_bits, uint8_t *codes)
{
    grid_t g = make_grid(x, n, 1);
    *s_bits = g.s_bits;
    *z_bits = g.z_bits;
    for (int i = 0; i < n; ++i)
        codes[i] = (uint8_t)code_of(x[i], &g);
}

float orc_dequant(int code, uint16_t s_bits, uint16_t z_bits)
{
    return fmaf((float)code, (float)orc_f16_value(s_bits), (float)orc_f16_value(z_bits));
}

/* ------------------------------------------------------------------------ */
/* Key transform k' = k T_K (§3.1 Eq. 1; applied to each new key before it is
 * stored, §3.4).  bf16 x bf16 products summed in fp64, ascending input
 * channel, rounded once to fp32.
 *   k  bf16 [T][Hkv][128], t_k bf16 [Hkv][128][128], out fp32 [T][Hkv][128] */
void orc_key_transform(const uint16_t *k, const uint16_t *t_k, int64_t T, int hkv, float *kprime)
{
    for (int64_t t = 0; t < T; ++t)
        for (int g = 0; g < hkv; ++g) {
            const uint16_t *kr = k + ((size_t)t * hkv + g) * HD;
            const uint16_t *tg = t_k + (size_t)g * HD * HD;
            for (int j = 0; j < HD; ++j) {
                double acc = 0.0;
                for (int i = 0; i < HD; ++i)
                    acc += (double)orc_bf16_value(kr[i]) * (double)orc_bf16_value(tg[(size_t)i * HD + j]);
                kprime[((size_t)t * hkv + g) * HD + j] = (float)acc;
            }
        }
}

/* RoPE rotation of one 128-channel vector in the rotate-half pairing
 * (channel i with channel i + 64): y_i = x_i c_i - x_{i+64} s_i and
 * y_{i+64} = x_{i+64} c_i + x_i s_i, every product and sum rounded to fp32.
 * With (c_i, s_i) = (cos(a theta_i), -sin(a theta_i)) it takes a vector
 * rotated for position n to position n - a (§3.4, App. C.4).               */
static void rope_rotate(const float *x, const float *cs, const float *sn, float *y)
{
    for (int i = 0; i < HD / 2; ++i) {
        float a = x[i] * cs[i], b = x[i + HD / 2] * sn[i];
        float c = x[i + HD / 2] * cs[i], d = x[i] * sn[i];
        y[i] = a - b;
        y[i + HD / 2] = c + d;
    }
}

/* Key transform in the bucket frame (§3.4 z_n = k_n T_b B, App. C.4): token
 * t of sequence sq (bucket (t - cu_tokens[sq]) / 2048) is rotated by its
 * bucket's table, rounded to bf16 (the MFMA operand, round to nearest even),
 * then multiplied by T_K as in orc_key_transform.                           */
#define ROPE_BUCKET 2048
void orc_key_transform_rope(const uint16_t *k, const uint16_t *t_k, int n_seqs, const int32_t *cu_tokens, int hkv,
                            const float *rope_cos, const float *rope_sin, float *kprime)
{
    for (int sq = 0; sq < n_seqs; ++sq)
        for (int64_t t = cu_tokens[sq]; t < cu_tokens[sq + 1]; ++t) {
            int64_t bk = (t - cu_tokens[sq]) / ROPE_BUCKET;
            for (int g = 0; g < hkv; ++g) {
                const uint16_t *kr = k + ((size_t)t * hkv + g) * HD;
                const uint16_t *tg = t_k + (size_t)g * HD * HD;
                float x[HD], y[HD];
                uint16_t yb[HD];
                for (int i = 0; i < HD; ++i)
                    x[i] = orc_bf16_value(kr[i]);
                rope_rotate(x, rope_cos + (size_t)bk * (HD / 2), rope_sin + (size_t)bk * (HD / 2), y);
                for (int i = 0; i < HD; ++i)
                    yb[i] = orc_bf16_round_nearest(y[i]);
                for (int j = 0; j < HD; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < HD; ++i)
                        acc += (double)orc_bf16_value(yb[i]) * (double)orc_bf16_value(tg[(size_t)i * HD + j]);
                    kprime[((size_t)t * hkv + g) * HD + j] = (float)acc;
                }
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Pack transformed keys and raw values of n_seqs sequences into 128-token
 * pages (§3.3: channel-major keys with channel 0 in bf16 outside the INT2
 * range; token-major values with separate metadata).  Key groups: one grid
 * per (page, KV head, channel 1..127) over the page's valid tokens.  Value
 * groups: one grid per (token, KV head, 32 consecutive channels).  Slots of a
 * page past the sequence end get code 0, ch0 0 and metadata 0.
 *   kprime fp32 [T][Hkv][128], v bf16 [T][Hkv][128]
 *   cu_tokens [n_seqs+1], page_table [n_seqs][max_pages]                    */
static void pack_impl(const float *kprime, const uint16_t *v, const float *vf32, float vclip, int token_grid, int hkv,
                      int n_seqs, const int32_t *cu_tokens, const int32_t *page_table, int max_pages,
                      uint8_t *k_codes, uint16_t *k_meta, uint16_t *k_ch0, uint8_t *v_codes, uint16_t *v_meta)
{
    for (int sq = 0; sq < n_seqs; ++sq) {
        int64_t t0 = cu_tokens[sq], L = (int64_t)cu_tokens[sq + 1] - t0;
        int64_t npages = (L + PG - 1) / PG;
        for (int64_t pi = 0; pi < npages; ++pi) {
            int64_t p = page_table[(size_t)sq * max_pages + pi];
            int nvalid = (int)((L - pi * PG) < PG ? (L - pi * PG) : PG);
            int64_t base_tok = t0 + pi * PG;
            for (int g = 0; g < hkv; ++g) {
                size_t pg = (size_t)p * hkv + g;
                uint16_t *k0 = k_ch0 + pg * PG;
                uint8_t *vc = v_codes + pg * PG * 32;
                uint16_t *vm = v_meta + pg * 2 * 4 * PG;
                for (int j = 0; j < HD; ++j) {
                    memset(k_codes + krow(p, g, hkv, j) * 32, 0, 32);
                    size_t mi = token_grid ? ktok(p, g, hkv, j) : krow(p, g, hkv, j); /* j: token or channel */
                    k_meta[mi * 2 + 0] = 0;
                    k_meta[mi * 2 + 1] = 0;
                }
                memset(k0, 0, PG * sizeof(uint16_t));
                memset(vc, 0, PG * 32);
                memset(vm, 0, 2 * 4 * PG * sizeof(uint16_t));
                const float *kp = kprime + ((size_t)base_tok * hkv + g) * HD; /* token stride hkv*HD */
                for (int s = 0; s < nvalid; ++s)
                    k0[s] = orc_bf16_round_nearest(kp[(size_t)s * hkv * HD + 0]);
                if (!token_grid) {
                    for (int j = 1; j < HD; ++j) {
                        uint8_t *kc = k_codes + krow(p, g, hkv, j) * 32;
                        uint16_t *km = k_meta + krow(p, g, hkv, j) * 2;
                        grid_t gr = make_grid(kp + j, nvalid, hkv * HD);
                        km[0] = gr.s_bits;
                        km[1] = gr.z_bits;
                        for (int s = 0; s < nvalid; ++s) {
                            int c = code_of(kp[(size_t)s * hkv * HD + j], &gr);
                            kc[s >> 2] |= (uint8_t)(c << (2 * (s & 3)));
                        }
                    }
                } else {
                    for (int s = 0; s < nvalid; ++s) {
                        const float *kt = kp + (size_t)s * hkv * HD;
                        grid_t gr = make_grid(kt + 1, HD - 1, 1); /* channel 0 outside the range */
                        k_meta[ktok(p, g, hkv, s) * 2 + 0] = gr.s_bits;
                        k_meta[ktok(p, g, hkv, s) * 2 + 1] = gr.z_bits;
                        for (int j = 1; j < HD; ++j)
                            k_codes[krow(p, g, hkv, j) * 32 + (s >> 2)] |= (uint8_t)(code_of(kt[j], &gr) << (2 * (s & 3)));
                    }
                }
                for (int s = 0; s < nvalid; ++s) {
                    size_t row = ((size_t)(base_tok + s) * hkv + g) * HD;
                    float vf[HD];
                    for (int c = 0; c < HD; ++c)
                        vf[c] = vf32 ? vf32[row + c] : orc_bf16_value(v[row + c]);
                    for (int q = 0; q < HD / VGROUP; ++q) {
                        grid_t gr = make_grid_clip(vf + q * VGROUP, VGROUP, 1, vclip);
                        vm[(0 * 4 + q) * PG + s] = gr.s_bits;
                        vm[(1 * 4 + q) * PG + s] = gr.z_bits;
                        for (int c = q * VGROUP; c < (q + 1) * VGROUP; ++c)
                            vc[s * 32 + (c >> 2)] |= (uint8_t)(code_of(vf[c], &gr) << (2 * (c & 3)));
                    }
                }
            }
        }
    }
}

void orc_pack_cache(const float *kprime, const uint16_t *v, int hkv, int n_seqs, const int32_t *cu_tokens,
                    const int32_t *page_table, int max_pages, uint8_t *k_codes, uint16_t *k_meta, uint16_t *k_ch0,
                    uint8_t *v_codes, uint16_t *v_meta)
{
    pack_impl(kprime, v, NULL, 1.0f, 0, hkv, n_seqs, cu_tokens, page_table, max_pages, k_codes, k_meta, k_ch0,
              v_codes, v_meta);
}

/* The same pack with one key grid per token and KV head over channels
 * 1..127 (§3.3: channel 0 kept in bf16 and left out of the range of the
 * others); the per-token (scale, zero) pairs at ktok.  Values as
 * orc_pack_cache.                                                            */
void orc_pack_cache_tokgrid(const float *kprime, const uint16_t *v, int hkv, int n_seqs, const int32_t *cu_tokens,
                            const int32_t *page_table, int max_pages, uint8_t *k_codes, uint16_t *k_meta,
                            uint16_t *k_ch0, uint8_t *v_codes, uint16_t *v_meta)
{
    pack_impl(kprime, v, NULL, 1.0f, 1, hkv, n_seqs, cu_tokens, page_table, max_pages, k_codes, k_meta, k_ch0,
              v_codes, v_meta);
}

/* The same pack with rotated values (§3.3, values paragraph, and App. B.2,
 * value quantization): the values arrive already rotated, v' = v R_V in fp32
 * [T][Hkv][128] (the row-vector product of orc_key_transform with R_V in
 * place of T_K), and each (token, KV head, 32-channel group) grid is fitted
 * to the clipped range [clip * min, clip * max].  Keys are packed exactly as
 * by orc_pack_cache (keys are not clipped).                                 */
void orc_pack_cache_vrot(const float *kprime, const float *vprime, float clip, int hkv, int n_seqs,
                         const int32_t *cu_tokens, const int32_t *page_table, int max_pages, uint8_t *k_codes,
                         uint16_t *k_meta, uint16_t *k_ch0, uint8_t *v_codes, uint16_t *v_meta)
{
    pack_impl(kprime, NULL, vprime, clip, 0, hkv, n_seqs, cu_tokens, page_table, max_pages, k_codes, k_meta, k_ch0,
              v_codes, v_meta);
}

/* Inverse value rotation after aggregation (§3.4, last step): per query head
 * h of KV head g = h / (hq / hkv), out_c = sum_j o_j R_inv[g][j][c] in fp64,
 * ascending j.  o, out fp64 [B][Hq][128] (out may not alias o);
 * r_inv fp32 [Hkv][128][128].                                               */
int orc_value_unrotate(const double *o, const float *r_inv, int batch, int hq, int hkv, double *out)
{
    if (hkv <= 0 || hq % hkv)
        return -2;
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < hq; ++h) {
            const double *orow = o + ((size_t)b * hq + h) * HD;
            const float *r = r_inv + (size_t)(h / grp) * HD * HD;
            double *dst = out + ((size_t)b * hq + h) * HD;
            for (int c = 0; c < HD; ++c) {
                double acc = 0.0;
                for (int j = 0; j < HD; ++j)
                    acc += orow[j] * (double)r[(size_t)j * HD + c];
                dst[c] = acc;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Query transform and dynamic channel selection (§3.2 Eq. 4, §3.3).
 * q'_{h,j} = sum_i q_{h,i} T_Q[g][i][j] as an fp32 fma chain over ascending i.
 * Pooled energy S_j = sum over the g query heads of KV head g (ascending h) of
 * q'_{h,j}^2, fp32 fma chain; e_j = sqrt(S_j) is monotone in S_j, so channels
 * are ranked by S_j descending, ties to the lower index.  The first n_keep
 * are written in ascending channel order.
 *   q bf16 [B][Hq][128], t_q fp32 [Hkv][128][128]
 *   q_prime fp32 [B][Hq][128], sel_idx int32 [B][Hkv][n_keep]               */
/* rope_cs / rope_sn (may be NULL): per-bucket rotation tables [nb][64]; the
 * query of (b, h) for bucket k is q[b][h] rotated by table k, and the results
 * go to q_prime[b][k][h], sel_idx[b][k][g]. */
static int select_impl_rope(const uint16_t *q, const float *t_q, const float *sel_scale, const float *rope_cs,
                            const float *rope_sn, int nb, int batch, int hq, int hkv, int n_keep, float *q_prime,
                            int32_t *sel_idx)
{
    if (hkv <= 0 || hq % hkv || n_keep < 1 || n_keep > HD || nb < 1)
        return -2;
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b)
        for (int k = 0; k < nb; ++k)
        for (int g = 0; g < hkv; ++g) {
            const float *tq = t_q + (size_t)g * HD * HD;
            float S[HD];
            for (int j = 0; j < HD; ++j)
                S[j] = 0.0f;
            for (int hh = 0; hh < grp; ++hh) {
                int h = g * grp + hh;
                const uint16_t *qr = q + ((size_t)b * hq + h) * HD;
                float *qp = q_prime + (((size_t)b * nb + k) * hq + h) * HD;
                float qf[HD], qx[HD];
                for (int i = 0; i < HD; ++i)
                    qf[i] = orc_bf16_value(qr[i]);
                if (rope_cs) {
                    rope_rotate(qf, rope_cs + (size_t)k * (HD / 2), rope_sn + (size_t)k * (HD / 2), qx);
                    memcpy(qf, qx, sizeof qf);
                }
                for (int j = 0; j < HD; ++j) {
                    float acc = 0.0f;
                    for (int i = 0; i < HD; ++i)
                        acc = fmaf(qf[i], tq[(size_t)i * HD + j], acc);
                    qp[j] = acc;
                }
                for (int j = 0; j < HD; ++j) {
                    float e = sel_scale ? qp[j] * sel_scale[(size_t)g * HD + j] : qp[j];
                    S[j] = fmaf(e, e, S[j]);
                }
            }
            int32_t *out = sel_idx + (((size_t)b * nb + k) * hkv + g) * n_keep;
            int w = 0;
            for (int j = 0; j < HD; ++j) {
                int rank = 0;
                for (int jj = 0; jj < HD; ++jj)
                    if (S[jj] > S[j] || (S[jj] == S[j] && jj < j))
                        ++rank;
                if (rank < n_keep)
                    out[w++] = j;
            }
        }
    return 0;
}

static int select_impl(const uint16_t *q, const float *t_q, const float *sel_scale, int batch, int hq, int hkv,
                       int n_keep, float *q_prime, int32_t *sel_idx)
{
    return select_impl_rope(q, t_q, sel_scale, NULL, NULL, 1, batch, hq, hkv, n_keep, q_prime, sel_idx);
}

/* Selection per bucket (§3.4: each bucket's anchor adjustment is applied to
 * the current queries, then Eq. 4; masks may differ across buckets).
 * q'_{b,k,h} = (q_{b,h} rotated by table k) T_Q.
 *   rope_cos, rope_sin fp32 [n_buckets][64]
 *   q_prime fp32 [B][n_buckets][Hq][128], sel_idx int32 [B][n_buckets][Hkv][n_keep] */
int orc_select_channels_rope(const uint16_t *q, const float *t_q, const float *rope_cos, const float *rope_sin,
                             int n_buckets, int batch, int hq, int hkv, int n_keep, float *q_prime, int32_t *sel_idx)
{
    return select_impl_rope(q, t_q, NULL, rope_cos, rope_sin, n_buckets, batch, hq, hkv, n_keep, q_prime, sel_idx);
}

int orc_select_channels(const uint16_t *q, const float *t_q, int batch, int hq, int hkv, int n_keep, float *q_prime,
                        int32_t *sel_idx)
{
    return select_impl(q, t_q, NULL, batch, hq, hkv, n_keep, q_prime, sel_idx);
}

/* Selection in the base coordinates (§3.3, diagonal refinement, and App.
 * C.2): with A = A_0 D folded into T_Q, the base query q A_0 is q' D^-1, so
 * the energy of channel j sums (q'_{h,j} * sel_scale[g][j])^2 with sel_scale
 * = 1 / delta_j (the product rounded to fp32, then the same fma chain); q'
 * itself, which scores, is unchanged.  sel_scale fp32 [Hkv][128].          */
int orc_select_channels_base(const uint16_t *q, const float *t_q, const float *sel_scale, int batch, int hq, int hkv,
                             int n_keep, float *q_prime, int32_t *sel_idx)
{
    return select_impl(q, t_q, sel_scale, batch, hq, hkv, n_keep, q_prime, sel_idx);
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the paged INT2 cache (§3.2, §3.3, §3.4).  For query
 * head h of sequence b and each token t < seq_lens[b]:
 *   k^_{t,0} = bf16 channel 0;  k^_{t,j} = fmaf(code, s_j, z_j)   (fp32)
 *   logit_t  = sm_scale * sum_{j in M} q'_{h,j} k^_{t,j}            (fp64)
 * where M is the KV head's selected set and sm_scale keeps the full-width
 * 1/sqrt(d) normalisation; one softmax over all tokens (fp64, max
 * subtracted); v^_{t,c} = fmaf(code, s_{t,grp}, z_{t,grp}) (fp32);
 * out_{h,c} = sum_t p_t v^_{t,c}, lse_h = max + log(sum exp).
 *   q_prime fp32 [B][Hq][128], sel_idx [B][Hkv][n_keep],
 *   page_table [B][max_pages], out fp64 [B][Hq][128], lse fp64 [B][Hq]     */
/* nb >= 1 buckets: token t scores with q_prime[b][t / 2048][h] and the
 * selection sel_idx[b][t / 2048][g] (a token past the last bucket is an
 * error); nb = 0: one query and one mask for the whole sequence. */
static int decode_impl(const uint8_t *k_codes, const uint16_t *k_meta, const uint16_t *k_ch0, const uint8_t *v_codes,
                       const uint16_t *v_meta, int token_grid, int nb, int hkv, const float *q_prime,
                       const int32_t *sel_idx, int n_keep, int batch, int hq, const int32_t *page_table,
                       int max_pages, const int32_t *seq_lens, double sm_scale, double *out, double *lse)
{
    if (hkv <= 0 || hq % hkv || n_keep < 1 || n_keep > HD || nb < 0)
        return -2;
    const int nq = nb > 0 ? nb : 1;
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        double *logit = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        if (!logit)
            return -7;
        for (int h = 0; h < hq; ++h) {
            int g = h / grp;
            double mx = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                int64_t bk = nb > 0 ? t / ROPE_BUCKET : 0;
                if (bk >= nq) {
                    free(logit);
                    return -2;
                }
                const float *qp = q_prime + (((size_t)b * nq + bk) * hq + h) * HD;
                const int32_t *M = sel_idx + (((size_t)b * nq + bk) * hkv + g) * n_keep;
                int64_t p = page_table[(size_t)b * max_pages + (t >> 7)];
                int s = (int)(t & (PG - 1));
                size_t pg = (size_t)p * hkv + g;
                double acc = 0.0;
                for (int m = 0; m < n_keep; ++m) {
                    int j = M[m];
                    float kv;
                    if (j == 0) {
                        kv = orc_bf16_value(k_ch0[pg * PG + s]);
                    } else {
                        size_t r = krow(p, g, hkv, j);
                        size_t mi = token_grid ? ktok(p, g, hkv, s) : r;
                        int c = (k_codes[r * 32 + (s >> 2)] >> (2 * (s & 3))) & 3;
                        kv = orc_dequant(c, k_meta[mi * 2], k_meta[mi * 2 + 1]);
                    }
                    acc += (double)qp[j] * (double)kv;
                }
                logit[t] = acc * sm_scale;
                if (logit[t] > mx)
                    mx = logit[t];
            }
            double l = 0.0, o[HD];
            for (int c = 0; c < HD; ++c)
                o[c] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double pw = exp(logit[t] - mx);
                l += pw;
                int64_t p = page_table[(size_t)b * max_pages + (t >> 7)];
                int s = (int)(t & (PG - 1));
                size_t pg = (size_t)p * hkv + g;
                const uint8_t *vr = v_codes + (pg * PG + s) * 32;
                const uint16_t *vm = v_meta + pg * 2 * 4 * PG;
                for (int c = 0; c < HD; ++c) {
                    int q = c / VGROUP;
                    int code = (vr[c >> 2] >> (2 * (c & 3))) & 3;
                    float vv = orc_dequant(code, vm[(0 * 4 + q) * PG + s], vm[(1 * 4 + q) * PG + s]);
                    o[c] += pw * (double)vv;
                }
            }
            for (int c = 0; c < HD; ++c)
                out[((size_t)b * hq + h) * HD + c] = o[c] / l;
            if (lse)
                lse[(size_t)b * hq + h] = mx + log(l);
        }
        free(logit);
    }
    return 0;
}

int orc_decode_attn(const uint8_t *k_codes, const uint16_t *k_meta, const uint16_t *k_ch0, const uint8_t *v_codes,
                    const uint16_t *v_meta, int hkv, const float *q_prime, const int32_t *sel_idx, int n_keep,
                    int batch, int hq, const int32_t *page_table, int max_pages, const int32_t *seq_lens,
                    double sm_scale, double *out, double *lse)
{
    return decode_impl(k_codes, k_meta, k_ch0, v_codes, v_meta, 0, 0, hkv, q_prime, sel_idx, n_keep, batch, hq,
                       page_table, max_pages, seq_lens, sm_scale, out, lse);
}

/* orc_decode_attn over a cache packed with per-token key grids: k^_{t,j} =
 * fmaf(code, s_t, z_t) with token t's own (scale, zero), j >= 1.           */
int orc_decode_attn_tokgrid(const uint8_t *k_codes, const uint16_t *k_meta, const uint16_t *k_ch0,
                            const uint8_t *v_codes, const uint16_t *v_meta, int hkv, const float *q_prime,
                            const int32_t *sel_idx, int n_keep, int batch, int hq, const int32_t *page_table,
                            int max_pages, const int32_t *seq_lens, double sm_scale, double *out, double *lse)
{
    return decode_impl(k_codes, k_meta, k_ch0, v_codes, v_meta, 1, 0, hkv, q_prime, sel_idx, n_keep, batch, hq,
                       page_table, max_pages, seq_lens, sm_scale, out, lse);
}

/* Decode with bucket-relative RoPE (§3.4): token t of sequence b scores with
 * its bucket's adjusted query and mask, q_prime[b][t / 2048][h] and
 * sel_idx[b][t / 2048][g], under one softmax over all tokens; the cache as
 * orc_decode_attn (keys stored in their bucket frames).                    */
int orc_decode_attn_rope(const uint8_t *k_codes, const uint16_t *k_meta, const uint16_t *k_ch0,
                         const uint8_t *v_codes, const uint16_t *v_meta, int hkv, const float *q_prime,
                         const int32_t *sel_idx, int n_keep, int n_buckets, int batch, int hq,
                         const int32_t *page_table, int max_pages, const int32_t *seq_lens, double sm_scale,
                         double *out, double *lse)
{
    if (n_buckets < 1)
        return -2;
    return decode_impl(k_codes, k_meta, k_ch0, v_codes, v_meta, 0, n_buckets, hkv, q_prime, sel_idx, n_keep, batch,
                       hq, page_table, max_pages, seq_lens, sm_scale, out, lse);
}

/* ------------------------------------------------------------------------ */
/* Unpruned BF16 reference decode (the comparison baseline of §4.4):
 * softmax(q k^T * sm_scale) v in fp64 on a paged bf16 cache
 * kb, vb bf16 [P][Hkv][128 tok][128 ch], in the original coordinates.      */
int orc_decode_bf16(const uint16_t *kb, const uint16_t *vb, int hkv, const uint16_t *q, int batch, int hq,
                    const int32_t *page_table, int max_pages, const int32_t *seq_lens, double sm_scale, double *out,
                    double *lse)
{
    if (hkv <= 0 || hq % hkv)
        return -2;
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        double *logit = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        if (!logit)
            return -7;
        for (int h = 0; h < hq; ++h) {
            int g = h / grp;
            const uint16_t *qr = q + ((size_t)b * hq + h) * HD;
            double mx = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                int64_t p = page_table[(size_t)b * max_pages + (t >> 7)];
                const uint16_t *kr = kb + (((size_t)p * hkv + g) * PG + (t & (PG - 1))) * HD;
                double acc = 0.0;
                for (int c = 0; c < HD; ++c)
                    acc += (double)orc_bf16_value(qr[c]) * (double)orc_bf16_value(kr[c]);
                logit[t] = acc * sm_scale;
                if (logit[t] > mx)
                    mx = logit[t];
            }
            double l = 0.0, o[HD];
            for (int c = 0; c < HD; ++c)
                o[c] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double pw = exp(logit[t] - mx);
                l += pw;
                int64_t p = page_table[(size_t)b * max_pages + (t >> 7)];
                const uint16_t *vr = vb + (((size_t)p * hkv + g) * PG + (t & (PG - 1))) * HD;
                for (int c = 0; c < HD; ++c)
                    o[c] += pw * (double)orc_bf16_value(vr[c]);
            }
            for (int c = 0; c < HD; ++c)
                out[((size_t)b * hq + h) * HD + c] = o[c] / l;
            if (lse)
                lse[(size_t)b * hq + h] = mx + log(l);
        }
        free(logit);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Protected BF16 tiers (§3.3: the first 64 and the most recent 256 tokens of
 * a sequence stay in BF16 for keys and values, under the same channel mask;
 * §3.4: one softmax over every token).  Reading: a sequence of length L keeps
 *   tokens [0, min(L, 64))            in the sink (slot t),
 *   tokens [64, 64 + 128 P)           in P INT2 pages, P = floor((L - 320)/128)
 *                                     for L >= 320, else 0 (a page is packed
 *                                     once all its tokens are older than the
 *                                     256 most recent),
 *   tokens [64 + 128 P, L)            in the tail (slot (t - 64) mod 384);
 * tier keys are k' = k T_K rounded to bf16, tier values the bf16 inputs.
 *   sink_k, sink_v  bf16 [batch][Hkv][64][128]
 *   tail_k, tail_v  bf16 [batch][Hkv][384][128]                              */
#define SINK 64
#define RECENT 256
#define TAIL_SLOTS 384

int64_t orc_tier_pages(int64_t L)
{
    return L >= SINK + RECENT ? (L - SINK - RECENT) / PG : 0;
}

int orc_decode_tiered(const uint8_t *k_codes, const uint16_t *k_meta, const uint16_t *k_ch0, const uint8_t *v_codes,
                      const uint16_t *v_meta, int hkv, const uint16_t *sink_k, const uint16_t *sink_v,
                      const uint16_t *tail_k, const uint16_t *tail_v, const float *q_prime, const int32_t *sel_idx,
                      int n_keep, int batch, int hq, const int32_t *page_table, int max_pages,
                      const int32_t *seq_lens, double sm_scale, double *out, double *lse)
{
    if (hkv <= 0 || hq % hkv || n_keep < 1 || n_keep > HD)
        return -2;
    int grp = hq / hkv;
    for (int b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        int64_t n_int2 = (int64_t)PG * orc_tier_pages(L);
        double *logit = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        if (!logit)
            return -7;
        for (int h = 0; h < hq; ++h) {
            int g = h / grp;
            const float *qp = q_prime + ((size_t)b * hq + h) * HD;
            const int32_t *M = sel_idx + ((size_t)b * hkv + g) * n_keep;
            double mx = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                double acc = 0.0;
                if (t < SINK || t >= SINK + n_int2) {
                    /* a BF16 tier token: k' rounded to bf16 */
                    const uint16_t *kr = t < SINK
                                             ? sink_k + (((size_t)b * hkv + g) * SINK + (size_t)t) * HD
                                             : tail_k + (((size_t)b * hkv + g) * TAIL_SLOTS +
                                                         (size_t)((t - SINK) % TAIL_SLOTS)) * HD;
                    for (int m = 0; m < n_keep; ++m)
                        acc += (double)qp[M[m]] * (double)orc_bf16_value(kr[M[m]]);
                } else {
                    int64_t i = t - SINK; /* INT2 token index */
                    int64_t p = page_table[(size_t)b * max_pages + (i >> 7)];
                    int s = (int)(i & (PG - 1));
                    size_t pg = (size_t)p * hkv + g;
                    for (int m = 0; m < n_keep; ++m) {
                        int j = M[m];
                        float kv;
                        if (j == 0) {
                            kv = orc_bf16_value(k_ch0[pg * PG + s]);
                        } else {
                            size_t r = krow(p, g, hkv, j);
                            int c = (k_codes[r * 32 + (s >> 2)] >> (2 * (s & 3))) & 3;
                            kv = orc_dequant(c, k_meta[r * 2], k_meta[r * 2 + 1]);
                        }
                        acc += (double)qp[j] * (double)kv;
                    }
                }
                logit[t] = acc * sm_scale;
                if (logit[t] > mx)
                    mx = logit[t];
            }
            double l = 0.0, o[HD];
            for (int c = 0; c < HD; ++c)
                o[c] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double pw = exp(logit[t] - mx);
                l += pw;
                if (t < SINK || t >= SINK + n_int2) {
                    const uint16_t *vr = t < SINK
                                             ? sink_v + (((size_t)b * hkv + g) * SINK + (size_t)t) * HD
                                             : tail_v + (((size_t)b * hkv + g) * TAIL_SLOTS +
                                                         (size_t)((t - SINK) % TAIL_SLOTS)) * HD;
                    for (int c = 0; c < HD; ++c)
                        o[c] += pw * (double)orc_bf16_value(vr[c]);
                } else {
                    int64_t i = t - SINK;
                    int64_t p = page_table[(size_t)b * max_pages + (i >> 7)];
                    int s = (int)(i & (PG - 1));
                    size_t pg = (size_t)p * hkv + g;
                    const uint8_t *vr = v_codes + (pg * PG + s) * 32;
                    const uint16_t *vm = v_meta + pg * 2 * 4 * PG;
                    for (int c = 0; c < HD; ++c) {
                        int q = c / VGROUP;
                        int code = (vr[c >> 2] >> (2 * (c & 3))) & 3;
                        o[c] += pw * (double)orc_dequant(code, vm[(0 * 4 + q) * PG + s], vm[(1 * 4 + q) * PG + s]);
                    }
                }
            }
            for (int c = 0; c < HD; ++c)
                out[((size_t)b * hq + h) * HD + c] = o[c] / l;
            if (lse)
                lse[(size_t)b * hq + h] = mx + log(l);
        }
        free(logit);
    }
    return 0;
}

/* bf16 bits of n fp32 values, round to nearest even (orc_bf16_round_nearest
 * element by element). */
void orc_bf16_round_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_round_nearest(x[i]);
}
