/*
 * sanitize_oracle.c -- test driver: runs every entry point of oracle/oracle.c
 * on small seeded inputs (ragged lengths, partial pages, page-edge lengths,
 * n_keep 1..128, groups 1 and 4, clipping, tiers) so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer sees every code path with
 * exactly sized buffers.  Checks return codes and that outputs are finite.
 * Test infrastructure only (built and run by tests/test_oracle_sanitized.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define HD 128
#define PG 128

double orc_f16_value(uint16_t h);
uint16_t orc_f16_round_down(float x);
uint16_t orc_f16_round_up(float x);
float orc_bf16_value(uint16_t b);
uint16_t orc_bf16_round_nearest(float x);
void orc_quantize_group(const float *x, int n, uint16_t *s, uint16_t *z, uint8_t *codes);
void orc_quantize_group_clip(const float *x, int n, float clip, uint16_t *s, uint16_t *z, uint8_t *codes);
float orc_dequant(int code, uint16_t s, uint16_t z);
void orc_key_transform(const uint16_t *k, const uint16_t *t_k, int64_t T, int hkv, float *kprime);
void orc_pack_cache(const float *kprime, const uint16_t *v, int hkv, int n_seqs, const int32_t *cu,
                    const int32_t *pt, int max_pages, uint8_t *kc, uint16_t *km, uint16_t *k0, uint8_t *vc,
                    uint16_t *vm);
void orc_pack_cache_vrot(const float *kprime, const float *vprime, float clip, int hkv, int n_seqs,
                         const int32_t *cu, const int32_t *pt, int max_pages, uint8_t *kc, uint16_t *km,
                         uint16_t *k0, uint8_t *vc, uint16_t *vm);
void orc_pack_cache_tokgrid(const float *kprime, const uint16_t *v, int hkv, int n_seqs, const int32_t *cu,
                            const int32_t *pt, int max_pages, uint8_t *kc, uint16_t *km, uint16_t *k0, uint8_t *vc,
                            uint16_t *vm);
int orc_decode_attn_tokgrid(const uint8_t *kc, const uint16_t *km, const uint16_t *k0, const uint8_t *vc,
                            const uint16_t *vm, int hkv, const float *qp, const int32_t *sel, int n_keep, int batch,
                            int hq, const int32_t *pt, int max_pages, const int32_t *lens, double sm, double *out,
                            double *lse);
int orc_value_unrotate(const double *o, const float *r_inv, int batch, int hq, int hkv, double *out);
int orc_select_channels(const uint16_t *q, const float *t_q, int batch, int hq, int hkv, int n_keep, float *qp,
                        int32_t *sel);
int orc_select_channels_base(const uint16_t *q, const float *t_q, const float *w, int batch, int hq, int hkv,
                             int n_keep, float *qp, int32_t *sel);
int orc_decode_attn(const uint8_t *kc, const uint16_t *km, const uint16_t *k0, const uint8_t *vc,
                    const uint16_t *vm, int hkv, const float *qp, const int32_t *sel, int n_keep, int batch,
                    int hq, const int32_t *pt, int max_pages, const int32_t *lens, double sm, double *out,
                    double *lse);
int orc_decode_bf16(const uint16_t *kb, const uint16_t *vb, int hkv, const uint16_t *q, int batch, int hq,
                    const int32_t *pt, int max_pages, const int32_t *lens, double sm, double *out, double *lse);
int64_t orc_tier_pages(int64_t L);
int orc_decode_tiered(const uint8_t *kc, const uint16_t *km, const uint16_t *k0, const uint8_t *vc,
                      const uint16_t *vm, int hkv, const uint16_t *sink_k, const uint16_t *sink_v,
                      const uint16_t *tail_k, const uint16_t *tail_v, const float *qp, const int32_t *sel,
                      int n_keep, int batch, int hq, const int32_t *pt, int max_pages, const int32_t *lens,
                      double sm, double *out, double *lse);
void orc_bf16_round_array(const float *x, int64_t n, uint16_t *out);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static double uni(void)
{
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (double)(rs >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss(void) { return (float)(uni() + uni() + uni() + uni() - 2.0) * 1.7320508f; }

static void *xcalloc(size_t n, size_t sz)
{
    void *p = calloc(n ? n : 1, sz);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}
static uint16_t *rand_bf16(size_t n, float scale)
{
    float *f = xcalloc(n, sizeof(float));
    uint16_t *b = xcalloc(n, sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i)
        f[i] = gauss() * scale;
    orc_bf16_round_array(f, (int64_t)n, b);
    free(f);
    return b;
}
static float *rand_f32(size_t n, float lo, float hi)
{
    float *f = xcalloc(n, sizeof(float));
    for (size_t i = 0; i < n; ++i)
        f[i] = (float)(lo + (hi - lo) * uni());
    return f;
}
static int finite_all(const double *x, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return 0;
    return 1;
}

static int failures = 0;
#define CHECK(cond, ...)                                                                                        \
    do {                                                                                                        \
        if (!(cond)) {                                                                                          \
            fprintf(stderr, __VA_ARGS__);                                                                       \
            fputc('\n', stderr);                                                                                \
            ++failures;                                                                                         \
        }                                                                                                       \
    } while (0)

typedef struct {
    uint8_t *kc, *vc;
    uint16_t *km, *k0, *vm;
} cache_t;

static cache_t cache_new(int P, int hkv)
{
    cache_t c;
    c.kc = xcalloc((size_t)P * hkv * HD * 32, 1);
    c.km = xcalloc((size_t)P * hkv * HD * 2, sizeof(uint16_t));
    c.k0 = xcalloc((size_t)P * hkv * PG, sizeof(uint16_t));
    c.vc = xcalloc((size_t)P * hkv * PG * 32, 1);
    c.vm = xcalloc((size_t)P * hkv * 2 * 4 * PG, sizeof(uint16_t));
    return c;
}
static void cache_free(cache_t *c)
{
    free(c->kc);
    free(c->km);
    free(c->k0);
    free(c->vc);
    free(c->vm);
}

static void run_case(int hkv, int grp, int n_seqs, const int32_t *lens, int n_keep)
{
    const int hq = hkv * grp;
    int32_t *cu = xcalloc((size_t)n_seqs + 1, sizeof(int32_t));
    int max_pages = 1, total_pages = 0;
    for (int b = 0; b < n_seqs; ++b) {
        cu[b + 1] = cu[b] + lens[b];
        int np = (lens[b] + PG - 1) / PG;
        if (np > max_pages)
            max_pages = np;
        total_pages += np;
    }
    const int P = (total_pages + 7) / 8 * 8;
    int32_t *pt = xcalloc((size_t)n_seqs * max_pages, sizeof(int32_t));
    for (int b = 0, next = 0; b < n_seqs; ++b)
        for (int i = 0; i < max_pages; ++i)
            pt[(size_t)b * max_pages + i] = i < (lens[b] + PG - 1) / PG ? next++ : 0;
    const int64_t T = cu[n_seqs];
    uint16_t *k = rand_bf16((size_t)T * hkv * HD, 1.0f);
    uint16_t *v = rand_bf16((size_t)T * hkv * HD, 1.0f);
    uint16_t *tk = rand_bf16((size_t)hkv * HD * HD, 0.09f);
    uint16_t *rv = rand_bf16((size_t)hkv * HD * HD, 0.09f);
    float *tq = rand_f32((size_t)hkv * HD * HD, -0.2f, 0.2f);
    float *rinv = rand_f32((size_t)hkv * HD * HD, -0.2f, 0.2f);
    float *wsel = rand_f32((size_t)hkv * HD, 0.5f, 2.0f);
    uint16_t *q = rand_bf16((size_t)n_seqs * hq * HD, 1.0f);
    float *kp = xcalloc((size_t)T * hkv * HD, sizeof(float));
    float *vp = xcalloc((size_t)T * hkv * HD, sizeof(float));
    orc_key_transform(k, tk, T, hkv, kp);
    orc_key_transform(v, rv, T, hkv, vp);

    float *qp = xcalloc((size_t)n_seqs * hq * HD, sizeof(float));
    int32_t *sel = xcalloc((size_t)n_seqs * hkv * n_keep, sizeof(int32_t));
    double *out = xcalloc((size_t)n_seqs * hq * HD, sizeof(double));
    double *out2 = xcalloc((size_t)n_seqs * hq * HD, sizeof(double));
    double *lse = xcalloc((size_t)n_seqs * hq, sizeof(double));
    const double sm = 1.0 / sqrt((double)HD);

    CHECK(orc_select_channels_base(q, tq, wsel, n_seqs, hq, hkv, n_keep, qp, sel) == 0, "select_base rc");
    CHECK(orc_select_channels(q, tq, n_seqs, hq, hkv, n_keep, qp, sel) == 0, "select rc");
    for (size_t i = 0; i < (size_t)n_seqs * hkv * n_keep; ++i)
        CHECK(sel[i] >= 0 && sel[i] < HD, "selected channel out of range");

    cache_t c = cache_new(P, hkv);
    orc_pack_cache(kp, v, hkv, n_seqs, cu, pt, max_pages, c.kc, c.km, c.k0, c.vc, c.vm);
    CHECK(orc_decode_attn(c.kc, c.km, c.k0, c.vc, c.vm, hkv, qp, sel, n_keep, n_seqs, hq, pt, max_pages, lens, sm,
                          out, lse) == 0,
          "decode rc");
    CHECK(finite_all(out, (size_t)n_seqs * hq * HD) && finite_all(lse, (size_t)n_seqs * hq), "decode finite");
    orc_pack_cache_tokgrid(kp, v, hkv, n_seqs, cu, pt, max_pages, c.kc, c.km, c.k0, c.vc, c.vm);
    CHECK(orc_decode_attn_tokgrid(c.kc, c.km, c.k0, c.vc, c.vm, hkv, qp, sel, n_keep, n_seqs, hq, pt, max_pages,
                                  lens, sm, out, lse) == 0,
          "decode (per-token key grids) rc");
    CHECK(finite_all(out, (size_t)n_seqs * hq * HD), "decode (per-token key grids) finite");
    orc_pack_cache_vrot(kp, vp, 0.92f, hkv, n_seqs, cu, pt, max_pages, c.kc, c.km, c.k0, c.vc, c.vm);
    CHECK(orc_decode_attn(c.kc, c.km, c.k0, c.vc, c.vm, hkv, qp, sel, n_keep, n_seqs, hq, pt, max_pages, lens, sm,
                          out, NULL) == 0,
          "decode (rotated values) rc");
    CHECK(orc_value_unrotate(out, rinv, n_seqs, hq, hkv, out2) == 0, "unrotate rc");
    CHECK(finite_all(out2, (size_t)n_seqs * hq * HD), "unrotate finite");

    /* BF16 pages in the original coordinates */
    uint16_t *kb = rand_bf16((size_t)P * hkv * PG * HD, 1.0f);
    uint16_t *vb = rand_bf16((size_t)P * hkv * PG * HD, 1.0f);
    CHECK(orc_decode_bf16(kb, vb, hkv, q, n_seqs, hq, pt, max_pages, lens, sm, out, lse) == 0, "bf16 rc");
    CHECK(finite_all(out, (size_t)n_seqs * hq * HD), "bf16 finite");

    /* tiers: the INT2 pages of each sequence are its first tier_pages(L) table entries */
    uint16_t *sk = rand_bf16((size_t)n_seqs * hkv * 64 * HD, 1.0f);
    uint16_t *sv = rand_bf16((size_t)n_seqs * hkv * 64 * HD, 1.0f);
    uint16_t *tkk = rand_bf16((size_t)n_seqs * hkv * 384 * HD, 1.0f);
    uint16_t *tvv = rand_bf16((size_t)n_seqs * hkv * 384 * HD, 1.0f);
    for (int b = 0; b < n_seqs; ++b)
        CHECK(orc_tier_pages(lens[b]) <= max_pages, "tier pages beyond the table");
    CHECK(orc_decode_tiered(c.kc, c.km, c.k0, c.vc, c.vm, hkv, sk, sv, tkk, tvv, qp, sel, n_keep, n_seqs, hq, pt,
                            max_pages, lens, sm, out, lse) == 0,
          "tiered rc");
    CHECK(finite_all(out, (size_t)n_seqs * hq * HD), "tiered finite");
    CHECK(orc_select_channels(q, tq, n_seqs, hq, 0, n_keep, qp, sel) == -2, "select shape check");
    CHECK(orc_select_channels(q, tq, n_seqs, hq, hkv, HD + 1, qp, sel) == -2, "select n_keep check");
    CHECK(orc_value_unrotate(out, rinv, n_seqs, hq, 0, out2) == -2, "unrotate shape check");

    cache_free(&c);
    free(kb), free(vb), free(sk), free(sv), free(tkk), free(tvv);
    free(cu), free(pt), free(k), free(v), free(tk), free(rv), free(tq), free(rinv), free(wsel), free(q);
    free(kp), free(vp), free(qp), free(sel), free(out), free(out2), free(lse);
}

int main(void)
{
    /* quantizer and number formats over every group size of the path */
    for (int n = 1; n <= 128; n = n < 8 ? n + 1 : n * 2) {
        float x[128];
        uint8_t codes[128];
        uint16_t s, z;
        for (int i = 0; i < n; ++i)
            x[i] = gauss() * (float)pow(10.0, (double)(int)(uni() * 8) - 4);
        orc_quantize_group(x, n, &s, &z, codes);
        orc_quantize_group_clip(x, n, 0.92f, &s, &z, codes);
        for (int i = 0; i < n; ++i)
            CHECK(codes[i] <= 3 && isfinite(orc_dequant(codes[i], s, z)), "quantizer");
    }
    for (int i = 0; i < 4096; ++i) {
        float f = gauss() * (float)pow(2.0, (double)(int)(uni() * 60) - 30);
        CHECK(isfinite(orc_f16_value(orc_f16_round_down(f))) || fabsf(f) > 65000.0f, "f16");
        (void)orc_f16_round_up(f);
        (void)orc_bf16_value(orc_bf16_round_nearest(f));
    }
    const int32_t l1[] = {1};
    const int32_t l2[] = {129, 5, 128};
    const int32_t l3[] = {320, 449, 127};
    const int32_t l4[] = {700, 256};
    run_case(1, 4, 1, l1, 1);
    run_case(2, 4, 3, l2, 77);
    run_case(2, 1, 3, l3, 128);
    run_case(1, 4, 2, l4, 52);
    run_case(2, 2, 2, l4, 2);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized oracle driver: all entry points ran clean\n");
    return 0;
}
