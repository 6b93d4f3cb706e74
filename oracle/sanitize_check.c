/*
 * sanitize_check.c -- TEST INFRASTRUCTURE ONLY: a driver that runs every entry
 * of dsa_oracle.c over small seeded inputs (all storage codes, ragged and
 * degenerate sizes: n = 0 and 1, n < k, n = k, all-equal scores, empty
 * selections) so that a build with -fsanitize=address,undefined checks the
 * oracle's own memory accesses and arithmetic.  It prints one line per case
 * and returns 0 when every output is finite where it must be.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_f64(uint16_t bits);
double orc_e4m3_to_f64(uint8_t code);
double orc_e2m1_to_f64(uint8_t code);
double orc_e8m0_to_f64(uint8_t e);
void orc_indexer_scores(const void *keys, const float *key_scales, int key_code, int dim,
                        const int32_t *page_row, int block_size,
                        const void *q, int q_code, const float *w, int n_heads,
                        int n, double *scores);
int orc_topk(const double *scores, int n, int k, int32_t *idx_out);
void orc_sparse_mla(const void *kv, const float *kv_scales, int kv_code,
                    int d_latent, int d_rope,
                    const int32_t *page_row, int block_size,
                    const void *q, int q_code, int n_heads,
                    const int32_t *sel, int n_sel, double scale,
                    double *out, double *lse);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 33);
}
static float next_f(void) { return (float)(next_u32() % 2001) / 1000.0f - 1.0f; }

/* a finite e4m3 code (never the NaN patterns 0x7F / 0xFF) */
static uint8_t e4m3_code(void)
{
    uint8_t c = (uint8_t)next_u32();
    return (c & 0x7F) == 0x7F ? (uint8_t)(c - 1) : c;
}

static int bad = 0;
static void expect_finite(const char *what, const double *v, int n)
{
    for (int i = 0; i < n; ++i)
        if (!isfinite(v[i])) {
            printf("non-finite %s[%d] = %g\n", what, i, v[i]);
            bad = 1;
            return;
        }
}

static void indexer_case(int code, int dim, int heads, int bs, int nblk, int n)
{
    size_t row_bytes = code == 0 ? 4u * (size_t)dim : code == 2 ? (size_t)dim : (size_t)(dim / 2 + dim / 32);
    size_t bytes = (size_t)nblk * (size_t)bs * row_bytes;
    uint8_t *keys = (uint8_t *)malloc(bytes ? bytes : 1);
    float *sig = (float *)malloc(sizeof(float) * (size_t)nblk * (size_t)bs);
    for (size_t i = 0; i < bytes; ++i)
        keys[i] = code == 2 ? e4m3_code() : (uint8_t)next_u32();
    if (code == 0)
        for (size_t i = 0; i < (size_t)nblk * bs * dim; ++i)
            ((float *)keys)[i] = next_f();
    if (code == 3) /* E8M0 bytes of every block: near 1.0, never NaN */
        for (int b = 0; b < nblk; ++b)
            for (int i = 0; i < bs * (dim / 32); ++i)
                keys[(size_t)b * bs * row_bytes + (size_t)bs * (dim / 2) + i] = (uint8_t)(124 + next_u32() % 7);
    for (int i = 0; i < nblk * bs; ++i)
        sig[i] = (float)(next_u32() % 100) / 50.0f;
    int32_t *pr = (int32_t *)malloc(sizeof(int32_t) * (size_t)nblk);
    for (int b = 0; b < nblk; ++b)
        pr[b] = nblk - 1 - b;
    int qcode = code == 0 ? 0 : 2;
    size_t qbytes = (size_t)heads * dim * (qcode == 0 ? 4 : 1);
    uint8_t *q = (uint8_t *)malloc(qbytes);
    for (size_t i = 0; i < qbytes; ++i)
        q[i] = e4m3_code();
    if (qcode == 0)
        for (int i = 0; i < heads * dim; ++i)
            ((float *)q)[i] = next_f();
    float *w = (float *)malloc(sizeof(float) * (size_t)heads);
    for (int h = 0; h < heads; ++h)
        w[h] = next_f();
    double *sc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    orc_indexer_scores(keys, sig, code, dim, pr, bs, q, qcode, w, heads, n, sc);
    expect_finite("scores", sc, n);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    for (int k = 1; k <= n + 1; k += (n > 8 ? n / 4 : 1)) {
        int m = orc_topk(sc, n, k, idx);
        if (m != (n < k ? n : k)) {
            printf("topk count %d for n %d k %d\n", m, n, k);
            bad = 1;
        }
    }
    printf("indexer code %d dim %d heads %d bs %d n %d ok\n", code, dim, heads, bs, n);
    free(idx);
    free(sc);
    free(w);
    free(q);
    free(pr);
    free(sig);
    free(keys);
}

static void mla_case(int code, int d, int r, int heads, int bs, int nblk, int n_sel)
{
    int W = d + r;
    size_t elems = (size_t)nblk * bs * W;
    size_t esz = code == 0 ? 4 : code == 1 ? 2 : 1;
    uint8_t *kv = (uint8_t *)malloc(elems * esz);
    for (size_t i = 0; i < elems * esz; ++i)
        kv[i] = code == 2 ? e4m3_code() : (uint8_t)(next_u32() & 0x3F);   /* small bf16 / fp32 bit patterns */
    if (code == 0)
        for (size_t i = 0; i < elems; ++i)
            ((float *)kv)[i] = next_f();
    float *scales = NULL;
    if (code == 2) {
        scales = (float *)malloc(sizeof(float) * (size_t)nblk * bs);
        for (int i = 0; i < nblk * bs; ++i)
            scales[i] = 0.01f * (float)(1 + next_u32() % 100);
    }
    int32_t *pr = (int32_t *)malloc(sizeof(int32_t) * (size_t)nblk);
    for (int b = 0; b < nblk; ++b)
        pr[b] = (b * 7) % nblk;
    int qcode = code == 0 ? 0 : 1;
    size_t qbytes = (size_t)heads * W * (qcode == 0 ? 4 : 2);
    uint8_t *q = (uint8_t *)malloc(qbytes);
    for (size_t i = 0; i < qbytes; ++i)
        q[i] = (uint8_t)(next_u32() & 0x3F);
    if (qcode == 0)
        for (int i = 0; i < heads * W; ++i)
            ((float *)q)[i] = next_f();
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_sel > 0 ? n_sel : 1));
    for (int j = 0; j < n_sel; ++j)
        sel[j] = (int32_t)((j * 13) % (nblk * bs));
    double *out = (double *)malloc(sizeof(double) * (size_t)heads * d);
    double *lse = (double *)malloc(sizeof(double) * (size_t)heads);
    orc_sparse_mla(kv, scales, code, d, r, pr, bs, q, qcode, heads, sel, n_sel, 1.0 / sqrt((double)W), out, lse);
    expect_finite("mla out", out, heads * d);
    if (n_sel > 0)
        expect_finite("mla lse", lse, heads);
    printf("mla code %d d %d r %d heads %d n_sel %d ok\n", code, d, r, heads, n_sel);
    free(lse);
    free(out);
    free(sel);
    free(q);
    free(pr);
    free(scales);
    free(kv);
}

int main(void)
{
    for (int c = 0; c < 256; ++c) {   /* every decoder over its whole code range */
        double v = orc_e4m3_to_f64((uint8_t)c) + orc_e8m0_to_f64((uint8_t)c) + orc_e2m1_to_f64((uint8_t)c);
        (void)v;
    }
    for (int c = 0; c < 65536; ++c)
        (void)orc_bf16_to_f64((uint16_t)c);
    int ns[] = {0, 1, 63, 64, 65, 200};
    for (unsigned i = 0; i < sizeof ns / sizeof ns[0]; ++i) {
        indexer_case(0, 32, 4, 64, 4, ns[i]);
        indexer_case(2, 128, 8, 64, 4, ns[i]);
        indexer_case(3, 64, 4, 32, 8, ns[i]);
    }
    {   /* all-equal scores: ties go to the lower index */
        double sc[10];
        int32_t idx[10];
        for (int i = 0; i < 10; ++i)
            sc[i] = 1.0;
        int m = orc_topk(sc, 10, 3, idx);
        if (m != 3 || idx[0] != 0 || idx[1] != 1 || idx[2] != 2) {
            printf("tie rule broken\n");
            bad = 1;
        }
    }
    int sels[] = {0, 1, 7, 100};
    for (unsigned i = 0; i < sizeof sels / sizeof sels[0]; ++i) {
        mla_case(0, 16, 8, 3, 16, 8, sels[i]);
        mla_case(1, 64, 16, 4, 64, 3, sels[i]);
        mla_case(2, 64, 16, 4, 64, 3, sels[i]);
    }
    printf(bad ? "FAILED\n" : "sanitized oracle run clean\n");
    return bad;
}
