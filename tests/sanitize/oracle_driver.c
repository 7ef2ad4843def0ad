/* Sanitizer driver for the oracle (plain C): calls every entry point on
 * small inputs, edge cases included (one token, empty selections, constant
 * groups, subnormal and extreme fp16 values), and checks a few invariants.
 * Built with -fsanitize=address,undefined; exit status 0 iff every check
 * held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_h2d(uint16_t h);
uint16_t oracle_f2h_rne(float x);
void oracle_quant_group(const uint16_t *x, int G, long stride, uint8_t *codes,
                        uint16_t *s, uint16_t *z);
void oracle_quant_group_bits(const uint16_t *x, int G, long stride, int bits,
                             uint8_t *codes, uint16_t *s, uint16_t *z);
float oracle_dequant(int code, uint16_t s, uint16_t z);
int oracle_budgets(int n, int L, int hn, int hd, int rn, int rd, int depth,
                   int pyramid, int32_t *k, int32_t *r);
void oracle_prefill_rows(int n, int D, int g, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const int32_t *rows, int n_rows,
                         double *o, double *lse, double *col);
int oracle_select(int n, const double *col, int n_hh, int n_recent, int32_t *sel);
int oracle_pack_unit(int D, int Gk, int Gv, const uint16_t *k, const uint16_t *v,
                     const int32_t *sel, int m, uint32_t *kq, uint16_t *ks,
                     uint16_t *kz, uint32_t *vq, uint16_t *vs, uint16_t *vz,
                     uint16_t *kres, uint16_t *vres);
int oracle_pack_unit_bits(int D, int Gk, int Gv, int kb, int vb, const uint16_t *k,
                          const uint16_t *v, const int32_t *sel, int m, uint32_t *kq,
                          uint16_t *ks, uint16_t *kz, uint32_t *vq, uint16_t *vs,
                          uint16_t *vz, uint16_t *kres, uint16_t *vres);
int oracle_dequant_unit(int D, int Gk, int Gv, int kb, int vb, int n_packed, int cap,
                        const uint32_t *kq, const uint16_t *ks, const uint16_t *kz,
                        const uint32_t *vq, const uint16_t *vs, const uint16_t *vz,
                        double *kh, double *vh);
int oracle_attend(int D, int g, const uint16_t *q, int T, const double *kh,
                  const double *vh, double *o);
int oracle_decode_unit(int D, int g, int Gk, int Gv, const uint16_t *q, int n_packed,
                       const uint32_t *kq, const uint16_t *ks, const uint16_t *kz,
                       const uint32_t *vq, const uint16_t *vs, const uint16_t *vz,
                       int n_res, const uint16_t *kres, const uint16_t *vres, double *o,
                       double *mass);
double oracle_cache_bytes(int L, int H, int D, int lp, int lg, double budget, int bits,
                          int group, double *full);
void oracle_diffkv_score(int n, int g, const double *col_h, double *score);
int oracle_diffkv_tiers(int n, const double *score, double thr_hi, double thr_lo, int Gk,
                        int32_t *hi, int32_t *lo, int32_t *counts);

static int fails = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            printf("check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                              \
        }                                                         \
    } while (0)

static uint32_t rng = 12345u;
static float frand(void) {
    rng = rng * 1664525u + 1013904223u;
    return ((rng >> 8) / 16777216.0f) * 4.0f - 2.0f;
}

int main(void) {
    enum { n = 96, D = 32, g = 2, G = 16 };
    for (uint32_t h = 0; h < 65536; ++h) {
        double x = oracle_h2d((uint16_t)h);
        if (!isnan(x)) CHECK(oracle_f2h_rne((float)x) == (uint16_t)h || x == 0.0);
    }
    uint16_t *q = malloc(sizeof(uint16_t) * g * n * D);
    uint16_t *k = malloc(sizeof(uint16_t) * n * D);
    uint16_t *v = malloc(sizeof(uint16_t) * n * D);
    for (int i = 0; i < g * n * D; ++i) q[i] = oracle_f2h_rne(frand());
    for (int i = 0; i < n * D; ++i) {
        k[i] = oracle_f2h_rne(frand() * (i % D == 3 ? 10.0f : 1.0f));
        v[i] = oracle_f2h_rne(frand());
    }
    k[5] = 0x0001;   /* a subnormal */
    v[7] = 0x7bff;   /* 65504 */
    /* codec, every width, constant group */
    uint8_t codes[G];
    uint16_t s, z, cst[G];
    for (int i = 0; i < G; ++i) cst[i] = 0x3c00;
    for (int bits = 2; bits <= 8; bits += 2) {
        if (bits == 6) continue;
        oracle_quant_group_bits(k, G, D, bits, codes, &s, &z);
        for (int i = 0; i < G; ++i) CHECK(codes[i] < (1 << bits));
        oracle_quant_group_bits(cst, G, 1, bits, codes, &s, &z);
        CHECK(s == 0);
    }
    oracle_quant_group(v, G, 1, codes, &s, &z);
    CHECK(isfinite(oracle_dequant(codes[0], s, z)));
    /* budgets */
    int32_t kb[32], r;
    CHECK(oracle_budgets(4096, 32, 1, 4, 1, 4, 7, 1, kb, &r) == 0 && r == 1024);
    CHECK(oracle_budgets(1, 1, 1, 4, 1, 4, 7, 1, kb, &r) == 0);
    CHECK(oracle_budgets(-1, 1, 1, 4, 1, 4, 7, 1, kb, &r) == -1);
    /* prefill: every row, then one row */
    int32_t rows[n];
    for (int i = 0; i < n; ++i) rows[i] = i;
    double *o = calloc((size_t)g * n * D, sizeof(double));
    double *lse = calloc((size_t)g * n, sizeof(double));
    double *col = calloc(n, sizeof(double));
    oracle_prefill_rows(n, D, g, q, k, v, rows, n, o, lse, col);
    double sum = 0;
    for (int j = 0; j < n; ++j) sum += col[j];
    CHECK(fabs(sum - g * n) < 1e-9 * g * n);
    oracle_prefill_rows(1, D, 1, q, k, v, rows, 1, o, lse, col);
    /* selection: empty, full, mixed */
    int32_t sel[n];
    CHECK(oracle_select(n, col, 0, 0, sel) == 0);
    CHECK(oracle_select(n, col, n, 0, sel) == 0);
    CHECK(oracle_select(n, col, 30, 20, sel) == 0);
    for (int i = 1; i < 50; ++i) CHECK(sel[i] > sel[i - 1]);
    CHECK(oracle_select(n, col, n, 1, sel) == -1);
    /* pack INT2 and every plane width; dequant and attention */
    uint32_t kq[4 * n * (D / 16)], vq[4 * (n / 16) * D];
    uint16_t ks[n * D], kz[n * D], vs[n * (D / G)], vz[n * (D / G)], kres[n * D], vres[n * D];
    double *kh = calloc((size_t)n * D, sizeof(double)), *vh = calloc((size_t)n * D, sizeof(double));
    double od[g * D], mass[n];
    int mp = oracle_pack_unit(D, G, G, k, v, sel, 50, kq, ks, kz, vq, vs, vz, kres, vres);
    CHECK(mp == 48);
    CHECK(oracle_decode_unit(D, g, G, G, q, mp, kq, ks, kz, vq, vs, vz, 2, kres, vres, od, mass) == 0);
    CHECK(oracle_decode_unit(D, g, G, G, q, 0, kq, ks, kz, vq, vs, vz, 0, kres, vres, od, mass) == -1);
    CHECK(oracle_pack_unit(D, G, G, k, v, sel, 0, kq, ks, kz, vq, vs, vz, kres, vres) == 0);
    const int widths[4][2] = {{2, 2}, {4, 4}, {4, 2}, {8, 4}};
    for (int w = 0; w < 4; ++w) {
        mp = oracle_pack_unit_bits(D, G, G, widths[w][0], widths[w][1], k, v, sel, 50, kq,
                                   ks, kz, vq, vs, vz, kres, vres);
        CHECK(mp == 48);
        CHECK(oracle_dequant_unit(D, G, G, widths[w][0], widths[w][1], mp, mp, kq, ks, kz, vq,
                                  vs, vz, kh, vh) == 0);
        CHECK(oracle_attend(D, g, q, mp, kh, vh, od) == 0);
        for (int i = 0; i < g * D; ++i) CHECK(isfinite(od[i]));
    }
    CHECK(oracle_pack_unit_bits(D, G, G, 6, 2, k, v, sel, 50, kq, ks, kz, vq, vs, vz, kres, vres) == -1);
    CHECK(oracle_attend(D, g, q, 0, kh, vh, od) == -1);
    /* cache size */
    double full = 0;
    CHECK(oracle_cache_bytes(32, 32, 128, 4096, 512, 0.5, 2, 16, &full) == 335544320.0);
    /* DiffKV */
    double *colh = calloc((size_t)g * n, sizeof(double)), score[n];
    for (int h = 0; h < g; ++h)
        oracle_prefill_rows(n, D, 1, q + (size_t)h * n * D, k, v, rows, n, NULL, NULL, colh + (size_t)h * n);
    oracle_diffkv_score(n, g, colh, score);
    int32_t hi[n], lo[n], cnt[2];
    CHECK(oracle_diffkv_tiers(n, score, 1.0 / n, 0.2 / n, G, hi, lo, cnt) == 0);
    CHECK(cnt[0] % G == 0 && cnt[1] % G == 0 && cnt[0] + cnt[1] <= n);
    CHECK(oracle_diffkv_tiers(0, score, 1.0, 0.0, G, hi, lo, cnt) == 0 && cnt[0] == 0);
    CHECK(oracle_diffkv_tiers(n, score, 1.0, 0.0, 0, hi, lo, cnt) == -1);
    free(q); free(k); free(v); free(o); free(lse); free(col); free(kh); free(vh); free(colh);
    printf("%s: %d failures\n", fails ? "FAIL" : "ok", fails);
    return fails ? 1 : 0;
}
