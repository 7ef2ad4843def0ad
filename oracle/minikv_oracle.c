/*
 * minikv_oracle.c -- plain, slow, obviously-correct CPU reference for
 * MiniKV-style compressed-KV attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; it is built by gcc with -O2 -ffp-contract=off and no
 * fast-math, so every fp32 operation below is a single IEEE round-to-nearest-
 * even operation in the order written.
 *
 * Sources (web pages on MiniKV, arXiv 2411.18077):
 *   [R]  "Pith review of MiniKV: Pushing the Limits of LLM Inference via 2-Bit
 *        Layer-Discriminative KV Cache" (pith.science), sections "What carries
 *        the argument", "Assumptions & free parameters", the authors'
 *        abstract and the figure captions (Fig. 1, Fig. 4).
 *   [V]  the pith.science verdict record for arXiv 2411.18077, fields
 *        pith_extraction.key_machinery, referee_report.major_comments,
 *        supporting_citations.
 *   [M]  "Don't Discard, but Keep It Small: Context-Preserving KV Cache
 *        Compression with Importance-Aware Adaptive Precision" (paperhub.cn),
 *        the rebuttal paragraph on permutation invariance of attention.
 *
 * Where the pages leave a step open the plainest reading is taken; each such
 * reading is named in a comment ("reading: ...").
 *
 * Every function here is either the plain definition of what the method
 * computes (attention, column sums of the attention matrix, top-k) written
 * out in fp64, or -- for the INT2 codec, which is an encoding -- its steps in
 * order.  No blocking, fusion or reordering.
 *
 * Parity pins (tests that tie this file to something other than itself) live
 * in tests/test_oracle_*.py.  Functions without such a pin say so below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32/64, written from the format definition.   */
/* ------------------------------------------------------------------------ */

/* Value of a binary16 bit pattern: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 is the subnormal range m * 2^-24. */
double oracle_h2d(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Encode a value that is already exactly representable in binary16. */
static uint16_t encode_exact_half(double a, int sign)
{
    uint16_t s = sign ? 0x8000 : 0;
    if (a == 0.0)
        return s;
    if (a < ldexp(1.0, -14))                      /* subnormal */
        return s | (uint16_t)(a / ldexp(1.0, -24));
    int e2;
    double f = frexp(a, &e2);                     /* a = f * 2^e2, f in [0.5,1) */
    int E = e2 - 1 + 15;                          /* biased exponent */
    if (E >= 31)
        return s | 0x7c00;
    int m = (int)((f * 2.0 - 1.0) * 1024.0);      /* exact: 10 fraction bits */
    return s | (uint16_t)(E << 10) | (uint16_t)m;
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t oracle_f2h_rne(float xf)
{
    double x = (double)xf;                        /* exact */
    if (isnan(x))
        return 0x7e00;
    int sign = signbit(x) ? 1 : 0;
    double a = fabs(x);
    /* 65504 is the largest finite half; the next quantum boundary 65520 is
     * the round-to-even tie towards infinity. */
    if (a >= 65520.0)
        return (uint16_t)((sign ? 0x8000 : 0) | 0x7c00);
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);
    } else {
        int e2;
        frexp(a, &e2);                            /* 2^(e2-1) <= a < 2^e2 */
        quantum = ldexp(1.0, e2 - 1 - 10);
    }
    double t = a / quantum;                       /* exact: power-of-two scale */
    double r = nearbyint(t);                      /* default mode: ties-to-even */
    return encode_exact_half(r * quantum, sign);
}

/* ------------------------------------------------------------------------ */
/* INT2 asymmetric codec on one quantization group.                         */
/*                                                                          */
/* [R] "What carries the argument" / [V] key_machinery: KIVI-style packing; */
/* sixteen 2-bit codes share one 32-bit word, and each group keeps an fp16  */
/* scale and an fp16 zero-point.  [V] supporting_citations: KIVI's codec is */
/* asymmetric 2-bit.                                                        */
/* reading: scale = (max - min) / 3 computed in fp32 (one subtraction, one  */
/*   correctly rounded division) and rounded to fp16; zero = min (exactly   */
/*   an fp16 value, with -0 canonicalised to +0 by adding +0.0f);           */
/*   code = round-half-even of d / scale, d = fp32(x - zero), decided by    */
/*   exact comparison against (c + 1/2) * scale, clamped to [0, 3];         */
/*   scale == 0 gives code 0 everywhere.                                    */
/* ------------------------------------------------------------------------ */

void oracle_quant_group(const uint16_t *x, int G, long stride,
                        uint8_t *codes, uint16_t *scale_out, uint16_t *zero_out)
{
    float mn = (float)oracle_h2d(x[0]);
    float mx = mn;
    for (int i = 1; i < G; ++i) {
        float xi = (float)oracle_h2d(x[(long)i * stride]);
        if (xi < mn) mn = xi;
        if (xi > mx) mx = xi;
    }
    float range = mx - mn;                        /* one fp32 rounding */
    float s32 = range / 3.0f;                     /* one fp32 rounding */
    uint16_t sh = oracle_f2h_rne(s32);
    float z32 = mn + 0.0f;                        /* -0 -> +0 */
    uint16_t zh = oracle_f2h_rne(z32);            /* exact: mn is a half */
    float sf = (float)oracle_h2d(sh);
    float zf = (float)oracle_h2d(zh);
    *scale_out = sh;
    *zero_out = zh;
    /* Thresholds (c + 1/2) * scale are exact in fp32: scale has at most 11
     * significant bits and c + 1/2 at most 3. */
    float t0 = 0.5f * sf, t1 = 1.5f * sf, t2 = 2.5f * sf;
    for (int i = 0; i < G; ++i) {
        if (sf == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float xi = (float)oracle_h2d(x[(long)i * stride]);
        float d = xi - zf;                        /* one fp32 rounding */
        /* round half to even of d/scale over the four codes:
         *   d == 0.5 s -> 0, d == 1.5 s -> 2, d == 2.5 s -> 2 */
        int c = 0;
        if (d > t0) c = 1;
        if (d >= t1) c = 2;
        if (d > t2) c = 3;
        codes[i] = (uint8_t)c;
    }
}

/* Dequantised value code * scale + zero in fp32.  The product is exact
 * (2-bit code times an 11-bit scale), so there is a single rounding. */
float oracle_dequant(int code, uint16_t scale, uint16_t zero)
{
    float p = (float)code * (float)oracle_h2d(scale);
    return p + (float)oracle_h2d(zero);
}

/* ------------------------------------------------------------------------ */
/* Per-layer budgets.                                                       */
/*                                                                          */
/* [R] "Assumptions & free parameters": half of the prompt is kept, a      */
/* quarter as heavy hitters and a quarter as the most recent tokens, in     */
/* every layer; a depth parameter (d = 7) sets how the heavy-hitter budget  */
/* is spread linearly over the layers, the lower layers getting more        */
/* ("Core claim").                                                          */
/* reading: r = floor(n * rw_num / rw_den), k = floor(n * hh_num / hh_den); */
/*   pyramid: k_min = floor(k / d), k_max = 2k - k_min, and layer l gets    */
/*   k_min + floor((k_max - k_min) * (L-1-l) / (L-1)) (L = 1: k), clamped   */
/*   to n - r.  PARITY UNPINNED beyond its own invariants: the pages give   */
/*   no formula and no per-layer value.                                     */
/* ------------------------------------------------------------------------ */

int oracle_budgets(int n, int n_layers, int hh_num, int hh_den, int rw_num,
                   int rw_den, int depth, int pyramid, int32_t *k_out,
                   int32_t *r_out)
{
    if (n < 0 || n_layers < 1 || hh_den <= 0 || rw_den <= 0 || hh_num < 0 ||
        rw_num < 0 || (pyramid && depth < 1))
        return -1;
    long long r = (long long)n * rw_num / rw_den;
    long long k = (long long)n * hh_num / hh_den;
    if (r > n) return -1;
    *r_out = (int32_t)r;
    for (int l = 0; l < n_layers; ++l) {
        long long kl;
        if (!pyramid || n_layers == 1) {
            kl = k;
        } else {
            long long kmin = k / depth;
            long long kmax = 2 * k - kmin;
            kl = kmin + (kmax - kmin) * (n_layers - 1 - l) / (n_layers - 1);
        }
        if (kl > n - r) kl = n - r;
        k_out[l] = (int32_t)kl;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Prefill attention of one (batch, kv-head) unit, selected query rows.     */
/*                                                                          */
/* [V] key_machinery / [R] "What carries the argument": the prefill kernel  */
/* makes two passes and returns both the attention output and, per key, the */
/* attention it received summed over query rows, in memory linear in n;     */
/* [R] "Assumptions": those accumulated scores pick the heavy hitters (the  */
/* H2O policy).                                                             */
/* reading: causal mask including the diagonal; scale 1/sqrt(D); natural   */
/*   exponent; the cumulative score of key j sums the softmax probability  */
/*   P[h][i][j] over every causal query row i >= j and over the g query     */
/*   heads that share the kv head (GQA sum).                                */
/*                                                                          */
/* This is the plain row-by-row definition: for each row, all logits, the   */
/* row max, the normaliser, the output and the row's contribution to the    */
/* column sums.  Everything in fp64 from the fp16 inputs.                   */
/*                                                                          */
/*   q [g][n][D], k [n][D], v [n][D]   fp16 bit patterns                    */
/*   rows[n_rows]                      query rows to evaluate               */
/*   o   [g][n_rows][D]  (nullable)    output rows                          */
/*   lse [g][n_rows]     (nullable)    M + ln(sum exp(s - M))               */
/*   col [n]             (nullable)    += contributions of these rows       */
/* ------------------------------------------------------------------------ */

void oracle_prefill_rows(int n, int D, int g, const uint16_t *q,
                         const uint16_t *k, const uint16_t *v,
                         const int32_t *rows, int n_rows, double *o,
                         double *lse, double *col)
{
    double *kd = (double *)malloc(sizeof(double) * (size_t)n * D);
    double *vd = (double *)malloc(sizeof(double) * (size_t)n * D);
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *qi = (double *)malloc(sizeof(double) * (size_t)D);
    for (long t = 0; t < (long)n * D; ++t) {
        kd[t] = oracle_h2d(k[t]);
        vd[t] = oracle_h2d(v[t]);
    }
    const double scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < g; ++h) {
        for (int ri = 0; ri < n_rows; ++ri) {
            int i = rows[ri];
            for (int c = 0; c < D; ++c)
                qi[c] = oracle_h2d(q[((long)h * n + i) * D + c]);
            double M = -INFINITY;
            for (int j = 0; j <= i; ++j) {
                double acc = 0.0;
                for (int c = 0; c < D; ++c)
                    acc += qi[c] * kd[(long)j * D + c];
                s[j] = acc * scale;
                if (s[j] > M) M = s[j];
            }
            double l = 0.0;
            for (int j = 0; j <= i; ++j) {
                s[j] = exp(s[j] - M);
                l += s[j];
            }
            if (o) {
                double *orow = o + ((long)h * n_rows + ri) * D;
                for (int c = 0; c < D; ++c) orow[c] = 0.0;
                for (int j = 0; j <= i; ++j) {
                    double p = s[j] / l;
                    for (int c = 0; c < D; ++c)
                        orow[c] += p * vd[(long)j * D + c];
                }
            }
            if (lse)
                lse[(long)h * n_rows + ri] = M + log(l);
            if (col)
                for (int j = 0; j <= i; ++j)
                    col[j] += s[j] / l;
        }
    }
    free(kd);
    free(vd);
    free(s);
    free(qi);
}

/* ------------------------------------------------------------------------ */
/* Persistent heavy-hitter + recent-window selection of one unit.           */
/*                                                                          */
/* [R] "What carries the argument": heavy hitters are chosen once from the  */
/* cumulative attention scores at the end of prefill and never re-selected; */
/* [R] "Assumptions": a recent window is retained alongside them.           */
/* reading: the recent window is the last n_recent tokens; heavy hitters    */
/*   are the top n_hh of the remaining candidates [0, n - n_recent) ordered */
/*   by (score descending, index ascending) -- ties go to the lower index;  */
/*   the selection is stored in ascending original-index order (attention   */
/*   is invariant to a common permutation of keys and values, [M]).         */
/* ------------------------------------------------------------------------ */

typedef struct {
    double score;
    int32_t idx;
} scored_t;

static int cmp_scored(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int oracle_select(int n, const double *col, int n_hh, int n_recent,
                  int32_t *sel)
{
    if (n < 0 || n_recent < 0 || n_recent > n || n_hh < 0 ||
        n_hh > n - n_recent)
        return -1;
    int nc = n - n_recent;
    scored_t *cand = (scored_t *)malloc(sizeof(scored_t) * (size_t)(nc > 0 ? nc : 1));
    for (int j = 0; j < nc; ++j) {
        cand[j].score = col[j];
        cand[j].idx = j;
    }
    qsort(cand, (size_t)nc, sizeof(scored_t), cmp_scored);
    for (int t = 0; t < n_hh; ++t)
        sel[t] = cand[t].idx;
    qsort(sel, (size_t)n_hh, sizeof(int32_t), cmp_i32);
    for (int t = 0; t < n_recent; ++t)
        sel[n_hh + t] = nc + t;
    free(cand);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Pack one unit's selected tokens.                                         */
/*                                                                          */
/* [R] "Assumptions": groups of 16 scalars for both the per-channel key     */
/* (sub-channel) and the per-token value quantisation; Fig. 1 caption: keys */
/* per channel, values per token; [V] key_machinery: sixteen 2-bit codes    */
/* per 32-bit word, fp16 scale and zero.                                    */
/* reading (layout): the pages fix sixteen codes per 32-bit word but not   */
/*   which sixteen.  Keys are quantised per channel over groups of Gk       */
/*   consecutive selected tokens; a key word holds 16 consecutive channels  */
/*   of one token.  Values are quantised per token over groups of Gv        */
/*   consecutive channels; a value word holds 16 consecutive selected       */
/*   tokens of one channel.  Each word thus runs along the dimension that   */
/*   attention sums over (channels for q.k, tokens for p.v).  Element e of  */
/*   a word sits at bits 2e..2e+1.                                          */
/* reading (ragged tail): the first floor(m / Gk) * Gk selected tokens are  */
/*   packed; the last m mod Gk stay in fp16 as the start of the residual.   */
/*                                                                          */
/*   k, v          [n][D] fp16 of this unit; sel[m] ascending indices       */
/*   kq  [mp][D/16] uint32;  ks, kz [mp/Gk][D] fp16                         */
/*   vq  [mp/16][D] uint32;  vs, vz [mp][D/Gv] fp16                         */
/*   kres, vres [m - mp][D] fp16                                            */
/* Returns mp (number of packed tokens) or -1 on bad arguments.             */
/* ------------------------------------------------------------------------ */

int oracle_pack_unit(int D, int Gk, int Gv, const uint16_t *k,
                     const uint16_t *v, const int32_t *sel, int m,
                     uint32_t *kq, uint16_t *ks, uint16_t *kz, uint32_t *vq,
                     uint16_t *vs, uint16_t *vz, uint16_t *kres,
                     uint16_t *vres)
{
    if (D % 16 || Gk % 16 || Gv % 16 || D % Gv || m < 0 || Gk <= 0 || Gv <= 0)
        return -1;
    int mp = (m / Gk) * Gk;
    uint16_t *x = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(Gk > Gv ? Gk : Gv));
    uint8_t *codes = (uint8_t *)malloc((size_t)(Gk > Gv ? Gk : Gv));

    memset(kq, 0, sizeof(uint32_t) * (size_t)mp * (D / 16));
    for (int gi = 0; gi < mp / Gk; ++gi) {
        for (int c = 0; c < D; ++c) {
            for (int t = 0; t < Gk; ++t)
                x[t] = k[(long)sel[gi * Gk + t] * D + c];
            oracle_quant_group(x, Gk, 1, codes, &ks[(long)gi * D + c],
                               &kz[(long)gi * D + c]);
            for (int t = 0; t < Gk; ++t) {
                int p = gi * Gk + t;
                kq[(long)p * (D / 16) + c / 16] |= (uint32_t)codes[t] << (2 * (c % 16));
            }
        }
    }

    memset(vq, 0, sizeof(uint32_t) * (size_t)(mp / 16) * D);
    for (int p = 0; p < mp; ++p) {
        const uint16_t *row = v + (long)sel[p] * D;
        for (int G = 0; G < D / Gv; ++G) {
            oracle_quant_group(row + G * Gv, Gv, 1, codes,
                               &vs[(long)p * (D / Gv) + G],
                               &vz[(long)p * (D / Gv) + G]);
            for (int i = 0; i < Gv; ++i) {
                int c = G * Gv + i;
                vq[(long)(p / 16) * D + c] |= (uint32_t)codes[i] << (2 * (p % 16));
            }
        }
    }

    for (int p = mp; p < m; ++p) {
        memcpy(kres + (long)(p - mp) * D, k + (long)sel[p] * D, sizeof(uint16_t) * D);
        memcpy(vres + (long)(p - mp) * D, v + (long)sel[p] * D, sizeof(uint16_t) * D);
    }
    free(x);
    free(codes);
    return mp;
}

/* ------------------------------------------------------------------------ */
/* Decode attention of one unit over its packed cache and fp16 residual.    */
/*                                                                          */
/* [V] forward_implications: the fixed layout enables 2-bit quantisation    */
/* and fused dequantisation during decoding.  [V] supporting_citations:     */
/* KIVI's streaming (residual) buffer keeps recent tokens in full precision.*/
/* reading: attention of each of the g query heads over every packed token  */
/*   (dequantised to fp32, code * scale + zero) and every residual token,   */
/*   softmax with scale 1/sqrt(D), no mask (all cached tokens precede the   */
/*   query).  fp64 accumulation.                                            */
/*                                                                          */
/*   q [g][D] fp16; cache arrays as oracle_pack_unit writes them with       */
/*   n_packed tokens (multiple of Gk); kres, vres [n_res][D] fp16;          */
/*   o [g][D] fp64.                                                         */
/*                                                                          */
/* mass (nullable) [n_packed + n_res] fp64: the attention weight of every   */
/*   cached token, summed over the g query heads, in cache order (packed    */
/*   tokens, then residual slots).  [V] referee_report.major_comments[0]    */
/*   and the verdict's falsifier field: whether the heavy hitters chosen at */
/*   the end of prefill stay the tokens decoding attends to is measured by  */
/*   this per-step attention mass.                                          */
/* ------------------------------------------------------------------------ */

int oracle_decode_unit(int D, int g, int Gk, int Gv, const uint16_t *q,
                       int n_packed, const uint32_t *kq, const uint16_t *ks,
                       const uint16_t *kz, const uint32_t *vq,
                       const uint16_t *vs, const uint16_t *vz, int n_res,
                       const uint16_t *kres, const uint16_t *vres, double *o,
                       double *mass)
{
    int T = n_packed + n_res;
    if (T <= 0 || n_packed % Gk || D % 16 || D % Gv)
        return -1;
    double *kh = (double *)malloc(sizeof(double) * (size_t)T * D);
    double *vh = (double *)malloc(sizeof(double) * (size_t)T * D);
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    for (int t = 0; t < n_packed; ++t) {
        for (int c = 0; c < D; ++c) {
            int kc = (int)((kq[(long)t * (D / 16) + c / 16] >> (2 * (c % 16))) & 3u);
            long km = (long)(t / Gk) * D + c;
            kh[(long)t * D + c] = (double)oracle_dequant(kc, ks[km], kz[km]);
            int vc = (int)((vq[(long)(t / 16) * D + c] >> (2 * (t % 16))) & 3u);
            long vm = (long)t * (D / Gv) + c / Gv;
            vh[(long)t * D + c] = (double)oracle_dequant(vc, vs[vm], vz[vm]);
        }
    }
    for (int t = 0; t < n_res; ++t) {
        for (int c = 0; c < D; ++c) {
            kh[(long)(n_packed + t) * D + c] = oracle_h2d(kres[(long)t * D + c]);
            vh[(long)(n_packed + t) * D + c] = oracle_h2d(vres[(long)t * D + c]);
        }
    }
    const double scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < g; ++h) {
        double M = -INFINITY;
        for (int t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += oracle_h2d(q[(long)h * D + c]) * kh[(long)t * D + c];
            s[t] = acc * scale;
            if (s[t] > M) M = s[t];
        }
        double l = 0.0;
        for (int t = 0; t < T; ++t) {
            s[t] = exp(s[t] - M);
            l += s[t];
        }
        if (mass) {
            for (int t = 0; t < T; ++t) {
                if (h == 0) mass[t] = 0.0;
                mass[t] += s[t] / l;
            }
        }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t)
                acc += s[t] * vh[(long)t * D + c];
            o[(long)h * D + c] = acc / l;
        }
    }
    free(kh);
    free(vh);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Closed-form KV-cache size.                                               */
/*                                                                          */
/* [V] referee_report.major_comments[2] (Appendix I): with lprompt = 4096   */
/* and lgen = 512 MiniKV stores (0.5 * 4096 + 512) tokens per head and      */
/* layer, about 0.33 GB, against 2.4 GB for the full fp16 cache ([R] "The   */
/* reading": an 86% reduction).                                             */
/* reading: both K and V cost `bits` per element plus an fp16 scale and an  */
/*   fp16 zero per `group` elements; the full cache is fp16 K and V over    */
/*   lprompt + lgen tokens.  Sizes in bytes.                                */
/* ------------------------------------------------------------------------ */

double oracle_cache_bytes(int n_layers, int n_heads, int head_dim, int lprompt,
                          int lgen, double budget_frac, int bits, int group,
                          double *full_bytes)
{
    double tokens = budget_frac * lprompt + lgen;
    double bits_per_elem = (double)bits + 2.0 * 16.0 / (double)group;
    double elems = 2.0 * n_layers * (double)n_heads * head_dim;
    if (full_bytes)
        *full_bytes = elems * (double)(lprompt + lgen) * 2.0;
    return elems * tokens * bits_per_elem / 8.0;
}

/* ======================================================================== */
/* Mixed-precision caches: MiKV (important tokens at high precision, the    */
/* rest kept at low precision instead of evicted) and DiffKV (keys with     */
/* more bits than values; tiers K8V4 / K4V2 / pruned by significance).      */
/*                                                                          */
/* [M] "Don't Discard, but Keep It Small", rebuttal [W1] and the [UPDATED]  */
/* implementation paragraph: evicted KVs are kept in low precision and      */
/* important ones in high precision (an average of 3 bits between KIVI's 2  */
/* and 4); the KV pairs are regrouped by precision, which attention allows  */
/* because it does not depend on the order of the cached pairs, and each    */
/* precision group is stored contiguously and attended with its own INTn x  */
/* FP16 product.  The importance policy is H2O's cumulative score.          */
/* [D] verdict record for arXiv 2412.03131, key_machinery / core_discovery: */
/* significance = average attention a token receives from later tokens,   */
/* max over the query heads of a GQA group, against thresholds alpha/N;     */
/* above alpha_h/N keys 8 bits and values 4 bits, between alpha_l/N and     */
/* alpha_h/N keys 4 and values 2, below alpha_l/N pruned; decided per head. */
/* ======================================================================== */

/* b-bit asymmetric codec (b = 2, 4 or 8) on one group.
 * reading: as the INT2 codec with 2^b - 1 in place of 3: scale =
 *   fp16((max - min) / (2^b - 1)) from one fp32 subtraction and one
 *   correctly rounded fp32 division, zero = min (-0 -> +0), and the code is
 *   the round-half-even of the exact d / scale (d = fp32(x - zero)) clamped
 *   to [0, 2^b - 1]: the number of thresholds T_j = (j + 1/2) scale,
 *   j = 0 .. 2^b - 2, that d exceeds, a tie d == T_j counting only for odd
 *   j (then j + 1 is the even neighbour).  T_j is exact in fp32: j + 1/2 has
 *   at most 9 significant bits and scale 11. */
void oracle_quant_group_bits(const uint16_t *x, int G, long stride, int bits,
                             uint8_t *codes, uint16_t *scale_out,
                             uint16_t *zero_out)
{
    int top = (1 << bits) - 1;
    float mn = (float)oracle_h2d(x[0]);
    float mx = mn;
    for (int i = 1; i < G; ++i) {
        float xi = (float)oracle_h2d(x[(long)i * stride]);
        if (xi < mn) mn = xi;
        if (xi > mx) mx = xi;
    }
    float range = mx - mn;                        /* one fp32 rounding */
    float s32 = range / (float)top;               /* one fp32 rounding */
    uint16_t sh = oracle_f2h_rne(s32);
    uint16_t zh = oracle_f2h_rne(mn + 0.0f);      /* exact: mn is a half */
    float sf = (float)oracle_h2d(sh);
    float zf = (float)oracle_h2d(zh);
    *scale_out = sh;
    *zero_out = zh;
    for (int i = 0; i < G; ++i) {
        if (sf == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float d = (float)oracle_h2d(x[(long)i * stride]) - zf;
        int c = 0;
        for (int j = 0; j < top; ++j) {
            float t = ((float)j + 0.5f) * sf;     /* exact */
            if (d > t || (d == t && (j & 1)))
                c = j + 1;
        }
        codes[i] = (uint8_t)c;
    }
}

/* Pack one unit's selected tokens at key_bits / value_bits (2, 4 or 8; 2 or
 * 4 for values).
 * reading (bit planes): a b-bit code is stored as b/2 two-bit planes; plane
 *   p holds bits 2p..2p+1 of every code, each plane in exactly the INT2
 *   word layout (a key word: 16 channels of one token; a value word: 16
 *   tokens of one channel; element e at bits 2e..2e+1).  The pages fix no
 *   layout for 4- or 8-bit codes; planes keep one word format for every
 *   precision.  Scales and zero-points as for INT2.
 *   kq [key_bits/2][mp][D/16], vq [value_bits/2][mp/16][D] (plane-major),
 *   ks, kz [mp/Gk][D], vs, vz [mp][D/Gv]; the last m mod Gk selected
 *   tokens go to kres, vres [m - mp][D] as fp16.  Returns mp, -1 on bad
 *   arguments. */
int oracle_pack_unit_bits(int D, int Gk, int Gv, int key_bits, int value_bits,
                          const uint16_t *k, const uint16_t *v,
                          const int32_t *sel, int m, uint32_t *kq, uint16_t *ks,
                          uint16_t *kz, uint32_t *vq, uint16_t *vs, uint16_t *vz,
                          uint16_t *kres, uint16_t *vres)
{
    if (D % 16 || Gk % 16 || Gv % 16 || D % Gv || m < 0 || Gk <= 0 || Gv <= 0 ||
        (key_bits != 2 && key_bits != 4 && key_bits != 8) ||
        (value_bits != 2 && value_bits != 4))
        return -1;
    int mp = (m / Gk) * Gk;
    int kp = key_bits / 2, vp = value_bits / 2;
    long kplane = (long)mp * (D / 16), vplane = (long)(mp / 16) * D;
    uint16_t *x = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(Gk > Gv ? Gk : Gv));
    uint8_t *codes = (uint8_t *)malloc((size_t)(Gk > Gv ? Gk : Gv));

    memset(kq, 0, sizeof(uint32_t) * (size_t)(kplane * kp));
    for (int gi = 0; gi < mp / Gk; ++gi) {
        for (int c = 0; c < D; ++c) {
            for (int t = 0; t < Gk; ++t)
                x[t] = k[(long)sel[gi * Gk + t] * D + c];
            oracle_quant_group_bits(x, Gk, 1, key_bits, codes, &ks[(long)gi * D + c],
                                    &kz[(long)gi * D + c]);
            for (int t = 0; t < Gk; ++t) {
                long p = (long)gi * Gk + t;
                for (int pl = 0; pl < kp; ++pl)
                    kq[pl * kplane + p * (D / 16) + c / 16] |=
                        (uint32_t)((codes[t] >> (2 * pl)) & 3) << (2 * (c % 16));
            }
        }
    }
    memset(vq, 0, sizeof(uint32_t) * (size_t)(vplane * vp));
    for (int p = 0; p < mp; ++p) {
        const uint16_t *row = v + (long)sel[p] * D;
        for (int G = 0; G < D / Gv; ++G) {
            oracle_quant_group_bits(row + G * Gv, Gv, 1, value_bits, codes,
                                    &vs[(long)p * (D / Gv) + G],
                                    &vz[(long)p * (D / Gv) + G]);
            for (int i = 0; i < Gv; ++i) {
                int c = G * Gv + i;
                for (int pl = 0; pl < vp; ++pl)
                    vq[pl * vplane + (long)(p / 16) * D + c] |=
                        (uint32_t)((codes[i] >> (2 * pl)) & 3) << (2 * (p % 16));
            }
        }
    }
    for (int p = mp; p < m; ++p) {
        memcpy(kres + (long)(p - mp) * D, k + (long)sel[p] * D, sizeof(uint16_t) * D);
        memcpy(vres + (long)(p - mp) * D, v + (long)sel[p] * D, sizeof(uint16_t) * D);
    }
    free(x);
    free(codes);
    return mp;
}

/* Dequantised keys and values of the first n_packed tokens of one unit's
 * packed segment (layout of oracle_pack_unit_bits, with room for `cap`
 * tokens: plane strides cap*D/16 and cap/16*D words), as fp32 values
 * code * scale + zero stored in fp64 arrays kh, vh [n_packed][D]. */
int oracle_dequant_unit(int D, int Gk, int Gv, int key_bits, int value_bits,
                        int n_packed, int cap, const uint32_t *kq,
                        const uint16_t *ks, const uint16_t *kz,
                        const uint32_t *vq, const uint16_t *vs,
                        const uint16_t *vz, double *kh, double *vh)
{
    if (n_packed < 0 || n_packed > cap || n_packed % Gk || cap % 16 || D % 16 ||
        D % Gv)
        return -1;
    int kp = key_bits / 2, vp = value_bits / 2;
    long kplane = (long)cap * (D / 16), vplane = (long)(cap / 16) * D;
    for (int t = 0; t < n_packed; ++t) {
        for (int c = 0; c < D; ++c) {
            int kc = 0, vc = 0;
            for (int pl = 0; pl < kp; ++pl)
                kc |= (int)((kq[pl * kplane + (long)t * (D / 16) + c / 16] >>
                             (2 * (c % 16))) & 3u) << (2 * pl);
            for (int pl = 0; pl < vp; ++pl)
                vc |= (int)((vq[pl * vplane + (long)(t / 16) * D + c] >>
                             (2 * (t % 16))) & 3u) << (2 * pl);
            long km = (long)(t / Gk) * D + c;
            long vm = (long)t * (D / Gv) + c / Gv;
            kh[(long)t * D + c] = (double)oracle_dequant(kc, ks[km], kz[km]);
            vh[(long)t * D + c] = (double)oracle_dequant(vc, vs[vm], vz[vm]);
        }
    }
    return 0;
}

/* Plain softmax attention of g query heads (fp16 q [g][D]) over T given key
 * and value rows (fp64 [T][D]), scale 1/sqrt(D), fp64: o [g][D]. */
int oracle_attend(int D, int g, const uint16_t *q, int T, const double *kh,
                  const double *vh, double *o)
{
    if (T <= 0)
        return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    const double scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < g; ++h) {
        double M = -INFINITY;
        for (int t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += oracle_h2d(q[(long)h * D + c]) * kh[(long)t * D + c];
            s[t] = acc * scale;
            if (s[t] > M) M = s[t];
        }
        double l = 0.0;
        for (int t = 0; t < T; ++t) {
            s[t] = exp(s[t] - M);
            l += s[t];
        }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t)
                acc += s[t] * vh[(long)t * D + c];
            o[(long)h * D + c] = acc / l;
        }
    }
    free(s);
    return 0;
}

/* DiffKV significance of every prompt token of one unit: the average of the
 * attention it receives from the n - j causal rows i >= j, per query head,
 * then the max over the g query heads of the group.
 *   col_h [g][n]: per-head column sums (oracle_prefill_rows with g = 1).
 *   score[j] = max_h col_h[h][j] / (n - j). */
void oracle_diffkv_score(int n, int g, const double *col_h, double *score)
{
    for (int j = 0; j < n; ++j) {
        double m = -INFINITY;
        for (int h = 0; h < g; ++h)
            if (col_h[(long)h * n + j] > m) m = col_h[(long)h * n + j];
        score[j] = m / (double)(n - j);
    }
}

/* DiffKV tiers of one unit from its significance scores.
 * reading: cnt_hi = #{score > thr_hi}, cnt_kept = #{score > thr_lo}
 *   (thr = alpha / n; the caller passes the thresholds); each count is
 *   rounded up to a whole number of key groups (so every kept token sits in
 *   a full group, none is left over), capped at floor(n / Gk) * Gk, with
 *   kept >= hi.  The high tier is the first c_hi tokens in the order (score
 *   descending, index ascending), the low tier the next c_kept - c_hi; the
 *   rest are pruned.  Each tier is written in ascending index order.
 *   counts[0] = c_hi, counts[1] = c_kept - c_hi.  Returns 0, -1 on bad
 *   arguments. */
int oracle_diffkv_tiers(int n, const double *score, double thr_hi,
                        double thr_lo, int Gk, int32_t *hi, int32_t *lo,
                        int32_t *counts)
{
    if (n < 0 || Gk <= 0)
        return -1;
    int cnt_hi = 0, cnt_kept = 0;
    for (int j = 0; j < n; ++j) {
        if (score[j] > thr_hi) ++cnt_hi;
        if (score[j] > thr_lo) ++cnt_kept;
    }
    int cap = (n / Gk) * Gk;
    int c_hi = (cnt_hi + Gk - 1) / Gk * Gk;
    int c_kept = (cnt_kept + Gk - 1) / Gk * Gk;
    if (c_hi > cap) c_hi = cap;
    if (c_kept > cap) c_kept = cap;
    if (c_kept < c_hi) c_kept = c_hi;
    scored_t *cand = (scored_t *)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    for (int j = 0; j < n; ++j) {
        cand[j].score = score[j];
        cand[j].idx = j;
    }
    qsort(cand, (size_t)n, sizeof(scored_t), cmp_scored);
    for (int t = 0; t < c_hi; ++t) hi[t] = cand[t].idx;
    for (int t = c_hi; t < c_kept; ++t) lo[t - c_hi] = cand[t].idx;
    qsort(hi, (size_t)c_hi, sizeof(int32_t), cmp_i32);
    qsort(lo, (size_t)(c_kept - c_hi), sizeof(int32_t), cmp_i32);
    counts[0] = c_hi;
    counts[1] = c_kept - c_hi;
    free(cand);
    return 0;
}
