/*
 * csa_oracle.c -- plain, slow, obviously correct CPU oracle for compressed
 * sparse attention (CSA) and heavily compressed attention (HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the tests, the smoke check and the CPU baseline of
 * the benchmark use it.  It shares no header, helper, table or constant with
 * the GPU library.
 *
 * Sources (all describe the method in prose; none prints a formula):
 *   [P1] hazakura.dev "DeepSeek V4とOpenCode", section "衝撃1：CSA + HCA"
 *   [P3] jiwasawa.github.io "deepseek-v4" post, section "コンテキストの壁を
 *        突破するハイブリッド Attention 機構" (sub-parts CSA and HCA)
 *   [P4] studioglobal.ai "DeepSeek V4 Flash" answer, sections "アテンションの
 *        ブレイクスルー：CSAとHCA" and "FP4/FP8混合精度"
 *   [P5] ai-papers.net "deepseek-v4-1m-context-window...", section
 *        "ハイブリッドアテンションの仕組み"
 *
 * Arithmetic: every floating-point step is done in double precision.  The
 * indexer score is computed exactly (it is a sum of products of FP4 grid
 * values and powers of two) and a guard reports whether that exact value is
 * representable in binary32 under every summation order.
 *
 * Pins: see tests/test_oracle_*.py.  The readings taken where the pages are
 * silent (pooling formula, window/compressed overlap, score form, MXFP4
 * rounding, tie order) are listed with each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

/* ------------------------------------------------------------------------ */
/* Step 1: sequence compression by softmax-gated pooling.                    */
/*                                                                          */
/* [P3, CSA, token-level compression]: the KV of m adjacent tokens becomes  */
/* one entry, so the effective length is 1/m.  [P4, CSA bullet]: the        */
/* operator is softmax-gated pooling.  [P1 and P3, HCA]: the same with a    */
/* much larger m'.                                                          */
/* Reading: blocks are aligned and do not overlap (block j = tokens         */
/* m*j .. m*j+m-1); only complete blocks are emitted; for every channel c   */
/* the weights are a softmax over the block's m gate logits of that channel */
/* (or of the single per-token logit when gate_channels == 1):              */
/*     out[b][j][c] = sum_i  exp(z_i - max_z) / sum_i' exp(z_i' - max_z)    */
/*                           * x[b][m*j+i][c]                               */
/* ------------------------------------------------------------------------ */
int oracle_compress(int64_t B, int64_t T, int64_t C, int64_t m,
                    const double *x, const double *gate, int64_t gate_channels,
                    double *out)
{
    if (B < 0 || T < 0 || C <= 0 || m <= 0) return 1;
    if (gate_channels != 1 && gate_channels != C) return 1;
    int64_t nout = T / m;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t j = 0; j < nout; ++j) {
            for (int64_t c = 0; c < C; ++c) {
                int64_t gc = (gate_channels == 1) ? 0 : c;
                double zmax = -INFINITY;
                for (int64_t i = 0; i < m; ++i) {
                    double z = gate[(b * T + m * j + i) * gate_channels + gc];
                    if (z > zmax) zmax = z;
                }
                double den = 0.0;
                for (int64_t i = 0; i < m; ++i) {
                    double z = gate[(b * T + m * j + i) * gate_channels + gc];
                    den += exp(z - zmax);
                }
                double acc = 0.0;
                for (int64_t i = 0; i < m; ++i) {
                    double z = gate[(b * T + m * j + i) * gate_channels + gc];
                    double w = exp(z - zmax) / den;
                    acc += w * x[(b * T + m * j + i) * C + c];
                }
                out[(b * nout + j) * C + c] = acc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 2: MXFP4 quantisation.                                              */
/*                                                                          */
/* [P4, FP4/FP8 mixed precision]: MXFP4 packs two 4-bit values per byte.    */
/* [P1, P3, P5]: the indexer runs at FP4.  Reading (OCP Microscaling v1.0): */
/* every run of 32 consecutive values shares one power-of-two scale 2^e,    */
/* stored as a biased byte e+127 (E8M0), with                               */
/*     e = floor(log2(max |x|)) - 2     (2 = largest exponent of e2m1),     */
/* clamped to [-127, 127]; an all-zero block takes e = -127.  Each value    */
/* x*2^-e is rounded to the nearest e2m1 magnitude                          */
/*     {0, 0.5, 1, 1.5, 2, 3, 4, 6}   (codes 0..7),                         */
/* ties to the even code, anything beyond 6 saturating to 6; the sign bit   */
/* (bit 3) copies the sign bit of x.  Element 2i of a row goes in the low   */
/* nibble of byte i, element 2i+1 in the high nibble.                       */
/* ------------------------------------------------------------------------ */
static const double E2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static int e2m1_round(double y)       /* y >= 0; nearest, ties to even code */
{
    int best = 0;
    double bestd = fabs(y - E2M1[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(y - E2M1[c]);
        if (d < bestd || (d == bestd && (c % 2 == 0) && (best % 2 != 0))) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

int oracle_quant_mxfp4(int64_t rows, int64_t d, const double *x,
                       uint8_t *codes, uint8_t *scales)
{
    if (rows < 0 || d <= 0 || d % 32 != 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t blk = 0; blk < d / 32; ++blk) {
            const double *v = x + r * d + blk * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i)
                if (fabs(v[i]) > amax) amax = fabs(v[i]);
            int e;
            if (amax == 0.0) {
                e = -127;
            } else {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1) */
                e = (ex - 1) - 2;          /* floor(log2 amax) - 2 */
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            scales[r * (d / 32) + blk] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                double y = ldexp(fabs(v[i]), -e);
                int code = e2m1_round(y) | (signbit(v[i]) ? 8 : 0);
                int64_t idx = blk * 32 + i;
                uint8_t *byte = codes + r * (d / 2) + idx / 2;
                if (idx % 2 == 0) *byte = (uint8_t)((*byte & 0xF0) | code);
                else              *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
            }
        }
    }
    return 0;
}

/* Value of one MXFP4 element: (-1)^s * e2m1[code & 7] * 2^(scale-127). */
double oracle_mxfp4_value(int code, int scale)
{
    double g = E2M1[code & 7];
    if (code & 8) g = -g;
    return ldexp(g, scale - 127);
}

/* ------------------------------------------------------------------------ */
/* Step 2b: FP8 storage of the compressed KV entries.                       */
/*                                                                          */
/* [P5, hybrid attention section]: most KV entries are stored in FP8, the   */
/* indexer runs at FP4.  [P4, FP4/FP8 mixed precision]: the FP4 side is     */
/* MXFP4.  Reading: "most" are the compressed entries (the raw window of W  */
/* tokens stays in the compute type), in the FP8 member of the same OCP     */
/* Microscaling family, MXFP8 E4M3: every run of 32 values shares a scale   */
/* 2^e stored as the byte e+127 with                                        */
/*     e = floor(log2(max |x|)) - 8     (8 = largest exponent of E4M3),     */
/* clamped to [-127, 127]; an all-zero run takes e = -127.  Each x*2^-e is  */
/* rounded to the nearest E4M3 magnitude (bias 7, three mantissa bits,      */
/* subnormals k*2^-9, largest finite 448; the all-ones code is NaN and is   */
/* never produced), ties to the even code, anything beyond 448 saturating   */
/* to 448; bit 7 copies the sign bit of x.                                  */
/* ------------------------------------------------------------------------ */

/* magnitude of E4M3 code c in 0..126 */
double oracle_e4m3_value(int c)
{
    c &= 0x7F;
    if (c < 8) return ldexp((double)c, -9);
    return ldexp(1.0 + (c & 7) / 8.0, (c >> 3) - 7);
}

static int e4m3_round(double y)       /* y >= 0; nearest, ties to even code */
{
    int best = 0;
    double bestd = y;
    for (int c = 1; c < 127; ++c) {
        double d = fabs(y - oracle_e4m3_value(c));
        if (d < bestd || (d == bestd && (c % 2 == 0) && (best % 2 != 0))) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* E4M3 encoding of rows of d values in runs of `run` values (run divides d), */
/* each run with its own scale exponent by the rule above; scales get one    */
/* byte per 32 values, the run's exponent repeated over the run.             */
static int quant_e4m3_runs(int64_t rows, int64_t d, int64_t run, const double *x,
                           uint8_t *codes, uint8_t *scales)
{
    if (rows < 0 || d <= 0 || d % 32 != 0 || run <= 0 || run % 32 != 0 || d % run != 0)
        return 1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t blk = 0; blk < d / run; ++blk) {
            const double *v = x + r * d + blk * run;
            double amax = 0.0;
            for (int64_t i = 0; i < run; ++i)
                if (fabs(v[i]) > amax) amax = fabs(v[i]);
            int e;
            if (amax == 0.0) {
                e = -127;
            } else {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1) */
                e = (ex - 1) - 8;          /* floor(log2 amax) - 8 */
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            for (int64_t s32 = 0; s32 < run / 32; ++s32)
                scales[r * (d / 32) + blk * (run / 32) + s32] = (uint8_t)(e + 127);
            for (int64_t i = 0; i < run; ++i) {
                double y = ldexp(fabs(v[i]), -e);
                codes[r * d + blk * run + i] =
                    (uint8_t)(e4m3_round(y) | (signbit(v[i]) ? 0x80 : 0));
            }
        }
    }
    return 0;
}

int oracle_quant_mxfp8(int64_t rows, int64_t d, const double *x,
                       uint8_t *codes, uint8_t *scales)
{
    return quant_e4m3_runs(rows, d, 32, x, codes, scales);
}

/* ------------------------------------------------------------------------ */
/* Step 2c: FP8 rows for FP8 attention arithmetic.                          */
/*                                                                          */
/* [P5, hybrid attention section]: most KV entries in FP8.  Reading R13d:   */
/* when attention itself runs in FP8, every row it reads (compressed K and  */
/* V entries, raw window rows, and each query head's row) is E4M3 with ONE  */
/* scale exponent for the whole row of d values, by the same rule as the    */
/* 32-value runs above (e = floor(log2 max|x|) - 8 over the row).  One      */
/* exponent per key is what a product that contracts over keys (P V) can   */
/* carry; the exponent is stored in each of the row's d/32 scale bytes, so  */
/* the result is also a valid MXFP8 row and decodes as one.                 */
/* ------------------------------------------------------------------------ */
int oracle_quant_fp8_rows(int64_t rows, int64_t d, const double *x,
                          uint8_t *codes, uint8_t *scales)
{
    return quant_e4m3_runs(rows, d, d, x, codes, scales);
}

/* Value of one MXFP8 element: (-1)^s * e4m3[code & 127] * 2^(scale-127). */
double oracle_mxfp8_value(int code, int scale)
{
    double g = oracle_e4m3_value(code & 0x7F);
    if (code & 0x80) g = -g;
    return ldexp(g, scale - 127);
}

/* ------------------------------------------------------------------------ */
/* Candidate set of a query.                                                */
/*                                                                          */
/* [P1 CSA bullets; P3 SWA branch; P4 CSA/HCA section]: a branch that      */
/* attends the newest W = 128 tokens uncompressed is always present.       */
/*  Reading: the window of a query at position t is the raw   */
/* tokens w0..t with w0 = max(0, t-W+1); a compressed block j is a          */
/* candidate when it is complete and visible (m*j+m-1 <= t) and starts      */
/* before the window (m*j < w0), so no token is reached twice through a     */
/* block that lies wholly inside the window.                                */
/* ------------------------------------------------------------------------ */
int64_t oracle_n_cand(int64_t t, int64_t m, int64_t W)
{
    int64_t w0 = t - W + 1;
    if (w0 < 0) w0 = 0;
    int64_t n = 0;
    for (int64_t j = 0; m * j + m - 1 <= t && m * j < w0; ++j) n++;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Step 3: Lightning Indexer score.                                         */
/*                                                                          */
/* [P3, CSA, indexer bullet]: every query token scores the compressed       */
/* entries with a lightweight indexer.  [P1, P5]: at FP4.  Reading: one     */
/* indexer key per compressed entry shared by the indexer heads, unit head  */
/* weights, and a ReLU per head before the head sum:                        */
/*     I(t, j) = sum_h max(0, qhat[t][h] . khat[j])                         */
/* The value is computed exactly from the integer codes: within a 32-block  */
/* every product of two e2m1 magnitudes is an integer multiple of 1/4, so   */
/* the block dot product is  S * 2^(eq + ek - 2)  with S an integer.        */
/* *exact is cleared when some partial sum of the terms could need more     */
/* than 24 significant bits, i.e. when binary32 accumulation in an          */
/* arbitrary order might not reproduce the exact value.                     */
/* ------------------------------------------------------------------------ */
static int nib(const uint8_t *codes, int64_t i)
{
    uint8_t b = codes[i / 2];
    return (i % 2 == 0) ? (b & 0xF) : (b >> 4);
}

static int64_t twice_mag(int code)     /* 2 * e2m1 magnitude, an integer */
{
    static const int64_t T2[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    return T2[code & 7];
}

/* Exact score of query row (HI heads) against one key. */
static float score_one(int64_t HI, int64_t dI,
                       const uint8_t *qc, const uint8_t *qs,
                       const uint8_t *kc, const uint8_t *ks, int *exact)
{
    int64_t nb = dI / 32;
    /* Every term is an integer multiple of 2^(emin-2); find emin and the sum */
    /* of |terms| in those units to run the exactness guard.                 */
    int emin = 1 << 20;
    for (int64_t h = 0; h < HI; ++h)
        for (int64_t b = 0; b < nb; ++b) {
            int e = (qs[h * nb + b] - 127) + (ks[b] - 127);
            if (e < emin) emin = e;
        }
    long double abs_units = 0.0L;      /* sum |terms| / 2^(emin-2)          */
    double total = 0.0;
    for (int64_t h = 0; h < HI; ++h) {
        double head = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            int64_t S = 0, Sabs = 0;
            for (int64_t i = 0; i < 32; ++i) {
                int a = nib(qc + h * (dI / 2), b * 32 + i);
                int c = nib(kc, b * 32 + i);
                int64_t p = twice_mag(a) * twice_mag(c);
                if ((a ^ c) & 8) p = -p;
                S += p;
                Sabs += (p < 0 ? -p : p);
            }
            int e = (qs[h * nb + b] - 127) + (ks[b] - 127);
            head += ldexp((double)S, e - 2);      /* exact: |S| < 2^13 */
            abs_units += ldexpl((long double)Sabs, e - emin);
        }
        if (head > 0.0) total += head;
    }
    if (abs_units >= 16777216.0L) *exact = 0;   /* 2^24 units */
    float f = (float)total;
    if ((double)f != total) *exact = 0;
    if (f == 0.0f) f = 0.0f;                    /* canonical +0 */
    return f;
}

/* Scores of every (query, key) pair; non-candidates are written as -1.    */
/* qc [B,Tq,HI,dI/2], qs [B,Tq,HI,dI/32], kc [B,Nc,dI/2], ks [B,Nc,dI/32],  */
/* q_pos [Tq] positions (shared by the batch), scores [B,Tq,Nc].           */
int oracle_index_scores(int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                        int64_t Nc, int64_t m, int64_t W, const int64_t *q_pos,
                        const uint8_t *qc, const uint8_t *qs,
                        const uint8_t *kc, const uint8_t *ks,
                        float *scores, int *exact)
{
    if (dI % 32 != 0) return 1;
    *exact = 1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Tq; ++q) {
            int64_t nc = oracle_n_cand(q_pos[q], m, W);
            if (nc > Nc) return 2;
            for (int64_t j = 0; j < Nc; ++j) {
                float s = -1.0f;
                if (j < nc)
                    s = score_one(HI, dI,
                                  qc + ((b * Tq + q) * HI) * (dI / 2),
                                  qs + ((b * Tq + q) * HI) * (dI / 32),
                                  kc + (b * Nc + j) * (dI / 2),
                                  ks + (b * Nc + j) * (dI / 32), exact);
                scores[(b * Tq + q) * Nc + j] = s;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 4: top-k selection.                                                 */
/*                                                                          */
/* [P3, CSA, indexer bullet]: a top-k selector keeps the k compressed       */
/* entries with the highest scores.  [P4, CSA bullet]: k = 512 blocks per   */
/* query.  Reading: order by (score descending, index ascending), take the  */
/* first min(k, n_cand), emit them in ascending index order, pad with -1.   */
/* ------------------------------------------------------------------------ */
typedef struct { float s; int32_t j; } cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int int_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

static void select_row(const float *s, int64_t nc, int64_t k, int32_t *out,
                       cand_t *buf)
{
    for (int64_t j = 0; j < nc; ++j) { buf[j].s = s[j]; buf[j].j = (int32_t)j; }
    qsort(buf, (size_t)nc, sizeof(cand_t), cand_cmp);
    int64_t n = nc < k ? nc : k;
    for (int64_t i = 0; i < n; ++i) out[i] = buf[i].j;
    qsort(out, (size_t)n, sizeof(int32_t), int_cmp);
    for (int64_t i = n; i < k; ++i) out[i] = -1;
}

int oracle_select_topk(int64_t B, int64_t Tq, int64_t Nc, int64_t m, int64_t W,
                       int64_t k, const int64_t *q_pos, const float *scores,
                       int32_t *topk)
{
    cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(Nc > 0 ? Nc : 1));
    if (!buf) return 3;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Tq; ++q) {
            int64_t nc = oracle_n_cand(q_pos[q], m, W);
            if (nc > Nc) { free(buf); return 2; }
            select_row(scores + (b * Tq + q) * Nc, nc, k,
                       topk + (b * Tq + q) * k, buf);
        }
    free(buf);
    return 0;
}

/* Steps 3+4 fused per row so that large problems need no [Tq,Nc] buffer.   */
/* Rows are independent; OpenMP only spreads them over host threads.       */
int oracle_index_topk(int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                      int64_t Nc, int64_t m, int64_t W, int64_t k,
                      const int64_t *q_pos,
                      const uint8_t *qc, const uint8_t *qs,
                      const uint8_t *kc, const uint8_t *ks,
                      int32_t *topk, int *exact)
{
    if (dI % 32 != 0) return 1;
    for (int64_t q = 0; q < Tq; ++q)
        if (oracle_n_cand(q_pos[q], m, W) > Nc) return 2;
    int ex_all = 1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(&& : ex_all)
    for (int64_t bq = 0; bq < B * Tq; ++bq) {
        int64_t b = bq / Tq, q = bq % Tq;
        int64_t nc = oracle_n_cand(q_pos[q], m, W);
        float *s = (float *)malloc(sizeof(float) * (size_t)(nc > 0 ? nc : 1));
        cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nc > 0 ? nc : 1));
        if (!s || !buf) {
#pragma omp atomic write
            err = 3;
        } else {
            int ex = 1;
            for (int64_t j = 0; j < nc; ++j)
                s[j] = score_one(HI, dI,
                                 qc + (bq * HI) * (dI / 2),
                                 qs + (bq * HI) * (dI / 32),
                                 kc + (b * Nc + j) * (dI / 2),
                                 ks + (b * Nc + j) * (dI / 32), &ex);
            select_row(s, nc, k, topk + bq * k, buf);
            ex_all = ex_all && ex;
        }
        free(s);
        free(buf);
    }
    *exact = ex_all;
    return err;
}

/* ------------------------------------------------------------------------ */
/* Step 5: attention over the selected (CSA) or all (HCA) compressed        */
/* entries joined with the raw window.                                      */
/*                                                                          */
/* [P3, CSA, "Shared Key-Value MQA" bullet]: multi-query attention over the */
/* k selected entries, one key/value head shared by every query head.       */
/* [P3, HCA; P1 HCA bullets]: HCA attends densely over every compressed     */
/* entry.  [P3, SWA branch; P4]: a sliding window over the newest 128       */
/* tokens is always present.  Reading: one softmax over the union of the    */
/* compressed key set and the raw window w0..t:                             */
/*     l_s = scale * q[t][h] . key_s,   o[t][h] = sum_s softmax(l)_s val_s   */
/* topk == NULL selects every candidate (HCA).  With topk given, only its  */
/* first min(k, n_cand) slots are read (the selector fills exactly those);  */
/* a slot holding an index outside [0, n_cand) contributes nothing.         */
/* q [B,Tq,H,D], ck/cv [B,Nc,D], topk [B,Tq,k], rk/rv [B,raw_len,D] with    */
/* raw row r at position raw_pos0 + r, o [B,Tq,H,D].                        */
/* ------------------------------------------------------------------------ */
/* As oracle_attend below; when amean / rms are given ([B,Tq,H,D] each), */
/* they receive, per output element, the weighted means                   */
/*     amean = sum_s p_s |v_s[c]| / sum_s p_s,                             */
/*     rms   = sqrt(sum_s p_s^2 v_s[c]^2) / sum_s p_s,                     */
/* of the softmax weights p_s over the key list: the scales on which a     */
/* relative perturbation of each weight moves the output (its worst case   */
/* and its root-mean-square for independent perturbations).                */
int oracle_attend_stats(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                        int64_t m, int64_t W, int64_t k, const int64_t *q_pos,
                        double scale, const double *q, const double *ck,
                        const double *cv, const int32_t *topk, const double *rk,
                        const double *rv, int64_t raw_pos0, int64_t raw_len,
                        double *o, double *amean, double *rms)
{
    for (int64_t i = 0; i < Tq; ++i) {
        int64_t t = q_pos[i];
        int64_t w0 = t - W + 1 < 0 ? 0 : t - W + 1;
        if (oracle_n_cand(t, m, W) > Nc) return 2;
        if (w0 < raw_pos0 || t >= raw_pos0 + raw_len) return 4;
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bq = 0; bq < B * Tq; ++bq) {
        int64_t b = bq / Tq, i = bq % Tq;
        int64_t t = q_pos[i];
        int64_t w0 = t - W + 1 < 0 ? 0 : t - W + 1;
        int64_t nc = oracle_n_cand(t, m, W);
        /* key list: compressed entries (index >= 0) then raw rows           */
        int64_t nsel = topk ? (k < nc ? k : nc) : nc;
        int64_t nkeys = nsel + (t - w0 + 1);
        const double **kp = (const double **)malloc(sizeof(double *) * (size_t)nkeys);
        const double **vp = (const double **)malloc(sizeof(double *) * (size_t)nkeys);
        double *l = (double *)malloc(sizeof(double) * (size_t)nkeys);
        if (!kp || !vp || !l) {
#pragma omp atomic write
            err = 3;
            free(kp); free(vp); free(l);
            continue;
        }
        int64_t n = 0;
        for (int64_t s = 0; s < nsel; ++s) {
            int64_t j = topk ? topk[bq * k + s] : s;
            if (j < 0 || j >= nc) continue;    /* not a candidate: ignored */
            kp[n] = ck + (b * Nc + j) * D;
            vp[n] = cv + (b * Nc + j) * D;
            n++;
        }
        for (int64_t u = w0; u <= t; ++u) {
            kp[n] = rk + (b * raw_len + (u - raw_pos0)) * D;
            vp[n] = rv + (b * raw_len + (u - raw_pos0)) * D;
            n++;
        }
        for (int64_t h = 0; h < H; ++h) {
            const double *qv = q + ((b * Tq + i) * H + h) * D;
            double lmax = -INFINITY;
            for (int64_t s = 0; s < n; ++s) {
                double dot = 0.0;
                for (int64_t c = 0; c < D; ++c) dot += qv[c] * kp[s][c];
                l[s] = scale * dot;
                if (l[s] > lmax) lmax = l[s];
            }
            double den = 0.0;
            for (int64_t s = 0; s < n; ++s) den += exp(l[s] - lmax);
            double *ov = o + ((b * Tq + i) * H + h) * D;
            for (int64_t c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int64_t s = 0; s < n; ++s)
                    acc += exp(l[s] - lmax) / den * vp[s][c];
                ov[c] = acc;
            }
            if (amean && rms) {
                double *av = amean + ((b * Tq + i) * H + h) * D;
                double *rv2 = rms + ((b * Tq + i) * H + h) * D;
                for (int64_t c = 0; c < D; ++c) {
                    double a = 0.0, r2 = 0.0;
                    for (int64_t s = 0; s < n; ++s) {
                        double p = exp(l[s] - lmax) / den;
                        a += p * fabs(vp[s][c]);
                        r2 += p * p * vp[s][c] * vp[s][c];
                    }
                    av[c] = a;
                    rv2[c] = sqrt(r2);
                }
            }
        }
        free(kp); free(vp); free(l);
    }
    return err;
}

int oracle_attend(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                  int64_t m, int64_t W, int64_t k, const int64_t *q_pos,
                  double scale, const double *q, const double *ck,
                  const double *cv, const int32_t *topk, const double *rk,
                  const double *rv, int64_t raw_pos0, int64_t raw_len,
                  double *o)
{
    return oracle_attend_stats(B, Tq, H, D, Nc, m, W, k, q_pos, scale, q, ck, cv, topk,
                               rk, rv, raw_pos0, raw_len, o, NULL, NULL);
}
