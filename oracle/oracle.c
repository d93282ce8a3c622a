/*
 * oracle.c -- plain, slow fp64 CPU reference for block-sparse causal attention
 * with learned block selection (block summaries -> scores -> optional softmax
 * log gate -> top-K -> exact softmax attention -> backward incl. gate grad).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: it decodes its own inputs, rounds with its own routines and
 * follows the definitions below loop by loop.
 *
 * Sources (pages of the reference, cited by title and section):
 *  [SAS]  "SAS: Simple Attention Sparsification via End-to-End Optimization of
 *         Context Ranking" (review page).  Background §3 Eq. 1-3 (attention,
 *         block-sparse attention, C = n/b blocks + selector + top-K);
 *         §4.1 Eq. 4 (historical set H, current block B0 with gate 1);
 *         §4.2.2 Eq. 5 (inner-gate gradient), softmax gate
 *         log g = s - LSE(s); §4.3 Eq. 9 (log-gate bias inside the softmax);
 *         Alg. 1 / Alg. 2 and the worked example (n=256, b=64, K=2).
 *  [FS]   "FreeSolo ... zero-shot retrieval up to 64x the training length"
 *         (review page), section "How it works": cells of s tokens, mean key,
 *         centre position, max key norm, query-block prefix of B=128,
 *         r_ic = q_i.kbar_c/sqrt(d) + lambda_h a_c erf((i-p_c)/(2 sigma_h)),
 *         per-query top-K cells read with one softmax, sliding-window branch
 *         of w tokens, per-head alpha_h mix.
 *  [MONO] "Monodratic claims learned routing ..." (news page): guaranteed
 *         local block + exact causal softmax over the selected set.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - 1/sqrt(d) scaling of every dot product (stated only on [FS]).
 *  - n context positions form C historical blocks; the query sits in the
 *    current block B0 = floor(i/b); candidates are c < floor(i/b) [SAS].
 *    [FS] candidates are cells fully before the query block:
 *    (c+1) s <= B floor(i/B).
 *  - GQA: with share_group=1 one selection per kv head from the mean of
 *    its G query heads (score = mean of the per-head scores).
 *  - Gate LSE runs over ALL candidates (the worked example normalises over
 *    all four blocks, then biases the two chosen ones).
 *  - Ties: higher score first, lower block index wins; indices are emitted
 *    in ascending order, -1 padded; K_eff = min(K, #candidates).
 *  - Summaries: exact mean rounded to nearest-even in the key dtype;
 *    a_c = max over the block of the L2 norm, rounded to fp32;
 *    p_c = c b + (b-1)/2.
 *  - Mix: o = alpha_h o_L + (1 - alpha_h) o_S, o_L = 0 when no cell exists.
 *  - Backward: dS_ij = p_ij (do_i.v_j - do_i.o_i); dg_m = sum_{j in B_m}
 *    dS_ij / g_m, summed over the query heads sharing the gate.
 *
 * Layouts (all row-major, contiguous):
 *   q [B, Hq, nq, d], k/v [B, Hkv, L, d], kbar [B, Hkv, Ccap, d],
 *   max_norm [B, Hkv, Ccap], centre [Ccap], idx/logg [B, Hsel, nq, K].
 *   dtype 0 = fp32, 1 = bf16 (raw uint16 bit patterns), 2 = fp64 (summaries
 *   rebuilt from fp8 codes, exact).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

/* ---------------------------------------------------------------- decode */

static double orc_bf16_to_double(uint16_t h)
{
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double orc_load(const void *p, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_double(((const uint16_t *)p)[i]);
    if (dtype == ORC_F64)
        return ((const double *)p)[i];
    return (double)((const float *)p)[i];
}

/* Round a double to the nearest bf16 (ties to even), directly from the
 * double: quantum = 2^(e-8) for x = m 2^e, m in [0.5, 1), floored at the
 * bf16 subnormal spacing 2^-133.  The rounded value is exact in fp32. */
static uint16_t orc_double_to_bf16_rne(double x)
{
    if (x == 0.0) {
        return signbit(x) ? 0x8000u : 0u;
    }
    int e;
    (void)frexp(x, &e);
    int qexp = e - 8;
    if (qexp < -133)
        qexp = -133;
    double scaled = ldexp(x, -qexp);          /* exact: power-of-two scale */
    double r = nearbyint(scaled);             /* ties-to-even (default mode) */
    double v = ldexp(r, qexp);
    float f = (float)v;                       /* exact: v has <= 8 bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(bits >> 16);
}

static void orc_store_key_dtype(void *p, int dtype, int64_t i, double x)
{
    if (dtype == ORC_BF16)
        ((uint16_t *)p)[i] = orc_double_to_bf16_rne(x);
    else
        ((float *)p)[i] = (float)x;           /* C conversion rounds to nearest even */
}

/* Exposed so the tests can pin the rounding against known bit patterns. */
uint16_t orc_round_bf16(double x) { return orc_double_to_bf16_rne(x); }

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------- fp8 summaries (decode) */
/*
 * Optional 8-bit block summaries for the decode scorer.  Format: OCP 8-bit
 * floating point, E4M3 with no infinities (sign, 4 exponent bits biased by
 * 7, 3 mantissa bits; exponent field 0 is subnormal, value m/8 2^-6; the all-
 * ones pattern S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 2^8 = 448).  Each block c of each (batch, kv head) is scaled by its
 * largest magnitude: amax = max_e |kbar_c[e]|, inv = 448 / amax and
 * scale_c = amax / 448, both single precision (IEEE division), y_e =
 * kbar_c[e] inv (single precision product), code_e = y_e rounded to the
 * nearest E4M3 value (ties to the even code), magnitudes past 448 held at
 * 448, the sign kept (so -0 and negatives that round to zero give 0x80).
 * A block of zeros has scale 0 and zero codes.  The summary the scorer reads
 * is scale_c decode(code_e).  (The scale and code arithmetic is single
 * precision on purpose: it decides integer codes, and both sides take that
 * decision in the same precision.)
 */
double orc_fp8_decode(uint8_t code)
{
    int sgn = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    double v;
    if (ex == 15 && man == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)man, -9);                   /* m/8 2^-6 */
    else
        v = ldexp(8.0 + man, ex - 10);                /* (1 + m/8) 2^(e-7) */
    return sgn ? -v : v;
}

/* Nearest E4M3 magnitude code to |y| by brute force over the 127 finite
 * non-negative codes (ties to the even code), sign from y. */
uint8_t orc_fp8_encode(float y)
{
    double a = fabs((double)y);
    int best = 0;
    double bd = INFINITY;
    if (a >= 448.0) {
        best = 0x7E;
    } else {
        for (int c = 0; c <= 0x7E; ++c) {
            double dlt = fabs(orc_fp8_decode((uint8_t)c) - a);
            if (dlt < bd || (dlt == bd && (c & 1) == 0 && (best & 1) == 1)) {
                bd = dlt;
                best = c;
            }
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* codes [B, Hkv, Ccap, d] uint8 and scales [B, Hkv, Ccap] fp32 of blocks
 * [first, first + num) from kbar [B, Hkv, Ccap, d] (dtype). */
void orc_quantize_fp8(const void *kbar, int dtype, int B, int Hkv, int64_t Ccap, int d, int64_t first,
                      int64_t num, uint8_t *codes, float *scales)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < (int64_t)B * Hkv; ++bh) {
        for (int64_t c = first; c < first + num; ++c) {
            const int64_t row = (bh * Ccap + c) * (int64_t)d;
            float amax = 0.0f;
            for (int e = 0; e < d; ++e) {
                float x = (float)orc_load(kbar, dtype, row + e);
                if (fabsf(x) > amax)
                    amax = fabsf(x);
            }
            if (amax == 0.0f) {
                scales[bh * Ccap + c] = 0.0f;
                for (int e = 0; e < d; ++e)
                    codes[row + e] = 0;
                continue;
            }
            volatile float inv = 448.0f / amax;       /* single precision, as the format rule says */
            volatile float sc = amax / 448.0f;
            scales[bh * Ccap + c] = sc;
            for (int e = 0; e < d; ++e) {
                volatile float y = (float)orc_load(kbar, dtype, row + e) * inv;
                codes[row + e] = orc_fp8_encode(y);
            }
        }
    }
}

/* The summaries the scorer reads, exact in fp64: out = scale_c decode(code). */
void orc_dequantize_fp8(const uint8_t *codes, const float *scales, int64_t rows, int d, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int e = 0; e < d; ++e)
            out[r * d + e] = (double)scales[r] * orc_fp8_decode(codes[r * d + e]);
}

/* ------------------------------------------------------ a1: summaries */
/*
 * [SAS] §3 Eq. 3 partitions the context into blocks of b tokens and the
 * selector reads a pooled key summary of each; [FS] "How it works" names the
 * three cell summaries: mean key, centre position, max key norm.
 * Summarises blocks c in [0, nblocks) (each must be full: (c+1) b <= L).
 */
void orc_block_summaries(const void *k, int dtype, int B, int Hkv, int64_t L,
                         int d, int b, int64_t nblocks, int64_t Ccap,
                         void *kbar, float *max_norm, float *centre)
{
    int64_t bh;
#pragma omp parallel for schedule(dynamic)
    for (bh = 0; bh < (int64_t)B * Hkv; ++bh) {
        const int64_t kbase = bh * L * d;
        for (int64_t c = 0; c < nblocks; ++c) {
            /* mean key: exact fp64 sum, divided by b (a power of two) */
            for (int e = 0; e < d; ++e) {
                double sum = 0.0;
                for (int j = 0; j < b; ++j)
                    sum += orc_load(k, dtype, kbase + (c * b + j) * (int64_t)d + e);
                orc_store_key_dtype(kbar, dtype, (bh * Ccap + c) * (int64_t)d + e,
                                    sum / (double)b);
            }
            /* max key norm over the block */
            double best = 0.0;
            for (int j = 0; j < b; ++j) {
                double ss = 0.0;
                for (int e = 0; e < d; ++e) {
                    double x = orc_load(k, dtype, kbase + (c * b + j) * (int64_t)d + e);
                    ss += x * x;
                }
                double nrm = sqrt(ss);
                if (nrm > best)
                    best = nrm;
            }
            max_norm[bh * Ccap + c] = (float)best;
        }
    }
    if (centre) {
        for (int64_t c = 0; c < nblocks; ++c)
            centre[c] = (float)((double)c * b + (double)(b - 1) / 2.0);
    }
}

/* ------------------------------------------------------ candidates */
/* prefix_mode 0 = current block ([SAS] historical blocks before B0),
 *             1 = query-block prefix ([FS] cells before the query block). */
int64_t orc_num_candidates(int64_t i, int b, int prefix_mode, int qblock)
{
    if (prefix_mode == 0)
        return i / b;
    return (qblock * (i / qblock)) / b;
}

/* ---------------------------------------- a3 + a4: gate and top-K select */
/*
 * [SAS] Alg. 1 and the worked example: g = softmax(s) over the historical
 * blocks, top-K of the scores, the chosen blocks get the bias log g.
 * Selection order: higher score first, lower index on ties; the K chosen
 * indices are emitted ascending, the remaining slots hold -1.
 * Returns K_eff.  gap = s_(K) - s_(K+1) (INFINITY when nothing is left out).
 * logg (nullable) receives s_c - LSE(s) for the chosen blocks, 0 in pads;
 * lse_out (nullable) receives LSE over all candidates.
 */
int orc_select_from_scores(const double *s, int64_t ncand, int K, int gate,
                           int32_t *idx, double *logg, double *gap,
                           double *lse_out)
{
    int keff = (int)((int64_t)K < ncand ? K : ncand);
    char *taken = (char *)calloc((size_t)(ncand > 0 ? ncand : 1), 1);
    int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    double kth = INFINITY;
    for (int t = 0; t < keff; ++t) {
        int64_t best = -1;
        for (int64_t c = 0; c < ncand; ++c) {
            if (taken[c])
                continue;
            if (best < 0 || s[c] > s[best])   /* strict: lower index wins ties */
                best = c;
        }
        taken[best] = 1;
        chosen[t] = (int32_t)best;
        kth = s[best];
    }
    /* best score left out */
    double rest = -INFINITY;
    for (int64_t c = 0; c < ncand; ++c)
        if (!taken[c] && s[c] > rest)
            rest = s[c];
    if (gap)
        *gap = (keff < ncand) ? (kth - rest) : INFINITY;

    /* ascending order of the chosen indices (insertion sort) */
    for (int a = 1; a < keff; ++a) {
        int32_t x = chosen[a];
        int bpos = a - 1;
        while (bpos >= 0 && chosen[bpos] > x) {
            chosen[bpos + 1] = chosen[bpos];
            --bpos;
        }
        chosen[bpos + 1] = x;
    }

    /* log-sum-exp over every candidate (max-shifted) */
    double lse = -INFINITY;
    if (ncand > 0) {
        double m = -INFINITY;
        for (int64_t c = 0; c < ncand; ++c)
            if (s[c] > m)
                m = s[c];
        double acc = 0.0;
        for (int64_t c = 0; c < ncand; ++c)
            acc += exp(s[c] - m);
        lse = m + log(acc);
    }
    if (lse_out)
        *lse_out = lse;

    for (int t = 0; t < K; ++t) {
        if (t < keff) {
            idx[t] = chosen[t];
            if (logg)
                logg[t] = gate ? (s[chosen[t]] - lse) : 0.0;
        } else {
            idx[t] = -1;
            if (logg)
                logg[t] = 0.0;
        }
    }
    free(taken);
    free(chosen);
    return keff;
}

/* ----------------------------------------------------------- a2: scores */
/*
 * Scores of every candidate of one query row, for one selection head hs.
 * [SAS] §3 Eq. 3: s_c = R(q, summary_c); here R is q_hat . ktilde_c / sqrt(d)
 * with q_hat = q_h (share_group=0) or the mean over the G query heads of kv
 * head hs (share_group=1), and ktilde_c = kbar_c, or W kbar_c when a
 * projection W [d, d] (row-major, ktilde_e = sum_f W[e][f] kbar_f) is given.
 * [FS] adds lambda_h a_c erf((i - p_c) / (2 sigma_h)).
 */
static void orc_scores_row(const void *q, int qdtype, int Hq, int Hkv, int nq, int d,
                           int bidx, int hs, int64_t row, int64_t pos,
                           const void *kbar, int kdtype, const float *max_norm,
                           const float *centre, int64_t Ccap, int share_group,
                           const float *proj_w, const float *erf_lambda,
                           const float *erf_sigma, int64_t ncand, double *s_out)
{
    double *qh = (double *)calloc((size_t)d, sizeof(double));
    int G = Hq / Hkv;
    int kvh = share_group ? hs : hs / G;
    if (share_group) {
        for (int g = 0; g < G; ++g) {
            int h = hs * G + g;
            for (int e = 0; e < d; ++e)
                qh[e] += orc_load(q, qdtype, (((int64_t)bidx * Hq + h) * nq + row) * d + e);
        }
        for (int e = 0; e < d; ++e)
            qh[e] /= (double)G;
    } else {
        for (int e = 0; e < d; ++e)
            qh[e] = orc_load(q, qdtype, (((int64_t)bidx * Hq + hs) * nq + row) * d + e);
    }
    double scale = 1.0 / sqrt((double)d);
    double *kt = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t c = 0; c < ncand; ++c) {
        const int64_t kb = (((int64_t)bidx * Hkv + kvh) * Ccap + c) * d;
        if (proj_w) {
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int f = 0; f < d; ++f)
                    acc += (double)proj_w[e * d + f] * orc_load(kbar, kdtype, kb + f);
                kt[e] = acc;
            }
        } else {
            for (int e = 0; e < d; ++e)
                kt[e] = orc_load(kbar, kdtype, kb + e);
        }
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qh[e] * kt[e];
        double sc = dot * scale;
        if (erf_lambda) {
            double lam = (double)erf_lambda[hs];
            double sig = (double)erf_sigma[hs];
            double a = (double)max_norm[((int64_t)bidx * Hkv + kvh) * Ccap + c];
            double p = (double)centre[c];
            sc += lam * a * erf(((double)pos - p) / (2.0 * sig));
        }
        s_out[c] = sc;
    }
    free(kt);
    free(qh);
}

/*
 * a2-a4 for a set of rows.  rows (nullable) lists row numbers r in [0, nq)
 * to evaluate (all rows when NULL, nrows ignored); outputs are written at
 * the full-size positions [B, Hsel, nq, K] / [B, Hsel, nq].
 * Hsel = Hkv when share_group else Hq.
 */
void orc_score_select(const void *q, int qdtype, int B, int Hq, int Hkv, int nq,
                      int d, int64_t q_pos0, const void *kbar, int kdtype,
                      const float *max_norm, const float *centre, int64_t Ccap,
                      int b, int prefix_mode, int qblock, int share_group,
                      const float *proj_w, const float *erf_lambda,
                      const float *erf_sigma, int K, int gate,
                      const int64_t *rows, int64_t nrows,
                      int32_t *idx, double *logg, int32_t *k_eff, double *gap,
                      double *lse_cand)
{
    int Hsel = share_group ? Hkv : Hq;
    int64_t nr = rows ? nrows : nq;
    int64_t total = (int64_t)B * Hsel * nr;
    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < total; ++w) {
        int64_t rr = w % nr;
        int hs = (int)((w / nr) % Hsel);
        int bidx = (int)(w / nr / Hsel);
        int64_t row = rows ? rows[rr] : rr;
        int64_t pos = q_pos0 + row;
        int64_t ncand = orc_num_candidates(pos, b, prefix_mode, qblock);
        double *s = (double *)malloc(sizeof(double) * (size_t)(ncand > 0 ? ncand : 1));
        orc_scores_row(q, qdtype, Hq, Hkv, nq, d, bidx, hs, row, pos, kbar, kdtype,
                       max_norm, centre, Ccap, share_group, proj_w, erf_lambda,
                       erf_sigma, ncand, s);
        int64_t o = ((int64_t)bidx * Hsel + hs) * nq + row;
        double lse = 0.0, gp = 0.0;
        int ke = orc_select_from_scores(s, ncand, K, gate, idx + o * K,
                                        logg ? logg + o * K : NULL, &gp, &lse);
        if (k_eff)
            k_eff[o] = ke;
        if (gap)
            gap[o] = gp;
        if (lse_cand)
            lse_cand[o] = lse;
        free(s);
    }
}

/* Full score vector of one row (for tests that enumerate subsets). */
void orc_scores_one_row(const void *q, int qdtype, int B, int Hq, int Hkv, int nq,
                        int d, int64_t q_pos0, const void *kbar, int kdtype,
                        const float *max_norm, const float *centre, int64_t Ccap,
                        int b, int prefix_mode, int qblock, int share_group,
                        const float *proj_w, const float *erf_lambda,
                        const float *erf_sigma, int bidx, int hs, int64_t row,
                        double *s_out)
{
    (void)B;
    int64_t pos = q_pos0 + row;
    int64_t ncand = orc_num_candidates(pos, b, prefix_mode, qblock);
    orc_scores_row(q, qdtype, Hq, Hkv, nq, d, bidx, hs, row, pos, kbar, kdtype,
                   max_norm, centre, Ccap, share_group, proj_w, erf_lambda,
                   erf_sigma, ncand, s_out);
}

/* ------------------------------------------------ a5/a6: attention keys */
/*
 * Key set of query row at absolute position i for query head h.
 * Branch "L" (long / sparse):
 *   local == 0: the current block {j : floor(j/b) = floor(i/b), j <= i}
 *               with bias 0 ([SAS] §4.1: B0 always kept, gate 1), plus
 *   every selected unit c that is a valid candidate of i, whole (b tokens),
 *   with bias logg (0 when logg is NULL) ([SAS] §4.3 Eq. 9; [FS] routed cells).
 * Branch "S" (window): {j : i - w < j <= i} ([FS] sliding-window branch).
 * Builds arrays of key positions and biases; returns the count.
 */
static int64_t orc_branch_L_keys(int64_t i, int b, int local, int prefix_mode,
                                 int qblock, const int32_t *sel, const double *lg,
                                 int K, int64_t *keys, double *bias, int *slot)
{
    int64_t n = 0;
    if (local == 0) {
        int64_t c0 = i / b;
        for (int64_t j = c0 * b; j <= i; ++j) {
            keys[n] = j;
            bias[n] = 0.0;
            slot[n] = -1;
            ++n;
        }
    }
    int64_t ncand = orc_num_candidates(i, b, prefix_mode, qblock);
    for (int t = 0; t < K; ++t) {
        int32_t c = sel[t];
        if (c < 0 || (int64_t)c >= ncand)
            continue;                      /* only candidate units are read */
        for (int64_t j = (int64_t)c * b; j < (int64_t)(c + 1) * b; ++j) {
            keys[n] = j;
            bias[n] = lg ? lg[t] : 0.0;
            slot[n] = t;
            ++n;
        }
    }
    return n;
}

/* softmax attention of one row over an explicit key list (fp64) */
static void orc_softmax_attend(const void *q, const void *k, const void *v, int dtype,
                               int64_t qoff, int64_t kvbase, int d,
                               const int64_t *keys, const double *bias, int64_t nk,
                               double *z, double *o, double *lse)
{
    double scale = 1.0 / sqrt((double)d);
    for (int e = 0; e < d; ++e)
        o[e] = 0.0;
    if (nk == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < nk; ++t) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += orc_load(q, dtype, qoff + e) * orc_load(k, dtype, kvbase + keys[t] * d + e);
        z[t] = dot * scale + bias[t];
        if (z[t] > m)
            m = z[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nk; ++t)
        l += exp(z[t] - m);
    for (int64_t t = 0; t < nk; ++t) {
        double p = exp(z[t] - m) / l;
        for (int e = 0; e < d; ++e)
            o[e] += p * orc_load(v, dtype, kvbase + keys[t] * d + e);
    }
    *lse = m + log(l);
}

/*
 * Forward attention for a set of rows.
 *   local: 0 = current block kept, 1 = none.
 *   window > 0 with alpha != NULL: o = alpha_h o_L + (1 - alpha_h) o_S.
 *   idx/logg are [B, Hsel, nq, K]; logg may be NULL (no bias).
 *   Outputs o [B, Hq, nq, d] and lse [B, Hq, nq] (lse of branch L), fp64.
 */
void orc_attn_fwd(const void *q, const void *k, const void *v, int dtype,
                  int B, int Hq, int Hkv, int nq, int d, int64_t L, int64_t q_pos0,
                  int b, int prefix_mode, int qblock, const int32_t *idx,
                  const double *logg, int K, int share_group, int local, int window,
                  const float *alpha, const int64_t *rows, int64_t nrows,
                  double *o, double *lse)
{
    int G = Hq / Hkv;
    int Hsel = share_group ? Hkv : Hq;
    int64_t nr = rows ? nrows : nq;
    int64_t total = (int64_t)B * Hq * nr;
    int64_t maxk = (int64_t)b + (int64_t)K * b + (window > 0 ? window : 0) + 1;
    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < total; ++w) {
        int64_t rr = w % nr;
        int h = (int)((w / nr) % Hq);
        int bidx = (int)(w / nr / Hq);
        int64_t row = rows ? rows[rr] : rr;
        int64_t i = q_pos0 + row;
        int kvh = h / G;
        int hs = share_group ? kvh : h;
        int64_t so = (((int64_t)bidx * Hsel + hs) * nq + row) * K;
        int64_t qoff = (((int64_t)bidx * Hq + h) * nq + row) * d;
        int64_t kvbase = ((int64_t)bidx * Hkv + kvh) * L * d;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxk);
        double *bias = (double *)malloc(sizeof(double) * (size_t)maxk);
        double *z = (double *)malloc(sizeof(double) * (size_t)maxk);
        int *slot = (int *)malloc(sizeof(int) * (size_t)maxk);
        double *oL = (double *)malloc(sizeof(double) * (size_t)d);
        double *oS = (double *)malloc(sizeof(double) * (size_t)d);
        double lseL, lseS;
        int64_t nk = orc_branch_L_keys(i, b, local, prefix_mode, qblock, idx + so,
                                       logg ? logg + so : NULL, K, keys, bias, slot);
        orc_softmax_attend(q, k, v, dtype, qoff, kvbase, d, keys, bias, nk, z, oL, &lseL);
        int64_t oo = ((int64_t)bidx * Hq + h) * nq + row;
        if (window > 0 && alpha) {
            int64_t ns = 0;
            int64_t j0 = i - window + 1;
            if (j0 < 0)
                j0 = 0;
            for (int64_t j = j0; j <= i; ++j) {
                keys[ns] = j;
                bias[ns] = 0.0;
                ++ns;
            }
            orc_softmax_attend(q, k, v, dtype, qoff, kvbase, d, keys, bias, ns, z, oS, &lseS);
            double a = (double)alpha[h];
            for (int e = 0; e < d; ++e)
                o[oo * d + e] = a * oL[e] + (1.0 - a) * oS[e];
        } else {
            for (int e = 0; e < d; ++e)
                o[oo * d + e] = oL[e];
        }
        if (lse)
            lse[oo] = lseL;
        free(keys); free(bias); free(z); free(slot); free(oL); free(oS);
    }
}

/* ------------------------------------------------------ a7: backward */
/*
 * Backward of the SAS branch (local = current block, no window), fp64.
 *   z_ij = q_i.k_j/sqrt(d) + [j in B_m, m selected] log g_m
 *   p_ij = softmax_j(z_ij), o_i = sum_j p_ij v_j, D_i = do_i . o_i
 *   dS_ij = p_ij (do_i . v_j - D_i)
 *   dq_i = sum_j dS_ij k_j / sqrt(d); dk_j = sum_i dS_ij q_i / sqrt(d);
 *   dv_j = sum_i p_ij do_i
 *   dg_m = sum_{j in B_m} dS_ij / g_m  ([SAS] §4.2.2 Eq. 5, inner gate:
 *          p~_j/g_m do.(v_j - o) summed over the block = dS summed / g_m),
 *   summed over the G query heads when the gate is shared by a kv head.
 * With logg NULL the gate is 1 and dg is the gradient at g = 1.
 * Pass 1 runs per row (dq, dg, saves lse and D); pass 2 per key block
 * (dk, dv) gathers every row that reads the block.
 * kv_slice >= 0 restricts the work to one (batch, kv head) pair given as
 * b*Hkv + kvh (outputs of other pairs are left untouched).
 */
void orc_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                  int dtype, int B, int Hq, int Hkv, int nq, int d, int64_t L,
                  int64_t q_pos0, int b, const int32_t *idx, const double *logg,
                  int K, int share_group, int64_t kv_slice,
                  double *dq, double *dk, double *dv, double *dg)
{
    int G = Hq / Hkv;
    int Hsel = share_group ? Hkv : Hq;
    double scale = 1.0 / sqrt((double)d);
    int64_t maxk = (int64_t)b + (int64_t)K * b + 1;
    double *lse_all = (double *)malloc(sizeof(double) * (size_t)B * Hq * nq);
    double *D_all = (double *)malloc(sizeof(double) * (size_t)B * Hq * nq);
    /* per (b, q head, row, slot) block sums of dS, combined over heads below */
    double *dgh = (double *)calloc((size_t)B * Hq * nq * K, sizeof(double));

    int64_t total = (int64_t)B * Hq * nq;
    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < total; ++w) {
        int64_t row = w % nq;
        int h = (int)((w / nq) % Hq);
        int bidx = (int)(w / nq / Hq);
        int kvh = h / G;
        if (kv_slice >= 0 && (int64_t)bidx * Hkv + kvh != kv_slice)
            continue;
        int hs = share_group ? kvh : h;
        int64_t i = q_pos0 + row;
        int64_t so = (((int64_t)bidx * Hsel + hs) * nq + row) * K;
        int64_t qoff = (((int64_t)bidx * Hq + h) * nq + row) * d;
        int64_t kvbase = ((int64_t)bidx * Hkv + kvh) * L * d;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxk);
        double *bias = (double *)malloc(sizeof(double) * (size_t)maxk);
        double *z = (double *)malloc(sizeof(double) * (size_t)maxk);
        int *slot = (int *)malloc(sizeof(int) * (size_t)maxk);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double lse;
        int64_t nk = orc_branch_L_keys(i, b, 0, 0, 1, idx + so, logg ? logg + so : NULL,
                                       K, keys, bias, slot);
        orc_softmax_attend(q, k, v, dtype, qoff, kvbase, d, keys, bias, nk, z, o, &lse);
        double D = 0.0;
        for (int e = 0; e < d; ++e)
            D += orc_load(dout, dtype, qoff + e) * o[e];
        lse_all[w] = lse;
        D_all[w] = D;
        for (int e = 0; e < d; ++e)
            dq[qoff + e] = 0.0;
        for (int64_t t = 0; t < nk; ++t) {
            double p = exp(z[t] - lse);
            double dp = 0.0;
            for (int e = 0; e < d; ++e)
                dp += orc_load(dout, dtype, qoff + e) * orc_load(v, dtype, kvbase + keys[t] * d + e);
            double ds = p * (dp - D);
            for (int e = 0; e < d; ++e)
                dq[qoff + e] += ds * orc_load(k, dtype, kvbase + keys[t] * d + e) * scale;
            if (slot[t] >= 0)
                dgh[w * K + slot[t]] += ds;
        }
        free(keys); free(bias); free(z); free(slot); free(o);
    }

    /* dg: divide by g_m and sum over the heads that share the selection */
    int64_t nsel = (int64_t)B * Hsel * nq;
#pragma omp parallel for schedule(static)
    for (w = 0; w < nsel; ++w) {
        int64_t row = w % nq;
        int hs = (int)((w / nq) % Hsel);
        int bidx = (int)(w / nq / Hsel);
        int kvh = share_group ? hs : hs / G;
        if (kv_slice >= 0 && (int64_t)bidx * Hkv + kvh != kv_slice)
            continue;
        for (int t = 0; t < K; ++t) {
            double acc = 0.0;
            if (idx[w * K + t] >= 0) {
                double g = logg ? exp(logg[w * K + t]) : 1.0;
                int h0 = share_group ? hs * G : hs;
                int h1 = share_group ? hs * G + G : hs + 1;
                for (int h = h0; h < h1; ++h)
                    acc += dgh[(((int64_t)bidx * Hq + h) * nq + row) * K + t] / g;
            }
            dg[w * K + t] = acc;
        }
    }

    /* pass 2: dk, dv per (batch, kv head, key block) */
    int64_t nblk = (L + b - 1) / b;
    int64_t tot2 = (int64_t)B * Hkv * nblk;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < tot2; ++w) {
        int64_t c = w % nblk;
        int kvh = (int)((w / nblk) % Hkv);
        int bidx = (int)(w / nblk / Hkv);
        if (kv_slice >= 0 && (int64_t)bidx * Hkv + kvh != kv_slice)
            continue;
        int64_t kvbase = ((int64_t)bidx * Hkv + kvh) * L * d;
        int64_t j0 = c * b, j1 = (c + 1) * b < L ? (c + 1) * b : L;
        for (int64_t j = j0; j < j1; ++j)
            for (int e = 0; e < d; ++e) {
                dk[kvbase + j * d + e] = 0.0;
                dv[kvbase + j * d + e] = 0.0;
            }
        for (int g = 0; g < G; ++g) {
            int h = kvh * G + g;
            int hs = share_group ? kvh : h;
            for (int64_t row = 0; row < nq; ++row) {
                int64_t i = q_pos0 + row;
                int64_t so = (((int64_t)bidx * Hsel + hs) * nq + row) * K;
                double bias_c;
                int reads = 0;
                if (i / b == c) {
                    reads = 1;                 /* current block, causal */
                    bias_c = 0.0;
                } else {
                    int64_t ncand = i / b;
                    for (int t = 0; t < K; ++t) {
                        if (idx[so + t] == (int32_t)c && c < ncand) {
                            reads = 2;
                            bias_c = logg ? logg[so + t] : 0.0;
                            break;
                        }
                    }
                }
                if (!reads)
                    continue;
                int64_t ww = ((int64_t)bidx * Hq + h) * nq + row;
                int64_t qoff = ww * d;
                for (int64_t j = j0; j < j1; ++j) {
                    if (reads == 1 && j > i)
                        continue;
                    double dot = 0.0, dp = 0.0;
                    for (int e = 0; e < d; ++e) {
                        dot += orc_load(q, dtype, qoff + e) * orc_load(k, dtype, kvbase + j * d + e);
                        dp += orc_load(dout, dtype, qoff + e) * orc_load(v, dtype, kvbase + j * d + e);
                    }
                    double p = exp(dot * scale + bias_c - lse_all[ww]);
                    double ds = p * (dp - D_all[ww]);
                    for (int e = 0; e < d; ++e) {
                        dk[kvbase + j * d + e] += ds * orc_load(q, dtype, qoff + e) * scale;
                        dv[kvbase + j * d + e] += p * orc_load(dout, dtype, qoff + e);
                    }
                }
            }
        }
    }
    free(lse_all);
    free(D_all);
    free(dgh);
}

/* ------------------------------------------- next: selector-side backward */
/*
 * Gradient of the gate into the selector's inputs ([SAS] "How it works",
 * step 5: the loss flows o -> g -> s -> selector, §4.3 Eq. 9; the gate is
 * log g_m = s_m - LSE(s) over every candidate of the row, §4.2.2).  With the
 * selection S of a row fixed and dg_m the gradient of the loss with respect
 * to g_m (what orc_attn_bwd returns), let dl_m = g_m dg_m (the gradient with
 * respect to log g_m) and p = softmax(s) over the candidates (so g_m = p_m).
 * Then
 *   ds_c = [c in S] dl_c - p_c sum_{m in S} dl_m
 *   dq_hat = sum_c ds_c ktilde_c / sqrt(d),   dktilde_c += ds_c q_hat / sqrt(d),
 * and each of the G query heads averaged into q_hat receives dq_hat / G.
 * ktilde = kbar, or W kbar with the learned projection ("SAS" review, the
 * 128 -> 128 projection of the mean keys); then dkbar_c = W^T dktilde_c and
 * dW = sum over (batch, kv head, summary) of dktilde_c kbar_c^T.
 * Scores are recomputed here in fp64 (orc_scores_row, no erf term); idx is
 * the forward's selection, dg is [B, Hsel, nq, K] (padded slots ignored).
 * Outputs (fp64, written): dq [B, Hq, nq, d], dkbar [B, Hkv, Ccap, d], and
 * dW [d, d] when proj_w is given (summed over the (batch, kv head) tasks in
 * task order).
 */
void orc_select_bwd(const void *q, int qdtype, int B, int Hq, int Hkv, int nq, int d,
                    int64_t q_pos0, const void *kbar, int kdtype, int64_t Ccap, int b,
                    int share_group, int K, const float *proj_w, const int32_t *idx,
                    const double *dg, double *dq, double *dkbar, double *dW)
{
    const int G = Hq / Hkv;
    const int Hsel = share_group ? Hkv : Hq;
    const double scale = 1.0 / sqrt((double)d);
    const int ntask = B * Hkv;
    memset(dq, 0, sizeof(double) * (size_t)B * Hq * nq * d);
    memset(dkbar, 0, sizeof(double) * (size_t)B * Hkv * Ccap * d);
    /* per-task partial dW, summed in task order below */
    double *dw_part = proj_w ? (double *)calloc((size_t)ntask * d * d, sizeof(double)) : NULL;
    /* one task per (batch, kv head): it owns dkbar of that head */
#pragma omp parallel for schedule(dynamic, 1) num_threads(orc_num_threads())
    for (int t = 0; t < ntask; ++t) {
        const int bidx = t / Hkv, kvh = t % Hkv;
        const int64_t kb0 = ((int64_t)bidx * Hkv + kvh) * Ccap;
        double *s = (double *)malloc(sizeof(double) * (size_t)(Ccap > 0 ? Ccap : 1));
        double *ds = (double *)malloc(sizeof(double) * (size_t)(Ccap > 0 ? Ccap : 1));
        double *qh = (double *)malloc(sizeof(double) * (size_t)d);
        /* the summaries as the scores see them, and their gradient */
        double *kt = (double *)malloc(sizeof(double) * (size_t)(Ccap > 0 ? Ccap : 1) * d);
        double *dkt = (double *)calloc((size_t)(Ccap > 0 ? Ccap : 1) * d, sizeof(double));
        for (int64_t c = 0; c < Ccap; ++c)
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                if (proj_w) {
                    for (int f = 0; f < d; ++f)
                        acc += (double)proj_w[e * d + f] * orc_load(kbar, kdtype, (kb0 + c) * d + f);
                } else {
                    acc = orc_load(kbar, kdtype, (kb0 + c) * d + e);
                }
                kt[c * d + e] = acc;
            }
        const int hs0 = share_group ? kvh : kvh * G;
        const int hs1 = share_group ? kvh + 1 : kvh * G + G;
        for (int hs = hs0; hs < hs1; ++hs) {
            for (int64_t row = 0; row < nq; ++row) {
                const int64_t pos = q_pos0 + row;
                int64_t ncand = orc_num_candidates(pos, b, 0, 128);
                if (ncand > Ccap)
                    ncand = Ccap;
                if (ncand <= 0)
                    continue;
                orc_scores_row(q, qdtype, Hq, Hkv, nq, d, bidx, hs, row, pos, kbar, kdtype, NULL,
                               NULL, Ccap, share_group, proj_w, NULL, NULL, ncand, s);
                double mx = s[0];
                for (int64_t c = 1; c < ncand; ++c)
                    if (s[c] > mx)
                        mx = s[c];
                double sum = 0.0;
                for (int64_t c = 0; c < ncand; ++c)
                    sum += exp(s[c] - mx);
                const double lse = mx + log(sum);
                const int64_t so = (((int64_t)bidx * Hsel + hs) * nq + row) * K;
                double dl_sum = 0.0;
                for (int64_t c = 0; c < ncand; ++c)
                    ds[c] = 0.0;
                for (int k = 0; k < K; ++k) {
                    const int32_t c = idx[so + k];
                    if (c < 0 || c >= ncand)
                        continue;
                    const double dl = exp(s[c] - lse) * dg[so + k];
                    ds[c] += dl;
                    dl_sum += dl;
                }
                for (int64_t c = 0; c < ncand; ++c)
                    ds[c] -= exp(s[c] - lse) * dl_sum;
                /* q_hat as the scores saw it */
                for (int e = 0; e < d; ++e)
                    qh[e] = 0.0;
                if (share_group) {
                    for (int g = 0; g < G; ++g)
                        for (int e = 0; e < d; ++e)
                            qh[e] += orc_load(q, qdtype, (((int64_t)bidx * Hq + hs * G + g) * nq + row) * d + e);
                    for (int e = 0; e < d; ++e)
                        qh[e] /= (double)G;
                } else {
                    for (int e = 0; e < d; ++e)
                        qh[e] = orc_load(q, qdtype, (((int64_t)bidx * Hq + hs) * nq + row) * d + e);
                }
                for (int e = 0; e < d; ++e) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < ncand; ++c)
                        acc += ds[c] * kt[c * d + e];
                    acc *= scale;
                    if (share_group) {
                        for (int g = 0; g < G; ++g)
                            dq[(((int64_t)bidx * Hq + hs * G + g) * nq + row) * d + e] += acc / (double)G;
                    } else {
                        dq[(((int64_t)bidx * Hq + hs) * nq + row) * d + e] += acc;
                    }
                }
                for (int64_t c = 0; c < ncand; ++c)
                    for (int e = 0; e < d; ++e)
                        dkt[c * d + e] += ds[c] * qh[e] * scale;
            }
        }
        for (int64_t c = 0; c < Ccap; ++c) {
            if (proj_w) {
                for (int f = 0; f < d; ++f) {
                    double acc = 0.0;
                    for (int e = 0; e < d; ++e)
                        acc += (double)proj_w[e * d + f] * dkt[c * d + e];
                    dkbar[(kb0 + c) * d + f] = acc;
                }
                for (int e = 0; e < d; ++e)
                    for (int f = 0; f < d; ++f)
                        dw_part[((size_t)t * d + e) * d + f] +=
                            dkt[c * d + e] * orc_load(kbar, kdtype, (kb0 + c) * d + f);
            } else {
                for (int e = 0; e < d; ++e)
                    dkbar[(kb0 + c) * d + e] = dkt[c * d + e];
            }
        }
        free(s);
        free(ds);
        free(qh);
        free(kt);
        free(dkt);
    }
    if (proj_w) {
        memset(dW, 0, sizeof(double) * (size_t)d * d);
        for (int t = 0; t < ntask; ++t)
            for (int e = 0; e < d * d; ++e)
                dW[e] += dw_part[(size_t)t * d * d + e];
        free(dw_part);
    }
}

/* ------------------------------------------- next: fixed-state retention */
/*
 * FS-L retention ("FreeSolo" review, the two variants: before any query
 * arrives, each head keeps only its W most recent cells and the P cells of
 * largest max key norm, and every query picks its top K inside that set).
 * Reading taken: of the ncand prefix cells 0 .. ncand-1, the W most recent
 * (ncand-W .. ncand-1) plus the P older cells of largest max_norm (lower index
 * first on equal norms), so min(ncand, W + P) cells are kept.  Per (batch, kv
 * head): cells [B, Hkv, W + P] ascending, -1 padded; count [B, Hkv].
 */
void orc_retain_cells(const float *max_norm, int B, int Hkv, int64_t Ccap, int64_t ncand, int W,
                      int P, int32_t *cells, int32_t *count)
{
    const int cap = W + P;
    const int64_t n_old = ncand > W ? ncand - W : 0;
    const int kp = (int)((int64_t)P < n_old ? P : n_old);
    char *taken = (char *)malloc((size_t)(n_old > 0 ? n_old : 1));
    int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap > 0 ? cap : 1));
    for (int t = 0; t < B * Hkv; ++t) {
        const float *a = max_norm + (int64_t)t * Ccap;
        memset(taken, 0, (size_t)(n_old > 0 ? n_old : 1));
        for (int j = 0; j < kp; ++j) {
            int64_t best = -1;
            for (int64_t c = 0; c < n_old; ++c) {
                if (taken[c])
                    continue;
                if (best < 0 || a[c] > a[best])   /* strict: lower index wins ties */
                    best = c;
            }
            taken[best] = 1;
            chosen[j] = (int32_t)best;
        }
        /* ascending (insertion sort), then the recent cells */
        for (int x = 1; x < kp; ++x) {
            int32_t v = chosen[x];
            int y = x - 1;
            while (y >= 0 && chosen[y] > v) {
                chosen[y + 1] = chosen[y];
                --y;
            }
            chosen[y + 1] = v;
        }
        int n = kp;
        for (int64_t c = n_old; c < ncand; ++c)
            chosen[n++] = (int32_t)c;
        for (int x = 0; x < cap; ++x)
            cells[(int64_t)t * cap + x] = x < n ? chosen[x] : -1;
        count[t] = n;
    }
    free(taken);
    free(chosen);
}

/*
 * Per-query selection inside a kept set: the row's scores (orc_scores_row) on
 * the listed cells that are candidates of the row, then the same gate and
 * top-K as orc_score_select over just those cells (the LSE runs over the kept
 * candidates), mapped back to cell ids (ascending, -1 padded).  cells / count
 * are per (batch, kv head) as orc_retain_cells writes them; a selection head
 * reads the list of its kv head.
 */
void orc_score_select_subset(const void *q, int qdtype, int B, int Hq, int Hkv, int nq, int d,
                             int64_t q_pos0, const void *kbar, int kdtype, const float *max_norm,
                             const float *centre, int64_t Ccap, int b, int prefix_mode, int qblock,
                             int share_group, const float *erf_lambda, const float *erf_sigma,
                             const int32_t *cells, const int32_t *count, int cap, int K, int gate,
                             int32_t *idx, double *logg, int32_t *k_eff, double *gap)
{
    const int Hsel = share_group ? Hkv : Hq;
    const int G = Hq / Hkv;
    const int64_t total = (int64_t)B * Hsel * nq;
    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < total; ++w) {
        const int64_t row = w % nq;
        const int hs = (int)((w / nq) % Hsel);
        const int bidx = (int)(w / nq / Hsel);
        const int kvh = share_group ? hs : hs / G;
        const int64_t pos = q_pos0 + row;
        const int64_t ncand = orc_num_candidates(pos, b, prefix_mode, qblock);
        double *s = (double *)malloc(sizeof(double) * (size_t)(ncand > 0 ? ncand : 1));
        double *sub = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap > 0 ? cap : 1));
        int32_t *pick = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
        orc_scores_row(q, qdtype, Hq, Hkv, nq, d, bidx, hs, row, pos, kbar, kdtype, max_norm, centre,
                       Ccap, share_group, NULL, erf_lambda, erf_sigma, ncand, s);
        const int32_t *lst = cells + ((int64_t)bidx * Hkv + kvh) * cap;
        const int nl = count[(int64_t)bidx * Hkv + kvh];
        int n = 0;
        for (int x = 0; x < nl; ++x)
            if (lst[x] >= 0 && lst[x] < ncand) {
                sub[n] = s[lst[x]];
                ids[n] = lst[x];
                ++n;
            }
        const int64_t o = ((int64_t)bidx * Hsel + hs) * nq + row;
        double gp = 0.0, lse = 0.0;
        const int ke = orc_select_from_scores(sub, n, K, gate, pick, logg ? logg + o * K : NULL, &gp, &lse);
        for (int k = 0; k < K; ++k)
            idx[o * K + k] = k < ke ? ids[pick[k]] : -1;
        if (k_eff)
            k_eff[o] = ke;
        if (gap)
            gap[o] = gp;
        free(s);
        free(sub);
        free(ids);
        free(pick);
    }
}

/* ------------------------------------------- next: hierarchical selection */
/*
 * FS-B forests ("FreeSolo" review, the two variants: no cell is dropped;
 * each head builds one forest over the whole prefix and one over the cells
 * whose max key norm is at or above the median; nodes hold a mean key, a
 * radius, a max norm and a min position; a beam search of width W_b per
 * level descends them, the node score U upper-bounding the scores of the
 * cells below; the cells reached are re-ranked by logsumexp over their token
 * keys and the top K are read).  Readings taken:
 *   - a forest over m member cells (ascending cell order) is a tree of fanout
 *     F: node j of level 1 groups members [jF, jF + F), node j of level l
 *     groups nodes [jF, jF + F) of level l - 1; levels are added until a
 *     level has at most F nodes (none when m <= F);
 *   - median: the ceil(n/2)-th largest max norm of the n prefix cells; the
 *     high-norm forest holds every cell whose norm is >= it;
 *   - node fields, rounded to fp32 (nearest): mu = (sum of the subtree's cell
 *     mean keys, summed child by child in fp64) / cells; r = max over the
 *     subtree's cells of ||kbar_c - mu|| (fp64); a = max a_c; p = min p_c;
 *   - U_v = q_hat . mu / sqrt(d) + ||q_hat|| r / sqrt(d)
 *           + lambda a erf((i - p) / (2 sigma)), an upper bound of every
 *     cell score below v for lambda >= 0 (Cauchy-Schwarz, erf increasing);
 *     a cell's own score (r = 0) is the FreeSolo cell score;
 *   - beam: the frontier starts as the top level; each step keeps the W_b
 *     children of the frontier with the largest score (lower index first on
 *     ties) until the frontier holds cells: the forest's reached cells;
 *   - re-rank: the union of both forests' reached cells, scored by
 *     logsumexp over the cell's tokens j of q_hat . k_j / sqrt(d); top K
 *     (lower index first on ties), emitted ascending.
 */
static int64_t orc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* internal nodes of a forest over m members, and the first index of each
 * level (lvl_off[0] = 0 for level 1); returns the number of levels */
int orc_forest_levels(int64_t m, int F, int64_t *lvl_n, int64_t *lvl_off, int maxlev)
{
    int nl = 0;
    int64_t cur = m, off = 0;
    while (cur > F && nl < maxlev) {
        cur = orc_ceil_div(cur, F);
        lvl_n[nl] = cur;
        lvl_off[nl] = off;
        off += cur;
        ++nl;
    }
    return nl;
}

int64_t orc_forest_nodes(int64_t m, int F)
{
    int64_t ln[32], lo[32];
    const int nl = orc_forest_levels(m, F, ln, lo, 32);
    return nl ? lo[nl - 1] + ln[nl - 1] : 0;
}

/* members [B, Hkv, 2, n] (-1 padded), nmem [B, Hkv, 2]; node fields
 * [B, Hkv, 2, NN(, d)] with NN = orc_forest_nodes(n, F) */
void orc_forest_build(const void *kbar, int kdtype, const float *max_norm, const float *centre, int B,
                      int Hkv, int d, int64_t Ccap, int64_t n, int F, int32_t *members, int32_t *nmem,
                      float *mu, float *rad, float *amax, float *pmin)
{
    const int64_t NN = orc_forest_nodes(n, F);
    for (int t = 0; t < B * Hkv; ++t) {
        const float *a = max_norm + (int64_t)t * Ccap;
        /* median: ceil(n/2)-th largest norm */
        float thr = 0.f;
        if (n > 0) {
            float *srt = (float *)malloc(sizeof(float) * (size_t)n);
            for (int64_t c = 0; c < n; ++c)
                srt[c] = a[c];
            /* selection sort of the largest ceil(n/2) (plain, small n) */
            const int64_t kk = (n + 1) / 2;
            for (int64_t x = 0; x < kk; ++x) {
                int64_t best = x;
                for (int64_t y = x + 1; y < n; ++y)
                    if (srt[y] > srt[best])
                        best = y;
                float tmp = srt[x];
                srt[x] = srt[best];
                srt[best] = tmp;
            }
            thr = srt[kk - 1];
            free(srt);
        }
        for (int f = 0; f < 2; ++f) {
            int32_t *mem = members + ((int64_t)t * 2 + f) * n;
            int64_t m = 0;
            for (int64_t c = 0; c < n; ++c)
                if (f == 0 || a[c] >= thr)
                    mem[m++] = (int32_t)c;
            for (int64_t x = m; x < n; ++x)
                mem[x] = -1;
            nmem[t * 2 + f] = (int32_t)m;
            int64_t ln[32], lo[32];
            const int nl = orc_forest_levels(m, F, ln, lo, 32);
            const int64_t fb = ((int64_t)t * 2 + f) * NN;
            const int64_t NNf = nl ? lo[nl - 1] + ln[nl - 1] : 0;
            double *sums = (double *)calloc((size_t)(NNf > 0 ? NNf : 1) * d, sizeof(double));
            int64_t *cnt = (int64_t *)calloc((size_t)(NNf > 0 ? NNf : 1), sizeof(int64_t));
            for (int l = 0; l < nl; ++l) {
                for (int64_t j = 0; j < ln[l]; ++j) {
                    const int64_t node = lo[l] + j;
                    double *sm = sums + node * d;
                    float am = 0.f, pm = INFINITY;
                    if (l == 0) {
                        for (int64_t x = j * F; x < (j + 1) * F && x < m; ++x) {
                            const int64_t c = mem[x];
                            for (int e = 0; e < d; ++e)
                                sm[e] += orc_load(kbar, kdtype, ((int64_t)t * Ccap + c) * d + e);
                            cnt[node] += 1;
                            if (a[c] > am)
                                am = a[c];
                            if (centre[c] < pm)
                                pm = centre[c];
                        }
                    } else {
                        const int64_t nprev = ln[l - 1];
                        for (int64_t x = j * F; x < (j + 1) * F && x < nprev; ++x) {
                            const int64_t ch = lo[l - 1] + x;
                            for (int e = 0; e < d; ++e)
                                sm[e] += sums[ch * d + e];
                            cnt[node] += cnt[ch];
                            if (amax[fb + ch] > am)
                                am = amax[fb + ch];
                            if (pmin[fb + ch] < pm)
                                pm = pmin[fb + ch];
                        }
                    }
                    for (int e = 0; e < d; ++e)
                        mu[(fb + node) * d + e] = (float)(sm[e] / (double)cnt[node]);
                    amax[fb + node] = am;
                    pmin[fb + node] = pm;
                }
            }
            /* radius: over the cells below each node */
            for (int l = 0; l < nl; ++l) {
                int64_t span = F;   /* members per node at this level */
                for (int x = 0; x < l; ++x)
                    span *= F;
                for (int64_t j = 0; j < ln[l]; ++j) {
                    const int64_t node = lo[l] + j;
                    double best = 0.0;
                    for (int64_t x = j * span; x < (j + 1) * span && x < m; ++x) {
                        const int64_t c = mem[x];
                        double ss = 0.0;
                        for (int e = 0; e < d; ++e) {
                            const double df = orc_load(kbar, kdtype, ((int64_t)t * Ccap + c) * d + e) -
                                              (double)mu[(fb + node) * d + e];
                            ss += df * df;
                        }
                        if (ss > best)
                            best = ss;
                    }
                    rad[fb + node] = (float)sqrt(best);
                }
            }
            for (int64_t x = NNf; x < NN; ++x) {   /* unused slots of the smaller forest */
                for (int e = 0; e < d; ++e)
                    mu[(fb + x) * d + e] = 0.f;
                rad[fb + x] = 0.f;
                amax[fb + x] = 0.f;
                pmin[fb + x] = 0.f;
            }
            free(sums);
            free(cnt);
        }
    }
}

/* U_v of one node for one query (q_hat, its norm, the row position) */
double orc_node_score(const double *qh, double qn, const float *mu, float rad, float amax, float pmin, int d,
                      double lam, double sig, double pos, int with_erf)
{
    double dot = 0.0;
    for (int e = 0; e < d; ++e)
        dot += qh[e] * (double)mu[e];
    const double isd = 1.0 / sqrt((double)d);
    double s = dot * isd + qn * (double)rad * isd;
    if (with_erf)
        s += lam * (double)amax * erf((pos - (double)pmin) / (2.0 * sig));
    return s;
}

/* top-w of s[0..cnt) by (score desc, position asc) into keep[]; returns the
 * number kept and the gap between the last kept and the best dropped score */
static int orc_top_w(const double *s, int cnt, int w, int *keep, double *gap)
{
    char *taken = (char *)calloc((size_t)(cnt > 0 ? cnt : 1), 1);
    const int kk = cnt < w ? cnt : w;
    double last = INFINITY;
    for (int t = 0; t < kk; ++t) {
        int best = -1;
        for (int x = 0; x < cnt; ++x)
            if (!taken[x] && (best < 0 || s[x] > s[best]))
                best = x;
        taken[best] = 1;
        keep[t] = best;
        last = s[best];
    }
    double rest = -INFINITY;
    for (int x = 0; x < cnt; ++x)
        if (!taken[x] && s[x] > rest)
            rest = s[x];
    if (gap && kk < cnt && last - rest < *gap)
        *gap = last - rest;
    free(taken);
    return kk;
}

void orc_forest_select(const void *q, int qdtype, int B, int Hq, int Hkv, int nq, int d, int64_t q_pos0,
                       const void *kbar, int kdtype, const float *max_norm, const float *centre,
                       int64_t Ccap, const void *k, int64_t L, int b, int share_group,
                       const float *erf_lambda, const float *erf_sigma, const int32_t *members,
                       const int32_t *nmem, const float *mu, const float *rad, const float *amax,
                       const float *pmin, int64_t n, int F, int Wb, int K, int32_t *idx, double *gap)
{
    const int Hsel = share_group ? Hkv : Hq;
    const int G = Hq / Hkv;
    const int64_t NN = orc_forest_nodes(n, F);
    const double isd = 1.0 / sqrt((double)d);
    const int64_t total = (int64_t)B * Hsel * nq;
    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < total; ++w) {
        const int64_t row = w % nq;
        const int hs = (int)((w / nq) % Hsel);
        const int bidx = (int)(w / nq / Hsel);
        const int kvh = share_group ? hs : hs / G;
        const int64_t t = (int64_t)bidx * Hkv + kvh;
        const double pos = (double)(q_pos0 + row);
        double *qh = (double *)calloc((size_t)d, sizeof(double));
        const int gq = share_group ? G : 1;
        const int h0 = share_group ? hs * G : hs;
        for (int g = 0; g < gq; ++g)
            for (int e = 0; e < d; ++e)
                qh[e] += orc_load(q, qdtype, (((int64_t)bidx * Hq + h0 + g) * nq + row) * d + e);
        double qn = 0.0;
        for (int e = 0; e < d; ++e) {
            qh[e] /= (double)gq;
            qn += qh[e] * qh[e];
        }
        qn = sqrt(qn);
        const double lam = erf_lambda ? (double)erf_lambda[hs] : 0.0;
        const double sig = erf_sigma ? (double)erf_sigma[hs] : 1.0;
        double g_min = INFINITY;
        int32_t reached[64];
        int nreach = 0;
        int64_t cid[256];
        double sc[256];
        int keep[256];
        for (int f = 0; f < 2; ++f) {
            const int32_t *mem = members + (t * 2 + f) * n;
            const int64_t m = nmem[t * 2 + f];
            const int64_t fb = (t * 2 + f) * NN;
            int64_t ln[32], lo[32];
            const int nl = orc_forest_levels(m, F, ln, lo, 32);
            /* frontier: ids at level `lev` (0 = member positions) */
            int64_t front[64];
            int nf = 0, lev = nl;
            const int64_t ntop = nl ? ln[nl - 1] : m;
            for (int64_t x = 0; x < ntop; ++x)
                front[nf++] = x;
            for (;;) {
                /* candidates: the frontier itself at the start of a level-0 forest,
                 * else the children of the frontier */
                int cnt = 0;
                const int child_lev = (lev == nl && nl == 0) ? 0 : lev - 1;
                if (lev == nl && nl == 0) {
                    for (int x = 0; x < nf; ++x)
                        cid[cnt++] = front[x];
                } else {
                    const int64_t nchild = child_lev == 0 ? m : ln[child_lev - 1];
                    for (int x = 0; x < nf; ++x)
                        for (int64_t y = front[x] * F; y < (front[x] + 1) * F && y < nchild; ++y)
                            cid[cnt++] = y;
                }
                for (int x = 0; x < cnt; ++x) {
                    double s;
                    if (child_lev == 0) {
                        const int64_t c = mem[cid[x]];
                        double dot = 0.0;
                        for (int e = 0; e < d; ++e)
                            dot += qh[e] * orc_load(kbar, kdtype, (t * Ccap + c) * d + e);
                        s = dot * isd;
                        if (erf_lambda)
                            s += lam * (double)max_norm[t * Ccap + c] * erf((pos - (double)centre[c]) / (2.0 * sig));
                    } else {
                        const int64_t node = fb + lo[child_lev - 1] + cid[x];
                        s = orc_node_score(qh, qn, mu + node * d, rad[node], amax[node], pmin[node], d, lam, sig,
                                           pos, erf_lambda != NULL);
                    }
                    sc[x] = s;
                }
                const int kk = orc_top_w(sc, cnt, Wb, keep, &g_min);
                /* keep the frontier in candidate order (ascending ids) */
                for (int x = 1; x < kk; ++x) {
                    int v = keep[x], y = x - 1;
                    while (y >= 0 && keep[y] > v) {
                        keep[y + 1] = keep[y];
                        --y;
                    }
                    keep[y + 1] = v;
                }
                nf = kk;
                for (int x = 0; x < kk; ++x)
                    front[x] = cid[keep[x]];
                if (child_lev == 0)
                    break;
                lev = child_lev;
            }
            for (int x = 0; x < nf; ++x) {
                const int32_t c = mem[front[x]];
                int dup = 0;
                for (int y = 0; y < nreach; ++y)
                    if (reached[y] == c)
                        dup = 1;
                if (!dup)
                    reached[nreach++] = c;
            }
        }
        /* re-rank the reached cells by logsumexp over their tokens */
        double *lse = (double *)malloc(sizeof(double) * 64);
        /* ascending cell order first, so that ties go to the lower cell */
        for (int x = 1; x < nreach; ++x) {
            int32_t v = reached[x];
            int y = x - 1;
            while (y >= 0 && reached[y] > v) {
                reached[y + 1] = reached[y];
                --y;
            }
            reached[y + 1] = v;
        }
        for (int x = 0; x < nreach; ++x) {
            const int64_t c = reached[x];
            double mx = -INFINITY, z[1024];
            for (int j = 0; j < b; ++j) {
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += qh[e] * orc_load(k, kdtype, (t * L + c * b + j) * d + e);
                z[j] = dot * isd;
                if (z[j] > mx)
                    mx = z[j];
            }
            double acc = 0.0;
            for (int j = 0; j < b; ++j)
                acc += exp(z[j] - mx);
            lse[x] = mx + log(acc);
        }
        int pick[64];
        const int kk = orc_top_w(lse, nreach, K, pick, &g_min);
        int32_t outc[64];
        for (int x = 0; x < kk; ++x)
            outc[x] = reached[pick[x]];
        for (int x = 1; x < kk; ++x) {
            int32_t v = outc[x];
            int y = x - 1;
            while (y >= 0 && outc[y] > v) {
                outc[y + 1] = outc[y];
                --y;
            }
            outc[y + 1] = v;
        }
        const int64_t o = ((int64_t)bidx * Hsel + hs) * nq + row;
        for (int x = 0; x < K; ++x)
            idx[o * K + x] = x < kk ? outc[x] : -1;
        if (gap)
            gap[o] = g_min;
        free(qh);
        free(lse);
    }
}

/*
 * [FS] "How it works", the FS-B variant: the re-rank score of a cell for one
 * row and selection head is the logsumexp over the cell's b token keys of
 * qhat.k_j / sqrt(d) (qhat = the group mean with share_group=1, no bias), for
 * every cell c < ncells.  The same quantity orc_forest_select ranks its
 * reached cells by, written out for all cells so that a different valid
 * re-rank (a cut whose margin is below 1e-6) can be checked.
 */
void orc_cell_token_lse(const void *q, int qdtype, int B, int Hq, int Hkv, int nq, int d, const void *k,
                        int kdtype, int64_t L, int b, int share_group, int bidx, int hs, int64_t row,
                        int64_t ncells, double *out)
{
    const int G = Hq / Hkv;
    const int kvh = share_group ? hs : hs / G;
    const int gq = share_group ? G : 1;
    const int h0 = share_group ? hs * G : hs;
    const int64_t t = (int64_t)bidx * Hkv + kvh;
    const double isd = 1.0 / sqrt((double)d);
    double *qh = (double *)calloc((size_t)d, sizeof(double));
    double *z = (double *)malloc(sizeof(double) * (size_t)b);
    (void)B;
    for (int g = 0; g < gq; ++g)
        for (int e = 0; e < d; ++e)
            qh[e] += orc_load(q, qdtype, (((int64_t)bidx * Hq + h0 + g) * nq + row) * d + e);
    for (int e = 0; e < d; ++e)
        qh[e] /= (double)gq;
    for (int64_t c = 0; c < ncells; ++c) {
        double mx = -INFINITY;
        for (int j = 0; j < b; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += qh[e] * orc_load(k, kdtype, (t * L + c * b + j) * d + e);
            z[j] = dot * isd;
            if (z[j] > mx)
                mx = z[j];
        }
        double acc = 0.0;
        for (int j = 0; j < b; ++j)
            acc += exp(z[j] - mx);
        out[c] = mx + log(acc);
    }
    free(qh);
    free(z);
}
