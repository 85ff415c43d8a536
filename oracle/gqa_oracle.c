/*
 * gqa_oracle.c -- CPU oracle for gated grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the GPU library, never
 * to stand in for it: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no source, header, table or helper with
 * the HIP code under gated_gqa_decode_amd/csrc/, and it never calls it.
 *
 * What it computes (plain definition, fp64, no blocking, no fusion):
 *
 *   For one query row q (head h, kv head g = h / (H_q / H_kv)) over L keys:
 *     s_j   = scale * sum_d q[d] * K_j[d]                 (fp64; products of
 *                                                           bf16 values are exact)
 *     m     = max_j s_j,   p_j = exp(s_j - m)
 *     O[d]  = (sum_j p_j V_j[d]) / (sum_j p_j)
 *     Ob    = bf16_rne(O)          sigma_b = bf16_rne(1 / (1 + exp(-gate)))
 *     out   = bf16_rne(Ob * sigma_b)                      (the fp64 product of two
 *                                                           bf16 values is exact)
 *   A row with L <= 0 (padded slot / dead row) gives out = +0.
 *
 * Attention-spec options (the _ex entry points; the plain ones pass none):
 *   visible keys   j < L, and with a window w > 0 only the last w of them
 *                  (decode: j >= L - w; prefill row i: j > i - w), and in
 *                  prefill with per-sequence key lengths also j < len[b]
 *   sink           a per-head logit that joins the softmax denominator only:
 *                  Z = sum_visible exp(s_j) + exp(sink_h)
 *   O              sum_visible exp(s_j) V_j / Z      (0 when Z = 0)
 *   lse            ln Z  (-inf when Z = 0), the softmax statistic of the row
 *   A row with no visible key is dead: out = +0 (its lse is the sink, or -inf).
 *
 * FP8 KV pool (oracle_decode_fp8): K and V are stored as OCP float8 e4m3
 * codes with one dequantisation factor per tensor (cuDNN Gated Attention
 * Block page, Quantization specs: static per-tensor scales):
 *   K_j[d] = k_descale * e4m3(code),  V_j[d] = v_descale * e4m3(code)
 * and attention proceeds as above on those values (exact in fp64).
 *
 * Sources (page title, then the part of the page):
 *  - cuDNN FE-OSS "Gated Attention Block (SM107)", Overview, stage (4) SDPA
 *    (softmax(Q K^T * scale + mask) V with GQA H_q / H_kv) and stage (5) gate
 *    (O * sigmoid(GATE)); Forward, fuse_gate ("after the dead-row select").
 *  - FreeToken PR #781 "Fuse the BF16 attention output sigmoid gate into the
 *    Triton decode stage2", Summary: the intermediate BF16 roundings are kept
 *    (O rounded to bf16, sigmoid rounded to bf16 as a per-gate table, and an
 *    explicit round-to-nearest-even of the product).
 *  - ROCm/ATOM PR #838, "PAD_SLOT_ID (-1) handling": padded slots write zeros.
 *  - sglang PR #27630 report, motivation: the unfused model code is
 *    gate = sigmoid(gate); attn_output = attn_output * gate (two ops, two
 *    roundings in bf16).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - GQA head map: query head h uses kv head h / (H_q / H_kv) (contiguous groups).
 *  - Every rounding is round-to-nearest-even of the exact (here fp64) value, with
 *    bf16 subnormals kept, overflow to +-inf, NaN kept as NaN.
 *  - Paged pool layout [num_pages][page_size][H_kv][D]; token j of sequence b is
 *    slot j % page_size of page block_table[b][j / page_size].
 *  - Causal prefill with S_q == S_kv: key j is visible to query i iff j <= i.
 *  - Window, sinks, lse and per-sequence key lengths: the pages name them (the
 *    FreeToken PR's dispatch excludes windows and sinks; the cuDNN page's
 *    Forward offers return_lse, "softmax stats [B, H_q, S] fp32", and
 *    seq_lens_present, per-batch KV lengths) without defining them; the
 *    definitions above are the plain ones: a window keeps the w most recent
 *    keys, a sink is an extra logit with a zero value row, lse = ln Z in
 *    natural-log units, and key lengths mask keys only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EBADARG (-1)
#define ORACLE_EPAGE (-2)
#define ORACLE_ENOMEM (-3)

/* ---------------------------------------------------------------------------
 * bf16 <-> fp64.  bf16 is the top half of an IEEE binary32: 1 sign bit,
 * 8 exponent bits (bias 127), 7 fraction bits.
 * ------------------------------------------------------------------------- */

double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f; /* exact: every binary32 value is a binary64 value */
}

/* Round an fp64 value to the nearest bf16, ties to the even significand.
 * Written from the format's definition: the representable magnitudes in the
 * binade [2^E, 2^(E+1)) are the multiples of 2^(E-7); below 2^-126 the spacing
 * stays 2^-133 (subnormals).  Values at or beyond the midpoint between the
 * largest finite bf16 and 2^128 become infinity. */
uint16_t oracle_bf16_rne(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);

    int e2;
    (void)frexp(a, &e2);   /* a = f * 2^e2 with f in [0.5, 1): floor(log2 a) = e2 - 1 */
    int E = e2 - 1;
    if (E < -126)
        E = -126;          /* subnormal range keeps the spacing of the lowest binade */
    double quantum = ldexp(1.0, E - 7);
    double n = a / quantum;            /* exact: division by a power of two */
    double fl = floor(n);
    double frac = n - fl;              /* exact */
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0))
        r = fl + 1.0;
    /* r is now an integer in [0, 256]; the rounded magnitude is r * quantum. */
    if (r == 0.0)
        return sign;                   /* underflow to signed zero */
    if (r == 256.0) {                  /* carried into the next binade */
        r = 128.0;
        E += 1;
    }
    if (r < 128.0)                     /* only possible when E == -126: subnormal */
        return (uint16_t)(sign | (uint16_t)r);
    int biased = E + 127;
    if (biased >= 255)
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)r - 128));
}

void oracle_bf16_rne_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

/* OCP float8 e4m3 (the "fn" variant: no infinities): 1 sign bit, 4 exponent
 * bits (bias 7), 3 fraction bits.  Exponent field 0 holds the subnormals
 * m * 2^-9; all-ones exponent and fraction (0x7F / 0xFF) is NaN; the largest
 * finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t c)
{
    int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return sign ? -mag : mag;
}

/* sigma_b = bf16_rne(1 / (1 + exp(-g))) evaluated in fp64 (FreeToken PR #781,
 * Summary: the sigmoid of each bf16 gate is itself a bf16 value). */
uint16_t oracle_sigmoid_bf16(uint16_t gate)
{
    double g = oracle_bf16_value(gate);
    double s = 1.0 / (1.0 + exp(-g));
    return oracle_bf16_rne(s);
}

void oracle_sigmoid_table(uint16_t *table /* [65536] */)
{
    for (uint32_t b = 0; b < 65536u; ++b)
        table[b] = oracle_sigmoid_bf16((uint16_t)b);
}

/* out = bf16_rne(Ob * sigma_b): the product of two bf16 values has at most
 * 16 significant bits and lies far inside the fp64 range, so it is exact. */
uint16_t oracle_gate_output(uint16_t ob, uint16_t sigma_b)
{
    return oracle_bf16_rne(oracle_bf16_value(ob) * oracle_bf16_value(sigma_b));
}

/* ---------------------------------------------------------------------------
 * One attention row (cuDNN Gated Attention Block page, Overview stage (4)).
 * krows[j] / vrows[j] point at the D bf16 values of the L visible keys /
 * values (L may be 0).  sink: NULL, or the row's sink logit.
 * o[d] receives O in fp64; mref[d] receives sum_j p_j |V_j[d]| / Z, the
 * magnitude the fp64 sum was formed from (used to size the tolerance);
 * *lse receives ln Z.  Returns 0 for a row with Z = 0 (no visible key and no
 * sink, or a sink of -inf), else 1.
 * ------------------------------------------------------------------------- */
/* K / V element d of a row: a bf16 pattern, or an e4m3 code times its
 * per-tensor dequantisation factor (exact in fp64). */
typedef struct {
    int fp8;
    double k_descale, v_descale;
} kv_format;

static double kv_elem(const void *row, int d, const kv_format *f, double descale)
{
    if (f && f->fp8)
        return descale * oracle_e4m3_value(((const uint8_t *)row)[d]);
    return oracle_bf16_value(((const uint16_t *)row)[d]);
}

static int attend_row(const uint16_t *qrow, const void *const *krows,
                      const void *const *vrows, int L, int D, double scale,
                      const double *sink, const kv_format *f, double *scores, double *o,
                      double *mref, double *lse)
{
    const double kd = f ? f->k_descale : 1.0, vd = f ? f->v_descale : 1.0;
    double m = sink ? *sink : -INFINITY;
    for (int j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += oracle_bf16_value(qrow[d]) * kv_elem(krows[j], d, f, kd);
        scores[j] = scale * dot;
        if (scores[j] > m)
            m = scores[j];
    }
    if (m == -INFINITY) { /* Z = 0: no visible key, and no sink (or a sink of -inf) */
        for (int d = 0; d < D; ++d)
            o[d] = mref[d] = 0.0;
        *lse = -INFINITY;
        return 0;
    }
    double den = sink ? exp(*sink - m) : 0.0;
    for (int j = 0; j < L; ++j) {
        scores[j] = exp(scores[j] - m); /* now p_j */
        den += scores[j];
    }
    for (int d = 0; d < D; ++d) {
        double num = 0.0, mag = 0.0;
        for (int j = 0; j < L; ++j) {
            double v = kv_elem(vrows[j], d, f, vd);
            num += scores[j] * v;
            mag += scores[j] * fabs(v);
        }
        o[d] = num / den;
        mref[d] = mag / den;
    }
    *lse = m + log(den);
    return 1;
}

/* Gate epilogue for one row (stage (5) of the cuDNN page with the bf16
 * rounding chain of FreeToken PR #781). */
static void gate_row(const double *o, const uint16_t *gate_row, int D, uint16_t *out)
{
    for (int d = 0; d < D; ++d) {
        uint16_t ob = oracle_bf16_rne(o[d]);
        uint16_t sb = oracle_sigmoid_bf16(gate_row[d]);
        out[d] = oracle_gate_output(ob, sb);
    }
}

/* ---------------------------------------------------------------------------
 * Decode over a paged KV pool.
 * q, gate, out : [B][H_q][D]                  bf16 bit patterns
 * k_pool,v_pool: [num_pages][page_size][H_kv][D]
 * block_table  : [B][max_pages]               int32 page ids
 * seq_lens     : [B]                          int32, <= 0 means padded slot
 * o_f64, mref  : [B][H_q][D] or NULL
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *q, *gate;
    const void *k_pool, *v_pool;
    const int32_t *block_table, *seq_lens;
    double scale;
    int B, Hq, Hkv, D, page_size, max_pages;
    int64_t num_pages;
    uint16_t *out;
    double *o_f64, *mref;
    const double *sinks; /* [H_q] or NULL */
    int window;          /* > 0: only the last `window` keys are visible */
    double *lse;         /* [B][H_q] or NULL */
    kv_format fmt;       /* bf16 pools, or e4m3 pools with their factors */
    int nthreads, tid;
    int status;
} decode_job;

static void *decode_worker(void *arg)
{
    decode_job *job = (decode_job *)arg;
    const int D = job->D, Hq = job->Hq, Hkv = job->Hkv, ps = job->page_size;
    const int group = Hq / Hkv;
    int maxL = job->max_pages * ps;
    const void **krows = malloc(sizeof(*krows) * (size_t)(maxL > 0 ? maxL : 1));
    const void **vrows = malloc(sizeof(*vrows) * (size_t)(maxL > 0 ? maxL : 1));
    double *scores = malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    const size_t esize = job->fmt.fp8 ? 1 : 2; /* bytes per pool element */
    double *o = malloc(sizeof(double) * (size_t)D);
    double *mref = malloc(sizeof(double) * (size_t)D);
    if (!krows || !vrows || !scores || !o || !mref) {
        job->status = ORACLE_ENOMEM;
        goto done;
    }
    for (int row = job->tid; row < job->B * Hq; row += job->nthreads) {
        int b = row / Hq, h = row % Hq, g = h / group;
        size_t rbase = ((size_t)b * Hq + h) * D;
        int L = job->seq_lens[b];
        if (L > maxL) {
            job->status = ORACLE_EBADARG;
            goto done;
        }
        int j0 = 0; /* first visible key */
        if (job->window > 0 && L - job->window > 0)
            j0 = L - job->window;
        int nvis = L > j0 ? L - j0 : 0;
        for (int j = j0; j < L; ++j) {
            int32_t page = job->block_table[(size_t)b * job->max_pages + j / ps];
            if (page < 0 || page >= job->num_pages) {
                job->status = ORACLE_EPAGE;
                goto done;
            }
            size_t off = (((size_t)page * ps + (size_t)(j % ps)) * Hkv + g) * D * esize;
            krows[j - j0] = (const char *)job->k_pool + off;
            vrows[j - j0] = (const char *)job->v_pool + off;
        }
        double lse;
        attend_row(job->q + rbase, krows, vrows, nvis, D, job->scale,
                   job->sinks ? &job->sinks[h] : NULL, &job->fmt, scores, o, mref, &lse);
        if (nvis == 0) { /* dead row (padded slot): the dead-row select gives +0 */
            for (int d = 0; d < D; ++d)
                job->out[rbase + d] = 0;
        } else {
            gate_row(o, job->gate + rbase, D, job->out + rbase);
        }
        if (job->lse)
            job->lse[(size_t)b * Hq + h] = lse;
        if (job->o_f64)
            memcpy(job->o_f64 + rbase, o, sizeof(double) * (size_t)D);
        if (job->mref)
            memcpy(job->mref + rbase, mref, sizeof(double) * (size_t)D);
    }
done:
    free(krows);
    free(vrows);
    free(scores);
    free(o);
    free(mref);
    return NULL;
}

static int run_jobs(void *jobs, size_t job_size, int nthreads, void *(*fn)(void *))
{
    pthread_t *th = malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th)
        return ORACLE_ENOMEM;
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, (char *)jobs + job_size * (size_t)t) != 0)
            break;
        started = t;
    }
    fn(jobs); /* thread 0 runs on the caller */
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    /* threads that failed to start: run their share here */
    for (int t = started + 1; t < nthreads; ++t)
        fn((char *)jobs + job_size * (size_t)t);
    free(th);
    return ORACLE_OK;
}

static int decode_any(const uint16_t *q, const uint16_t *gate, const void *k_pool,
                      const void *v_pool, const int32_t *block_table, const int32_t *seq_lens,
                      double scale, kv_format fmt, int B, int Hq, int Hkv, int D, int page_size,
                      int max_pages, int64_t num_pages, const double *sinks, int window,
                      uint16_t *out, double *o_f64, double *mref, double *lse, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || max_pages < 0 ||
        num_pages < 0 || Hq % Hkv != 0)
        return ORACLE_EBADARG;
    if (B == 0)
        return ORACLE_OK;
    if (!q || !gate || !k_pool || !v_pool || !block_table || !seq_lens || !out)
        return ORACLE_EBADARG;
    if (nthreads < 1)
        nthreads = 1;
    decode_job *jobs = calloc((size_t)nthreads, sizeof(decode_job));
    if (!jobs)
        return ORACLE_ENOMEM;
    for (int t = 0; t < nthreads; ++t) {
        decode_job j = {q, gate, k_pool, v_pool, block_table, seq_lens, scale,
                        B, Hq, Hkv, D, page_size, max_pages, num_pages,
                        out, o_f64, mref, sinks, window, lse, fmt, nthreads, t, ORACLE_OK};
        jobs[t] = j;
    }
    int st = run_jobs(jobs, sizeof(decode_job), nthreads, decode_worker);
    for (int t = 0; t < nthreads && st == ORACLE_OK; ++t)
        if (jobs[t].status != ORACLE_OK)
            st = jobs[t].status;
    free(jobs);
    return st;
}

int oracle_decode_ex(const uint16_t *q, const uint16_t *gate, const uint16_t *k_pool,
                     const uint16_t *v_pool, const int32_t *block_table, const int32_t *seq_lens,
                     double scale, int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                     int64_t num_pages, const double *sinks, int window, uint16_t *out,
                     double *o_f64, double *mref, double *lse, int nthreads)
{
    kv_format fmt = {0, 1.0, 1.0};
    return decode_any(q, gate, k_pool, v_pool, block_table, seq_lens, scale, fmt, B, Hq, Hkv, D,
                      page_size, max_pages, num_pages, sinks, window, out, o_f64, mref, lse,
                      nthreads);
}

/* Decode over e4m3 K / V pools ([num_pages][page_size][H_kv][D] bytes) with
 * per-tensor dequantisation factors; otherwise as oracle_decode_ex. */
int oracle_decode_fp8(const uint16_t *q, const uint16_t *gate, const uint8_t *k_pool,
                      const uint8_t *v_pool, const int32_t *block_table, const int32_t *seq_lens,
                      double scale, double k_descale, double v_descale, int B, int Hq, int Hkv,
                      int D, int page_size, int max_pages, int64_t num_pages,
                      const double *sinks, int window, uint16_t *out, double *o_f64,
                      double *mref, double *lse, int nthreads)
{
    kv_format fmt = {1, k_descale, v_descale};
    return decode_any(q, gate, k_pool, v_pool, block_table, seq_lens, scale, fmt, B, Hq, Hkv, D,
                      page_size, max_pages, num_pages, sinks, window, out, o_f64, mref, lse,
                      nthreads);
}

int oracle_decode(const uint16_t *q, const uint16_t *gate, const uint16_t *k_pool,
                  const uint16_t *v_pool, const int32_t *block_table, const int32_t *seq_lens,
                  double scale, int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                  int64_t num_pages, uint16_t *out, double *o_f64, double *mref, int nthreads)
{
    return oracle_decode_ex(q, gate, k_pool, v_pool, block_table, seq_lens, scale, B, Hq, Hkv,
                            D, page_size, max_pages, num_pages, NULL, 0, out, o_f64, mref,
                            NULL, nthreads);
}

/* ---------------------------------------------------------------------------
 * Dense prefill (cuDNN Gated Attention Block page, Overview: Q, GATE [B,S,H_q,D],
 * K, V [B,S,H_kv,D]; stage (4) with a causal or no mask; stage (5) gate).
 * rows: nrows (b, i) pairs selecting the query positions to evaluate (all
 * heads of each); rows == NULL evaluates every position and then nrows must
 * be B * S.  Results are written compactly: out[r][H_q][D] for r < nrows.
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *q, *gate, *k, *v;
    double scale;
    int causal, B, S, Hq, Hkv, D;
    const int32_t *rows;
    int nrows;
    uint16_t *out;
    double *o_f64, *mref;
    const int32_t *seq_lens; /* [B] key lengths or NULL (all S) */
    const double *sinks;     /* [H_q] or NULL */
    int window;              /* > 0: row i sees keys j > i - window */
    double *lse;             /* [nrows][H_q] or NULL */
    int nthreads, tid;
    int status;
} prefill_job;

static void *prefill_worker(void *arg)
{
    prefill_job *job = (prefill_job *)arg;
    const int D = job->D, Hq = job->Hq, Hkv = job->Hkv, S = job->S;
    const int group = Hq / Hkv;
    const void **krows = malloc(sizeof(*krows) * (size_t)S);
    const void **vrows = malloc(sizeof(*vrows) * (size_t)S);
    double *scores = malloc(sizeof(double) * (size_t)S);
    double *o = malloc(sizeof(double) * (size_t)D);
    double *mref = malloc(sizeof(double) * (size_t)D);
    if (!krows || !vrows || !scores || !o || !mref) {
        job->status = ORACLE_ENOMEM;
        goto done;
    }
    for (int item = job->tid; item < job->nrows * Hq; item += job->nthreads) {
        int r = item / Hq, h = item % Hq, g = h / group;
        int b, i;
        if (job->rows) {
            b = job->rows[2 * r];
            i = job->rows[2 * r + 1];
        } else {
            b = r / S;
            i = r % S;
        }
        if (b < 0 || b >= job->B || i < 0 || i >= S) {
            job->status = ORACLE_EBADARG;
            goto done;
        }
        /* visible keys: [j0, j1) -- key length, causal mask, window */
        int j1 = S;
        if (job->seq_lens) {
            int len = job->seq_lens[b];
            j1 = len < 0 ? 0 : (len < S ? len : S);
        }
        if (job->causal && i + 1 < j1)
            j1 = i + 1; /* keys j <= i are visible under the causal mask */
        int j0 = 0;
        if (job->window > 0 && i - job->window + 1 > 0)
            j0 = i - job->window + 1;
        int nvis = j1 > j0 ? j1 - j0 : 0;
        for (int j = j0; j < j1; ++j) {
            size_t off = (((size_t)b * S + j) * Hkv + g) * D;
            krows[j - j0] = job->k + off;
            vrows[j - j0] = job->v + off;
        }
        size_t qbase = (((size_t)b * S + i) * Hq + h) * D;
        size_t obase = ((size_t)r * Hq + h) * D;
        double lse;
        attend_row(job->q + qbase, krows, vrows, nvis, D, job->scale,
                   job->sinks ? &job->sinks[h] : NULL, NULL, scores, o, mref, &lse);
        if (nvis == 0) { /* dead row: +0 */
            for (int d = 0; d < D; ++d)
                job->out[obase + d] = 0;
        } else {
            gate_row(o, job->gate + qbase, D, job->out + obase);
        }
        if (job->lse)
            job->lse[(size_t)r * Hq + h] = lse;
        if (job->o_f64)
            memcpy(job->o_f64 + obase, o, sizeof(double) * (size_t)D);
        if (job->mref)
            memcpy(job->mref + obase, mref, sizeof(double) * (size_t)D);
    }
done:
    free(krows);
    free(vrows);
    free(scores);
    free(o);
    free(mref);
    return NULL;
}

int oracle_prefill_ex(const uint16_t *q, const uint16_t *gate, const uint16_t *k,
                      const uint16_t *v, double scale, int causal, int B, int S, int Hq,
                      int Hkv, int D, const int32_t *seq_lens, const double *sinks, int window,
                      const int32_t *rows, int nrows, uint16_t *out, double *o_f64,
                      double *mref, double *lse, int nthreads)
{
    if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || nrows < 0)
        return ORACLE_EBADARG;
    if (!rows && nrows != B * S)
        return ORACLE_EBADARG;
    if (nrows == 0)
        return ORACLE_OK;
    if (!q || !gate || !k || !v || !out)
        return ORACLE_EBADARG;
    if (nthreads < 1)
        nthreads = 1;
    prefill_job *jobs = calloc((size_t)nthreads, sizeof(prefill_job));
    if (!jobs)
        return ORACLE_ENOMEM;
    for (int t = 0; t < nthreads; ++t) {
        prefill_job j = {q, gate, k, v, scale, causal, B, S, Hq, Hkv, D, rows, nrows,
                         out, o_f64, mref, seq_lens, sinks, window, lse, nthreads, t,
                         ORACLE_OK};
        jobs[t] = j;
    }
    int st = run_jobs(jobs, sizeof(prefill_job), nthreads, prefill_worker);
    for (int t = 0; t < nthreads && st == ORACLE_OK; ++t)
        if (jobs[t].status != ORACLE_OK)
            st = jobs[t].status;
    free(jobs);
    return st;
}

int oracle_prefill(const uint16_t *q, const uint16_t *gate, const uint16_t *k, const uint16_t *v,
                   double scale, int causal, int B, int S, int Hq, int Hkv, int D,
                   const int32_t *rows, int nrows, uint16_t *out, double *o_f64, double *mref,
                   int nthreads)
{
    return oracle_prefill_ex(q, gate, k, v, scale, causal, B, S, Hq, Hkv, D, NULL, NULL, 0,
                             rows, nrows, out, o_f64, mref, NULL, nthreads);
}

/* ---------------------------------------------------------------------------
 * The step before attention: per-head QK-RMSNorm and partial RoPE on q and k,
 * with the token's K / V written to its pool slot (cuDNN Gated Attention
 * Block page, Overview stages (2)+(3): "QK-RMSNorm per head (optional) +
 * partial RoPE on the first rope_dim", one kernel for Q and K; Weights and
 * tables: cos, sin [.., rope_dim] rotary tables in the activation dtype,
 * rotate-half convention on the first rope_dim dims of every head; w_q_norm,
 * w_k_norm [D]; Fusion knobs: normed and rotated on fp32 values and written
 * once).
 *
 * For one head row x[D] of token t (bf16), in fp64:
 *   y_d   = x_d / sqrt(mean_d' x_d'^2 + eps) * w_d          (w == NULL: y = x)
 *   for i < R/2, p = i + R/2  (R = rope_dim, rotate-half):
 *     z_i = y_i cos[t][i] - y_p sin[t][i],   z_p = y_p cos[t][p] + y_i sin[t][p]
 *   z_d = y_d for d >= R;  out_d = bf16_rne(z_d)
 * and, for the magnitude a rotated value is formed from (tolerance sizing),
 *   mag_i = |y_i cos[t][i]| + |y_p sin[t][i]|, mag_p likewise, mag_d = |y_d|.
 * Readings (the pages are silent): eps is a parameter; the norm weight
 * multiplies the normalised value (no offset); a table entry is used as given
 * (the two halves' cos / sin are not assumed equal).
 * ------------------------------------------------------------------------- */
static void norm_rope_row(const uint16_t *x, const uint16_t *w, double eps, const uint16_t *cos_t,
                          const uint16_t *sin_t, int D, int R, uint16_t *out, double *z_out,
                          double *mag_out)
{
    double y[1024];
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
        y[d] = oracle_bf16_value(x[d]);
        ss += y[d] * y[d];
    }
    if (w) {
        double r = 1.0 / sqrt(ss / D + eps);
        for (int d = 0; d < D; ++d)
            y[d] = y[d] * r * oracle_bf16_value(w[d]);
    }
    for (int d = 0; d < D; ++d) {
        double z = y[d], mag = fabs(y[d]);
        if (d < R) {
            int half = R / 2;
            int i = d < half ? d : d - half; /* first-half index of the pair */
            double c = oracle_bf16_value(cos_t[d]), s = oracle_bf16_value(sin_t[d]);
            if (d < half) { /* z_i = y_i cos - y_p sin */
                z = y[i] * c - y[i + half] * s;
                mag = fabs(y[i] * c) + fabs(y[i + half] * s);
            } else {        /* z_p = y_p cos + y_i sin */
                z = y[d] * c + y[i] * s;
                mag = fabs(y[d] * c) + fabs(y[i] * s);
            }
        }
        out[d] = oracle_bf16_rne(z);
        if (z_out)
            z_out[d] = z;
        if (mag_out)
            mag_out[d] = mag;
    }
}

/* T tokens: q [T][H_q][D], k and v [T][H_kv][D]; cos, sin [T][R].
 * q_out [T][H_q][D] always.  With slot_mapping: K / V of token t go to slot
 * s = slot_mapping[t] of the pools k_out / v_out ([num_pages * page_size]
 * [H_kv][D]); s < 0 writes nothing.  Without: k_out / v_out are dense
 * [T][H_kv][D] (v_out may be NULL).  qz / qmag, kz / kmag (optional, the
 * shapes of q and k) receive the fp64 values before rounding and their
 * magnitudes.  Returns -1 for bad arguments or a slot outside the pools. */
int oracle_qk_norm_rope(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const uint16_t *w_q, const uint16_t *w_k, double eps,
                        const uint16_t *cos_tab, const uint16_t *sin_tab, const int64_t *slot_mapping,
                        int64_t T, int Hq, int Hkv, int D, int R, int64_t num_slots,
                        uint16_t *q_out, uint16_t *k_out, uint16_t *v_out,
                        double *qz, double *qmag, double *kz, double *kmag)
{
    if (T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 || R < 0 || R > D || R % 2 != 0)
        return ORACLE_EBADARG;
    if ((w_q == NULL) != (w_k == NULL))
        return ORACLE_EBADARG;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *ct = R ? cos_tab + t * R : NULL, *st = R ? sin_tab + t * R : NULL;
        for (int h = 0; h < Hq; ++h) {
            size_t off = ((size_t)t * Hq + h) * D;
            norm_rope_row(q + off, w_q, eps, ct, st, D, R, q_out + off, qz ? qz + off : NULL,
                          qmag ? qmag + off : NULL);
        }
        int64_t slot = slot_mapping ? slot_mapping[t] : t;
        if (slot_mapping && slot >= num_slots)
            return ORACLE_EBADARG;
        for (int h = 0; h < Hkv; ++h) {
            size_t in_off = ((size_t)t * Hkv + h) * D;
            uint16_t krow[1024];
            norm_rope_row(k + in_off, w_k, eps, ct, st, D, R, krow, kz ? kz + in_off : NULL,
                          kmag ? kmag + in_off : NULL);
            if (slot < 0)
                continue;
            size_t out_off = ((size_t)slot * Hkv + h) * D;
            memcpy(k_out + out_off, krow, sizeof(uint16_t) * (size_t)D);
            if (v_out)
                memcpy(v_out + out_off, v + in_off, sizeof(uint16_t) * (size_t)D);
        }
    }
    return ORACLE_OK;
}
