/*
 * rvq_oracle.c -- plain, slow CPU oracle for residual vector quantization.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it follows:
 *   - Encode: the residual loop of the "RVQ codec" section of the
 *     "Architecture" page (omnivoice.cpp). Stage by stage, pick the codeword
 *     with the smallest squared L2 distance to the current residual, emit
 *     its index, subtract the codeword. Identity projections: the codebooks
 *     act directly on the D-dim latent.
 *   - Ties go to the lowest index (strict "<" while scanning k upward).
 *   - Decode: the per-codebook accumulation of the same section (and of the
 *     "Audio tokenizer pipeline" decode listing): gather each stage's row,
 *     add it to an accumulator that starts at +0, stage 0 first.
 *   - Linear: y = W h + b with W in PyTorch (out, in) order, used for the
 *     fc 1024->64 prologue and fc2 64->1024 epilogue of the projected
 *     workload.
 *   - Per-stage projected encode and decode: the same section's loop with
 *     each codebook's own project_in (hidden -> dim, with bias) before the
 *     argmin and project_out (dim -> hidden, with bias) applied to the
 *     picked codeword before it is subtracted from the hidden-width
 *     residual; decode sums the projected codewords, stage 0 first.
 *   - Normalized (cosine) variant of it: the quantizer of the
 *     "Maintainer's guide -- moss-tts.cpp" page (gotchas, item 9) scales
 *     the projected encoding and every codeword to unit L2 norm (dividing by
 *     max(norm, 1e-12)) before the argmin; the decode and the residual
 *     update use the stored codeword, unscaled.
 *
 * Precision (the pages fix only that the codec is kept in F32):
 *   - distances: float64, direct form sum_j (r_j - c_j)^2, j ascending,
 *     one rounding per operation (built with -ffp-contract=off);
 *   - residual: float32, r_j <- fl32(r_j - c_j);
 *   - decode accumulator: float32, stage order ascending;
 *   - linear (and both per-stage projections): float64 sum, i ascending,
 *     bias added last, rounded once to float32;
 *   - normalization: float64 throughout (squares summed j ascending, sqrt,
 *     one division per element), distances in float64 on the normalized
 *     vectors, direct form.
 *
 * The best and second-best distances of every stage are reported too, so
 * a caller can classify near-ties (gap <= 1e-5 * best).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_MAX_THREADS 256

/* Squared L2 distance in float64, direct form, j ascending. */
static double sq_dist(const float *r, const float *c, int32_t dim)
{
    double s = 0.0;
    for (int32_t j = 0; j < dim; ++j) {
        double t = (double)r[j] - (double)c[j];
        s = s + t * t;
    }
    return s;
}

/* Index of the codeword of `book` [n_codes, dim] nearest to v, the lowest
 * index on ties (strict "<" while k ascends); *best and *second receive the
 * smallest and second-smallest distance. */
static int32_t nearest(const float *v, const float *book, int32_t n_codes, int32_t dim,
                       double *best, double *second)
{
    int32_t k1 = 0;
    double d1 = sq_dist(v, book, dim);
    double d2 = INFINITY;
    for (int32_t k = 1; k < n_codes; ++k) {
        double dk = sq_dist(v, book + (int64_t)k * dim, dim);
        if (dk < d1) {
            d2 = d1;
            d1 = dk;
            k1 = k;
        } else if (dk < d2) {
            d2 = dk;
        }
    }
    *best = d1;
    *second = d2;
    return k1;
}

/* out = v / max(||v||_2, 1e-12), all in float64. */
static void unit_vector(const float *v, int32_t dim, double *out)
{
    double ss = 0.0;
    for (int32_t j = 0; j < dim; ++j) ss = ss + (double)v[j] * (double)v[j];
    double norm = sqrt(ss);
    if (norm < 1e-12) norm = 1e-12;
    for (int32_t j = 0; j < dim; ++j) out[j] = (double)v[j] / norm;
}

/* As `nearest`, on float64 vectors: `units` [n_codes, dim] are the
 * normalized codewords, u the normalized encoding. */
static int32_t nearest_unit(const double *u, const double *units, int32_t n_codes, int32_t dim,
                            double *best, double *second)
{
    int32_t pick = 0;
    double lo = INFINITY, next = INFINITY;
    for (int32_t k = 0; k < n_codes; ++k) {
        const double *ck = units + (int64_t)k * dim;
        double acc = 0.0;
        for (int32_t j = 0; j < dim; ++j) {
            const double t = u[j] - ck[j];
            acc = acc + t * t;
        }
        if (acc < lo) {
            next = lo;
            lo = acc;
            pick = k;
        } else if (acc < next) {
            next = acc;
        }
    }
    *best = lo;
    *second = next;
    return pick;
}

/* y = W v + b for one vector: W [out_dim, in_dim] row-major, b nullable;
 * float64 sum over i ascending, bias added last, rounded once. */
static void linear_row(const float *w, const float *b, const float *v,
                       int32_t in_dim, int32_t out_dim, float *y)
{
    for (int32_t o = 0; o < out_dim; ++o) {
        const float *wo = w + (int64_t)o * in_dim;
        double s = 0.0;
        for (int32_t i = 0; i < in_dim; ++i) s = s + (double)v[i] * (double)wo[i];
        if (b) s = s + (double)b[o];
        y[o] = (float)s;
    }
}

typedef struct {
    const float *x;
    const float *books;
    int32_t dim, n_stages, n_codes;
    int32_t *codes;
    int32_t codes_ld;
    float *residual;      /* nullable */
    double *best;         /* nullable, [N, Q] */
    double *second;       /* nullable, [N, Q] */
    int64_t begin, end;
} encode_job;

static void encode_frames(const encode_job *jb)
{
    float *r = (float *)malloc(sizeof(float) * (size_t)jb->dim);
    for (int64_t n = jb->begin; n < jb->end; ++n) {
        memcpy(r, jb->x + n * jb->dim, sizeof(float) * (size_t)jb->dim);
        for (int32_t q = 0; q < jb->n_stages; ++q) {
            const float *book = jb->books + (int64_t)q * jb->n_codes * jb->dim;
            double d1, d2;
            int32_t k1 = nearest(r, book, jb->n_codes, jb->dim, &d1, &d2);
            jb->codes[n * jb->codes_ld + q] = k1;
            if (jb->best) jb->best[n * jb->n_stages + q] = d1;
            if (jb->second) jb->second[n * jb->n_stages + q] = d2;
            const float *c = book + (int64_t)k1 * jb->dim;
            for (int32_t j = 0; j < jb->dim; ++j) r[j] = (float)(r[j] - c[j]);
        }
        if (jb->residual) memcpy(jb->residual + n * jb->dim, r, sizeof(float) * (size_t)jb->dim);
    }
    free(r);
}

typedef struct {
    const int32_t *codes;
    int32_t codes_ld;
    const float *books;
    int32_t n_stages, n_codes, dim;
    float *out;
    int64_t begin, end;
} decode_job;

static void decode_frames(const decode_job *jb)
{
    for (int64_t n = jb->begin; n < jb->end; ++n) {
        float *o = jb->out + n * jb->dim;
        for (int32_t j = 0; j < jb->dim; ++j) o[j] = 0.0f;
        for (int32_t q = 0; q < jb->n_stages; ++q) {
            int32_t k = jb->codes[n * jb->codes_ld + q];
            if (k < 0 || k >= jb->n_codes) {
                for (int32_t j = 0; j < jb->dim; ++j) o[j] = NAN;
                break;
            }
            const float *c = jb->books + ((int64_t)q * jb->n_codes + k) * jb->dim;
            for (int32_t j = 0; j < jb->dim; ++j) o[j] = (float)(o[j] + c[j]);
        }
    }
}

typedef struct {
    const float *h;
    int32_t in_dim, out_dim;
    const float *w;
    const float *b;  /* nullable */
    float *y;
    int64_t begin, end;
} linear_job;

static void linear_rows(const linear_job *jb)
{
    for (int64_t n = jb->begin; n < jb->end; ++n)
        linear_row(jb->w, jb->b, jb->h + n * jb->in_dim, jb->in_dim, jb->out_dim,
                   jb->y + n * jb->out_dim);
}

typedef struct {
    const float *h;
    int32_t hidden, dim, n_stages, n_codes;
    const float *w_in, *b_in;    /* [Q, dim, hidden], [Q, dim] (nullable) */
    const float *books;          /* [Q, K, dim] */
    const float *w_out, *b_out;  /* [Q, hidden, dim], [Q, hidden] (nullable) */
    const float *e_given;        /* nullable [Q, N, dim] */
    const double *units;         /* nullable [Q, K, dim]: normalized codewords (cosine variant) */
    int32_t *codes;
    int32_t codes_ld;
    float *e_out;                /* nullable [Q, N, dim] */
    float *residual;             /* nullable [N, hidden] */
    double *best, *second;       /* nullable [N, Q] */
    int64_t n_frames;
    int64_t begin, end;
} projected_job;

/* Per-stage projected encode of frames [begin, end). For each stage q the
 * projection e = W_in[q] r + b_in[q] is computed; the argmin is taken on it,
 * or on e_given[q, n] when e_given is set (the residual chain then follows
 * those picks); the picked codeword is projected back with W_out[q] and
 * b_out[q] and subtracted from the hidden-width residual in float32. */
static void projected_frames(const projected_job *jb)
{
    const int32_t hid = jb->hidden, dim = jb->dim;
    float *r = (float *)malloc(sizeof(float) * (size_t)hid);
    float *p = (float *)malloc(sizeof(float) * (size_t)hid);
    float *e = (float *)malloc(sizeof(float) * (size_t)dim);
    double *u = (double *)malloc(sizeof(double) * (size_t)dim);
    for (int64_t n = jb->begin; n < jb->end; ++n) {
        memcpy(r, jb->h + n * hid, sizeof(float) * (size_t)hid);
        for (int32_t q = 0; q < jb->n_stages; ++q) {
            const float *b_in = jb->b_in ? jb->b_in + (int64_t)q * dim : NULL;
            linear_row(jb->w_in + (int64_t)q * dim * hid, b_in, r, hid, dim, e);
            const int64_t at = ((int64_t)q * jb->n_frames + n) * dim;
            if (jb->e_out) memcpy(jb->e_out + at, e, sizeof(float) * (size_t)dim);
            const float *pick_on = jb->e_given ? jb->e_given + at : e;
            const float *stage_book = jb->books + (int64_t)q * jb->n_codes * dim;
            double d1, d2;
            int32_t k1;
            if (jb->units) {
                unit_vector(pick_on, dim, u);
                k1 = nearest_unit(u, jb->units + (int64_t)q * jb->n_codes * dim, jb->n_codes, dim, &d1, &d2);
            } else {
                k1 = nearest(pick_on, stage_book, jb->n_codes, dim, &d1, &d2);
            }
            const int64_t nq = n * jb->n_stages + q;
            jb->codes[n * jb->codes_ld + q] = k1;
            if (jb->best) jb->best[nq] = d1;
            if (jb->second) jb->second[nq] = d2;
            const float *b_out = jb->b_out ? jb->b_out + (int64_t)q * hid : NULL;
            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book + (int64_t)k1 * dim, dim, hid, p);
            for (int32_t i = 0; i < hid; ++i) r[i] = (float)(r[i] - p[i]);
        }
        if (jb->residual) memcpy(jb->residual + n * hid, r, sizeof(float) * (size_t)hid);
    }
    free(u);
    free(e);
    free(p);
    free(r);
}

typedef struct {
    const int32_t *codes;
    int32_t codes_ld;
    const float *books;          /* [Q, K, dim] */
    const float *w_out, *b_out;  /* [Q, hidden, dim], [Q, hidden] (nullable) */
    int32_t n_stages, n_codes, dim, hidden;
    float *out;                  /* [N, hidden] */
    int64_t begin, end;
} projected_decode_job;

/* out[n] = sum_q (W_out[q] C[q, codes[n, q]] + b_out[q]): each stage's
 * projected codeword rounded to float32, then added to a float32
 * accumulator that starts at +0, stage 0 first. A code outside [0, K)
 * gives a NaN frame. */
static void projected_decode_frames(const projected_decode_job *jb)
{
    const int32_t hid = jb->hidden, dim = jb->dim;
    float *p = (float *)malloc(sizeof(float) * (size_t)hid);
    for (int64_t n = jb->begin; n < jb->end; ++n) {
        float *acc = jb->out + n * hid;
        for (int32_t i = 0; i < hid; ++i) acc[i] = 0.0f;
        for (int32_t q = 0; q < jb->n_stages; ++q) {
            int32_t code = jb->codes[n * jb->codes_ld + q];
            if (code < 0 || code >= jb->n_codes) {
                for (int32_t i = 0; i < hid; ++i) acc[i] = NAN;
                break;
            }
            const float *b_out = jb->b_out ? jb->b_out + (int64_t)q * hid : NULL;
            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out,
                       jb->books + ((int64_t)q * jb->n_codes + code) * dim, dim, hid, p);
            for (int32_t i = 0; i < hid; ++i) acc[i] = (float)(acc[i] + p[i]);
        }
    }
    free(p);
}

/* ---- threading: contiguous frame ranges, one pthread each ------------- */

enum { JOB_ENCODE, JOB_DECODE, JOB_LINEAR, JOB_PROJECTED, JOB_PROJECTED_DECODE };

typedef struct {
    int kind;
    union {
        encode_job e;
        decode_job d;
        linear_job l;
        projected_job p;
        projected_decode_job pd;
    } u;
} any_job;

static void *run_job(void *p)
{
    any_job *j = (any_job *)p;
    if (j->kind == JOB_ENCODE) encode_frames(&j->u.e);
    else if (j->kind == JOB_DECODE) decode_frames(&j->u.d);
    else if (j->kind == JOB_LINEAR) linear_rows(&j->u.l);
    else if (j->kind == JOB_PROJECTED) projected_frames(&j->u.p);
    else projected_decode_frames(&j->u.pd);
    return NULL;
}

static int pick_threads(int requested, int64_t n)
{
    int t = requested;
    if (t <= 0) {
        cpu_set_t set;
        CPU_ZERO(&set);
        if (sched_getaffinity(0, sizeof set, &set) == 0) t = CPU_COUNT(&set);
        if (t <= 0) {
            long c = sysconf(_SC_NPROCESSORS_ONLN);
            t = c > 0 ? (int)c : 1;
        }
    }
    if (t > ORACLE_MAX_THREADS) t = ORACLE_MAX_THREADS;
    if ((int64_t)t > n) t = (int)(n > 0 ? n : 1);
    return t;
}

/* Splits [0, n) into `t` contiguous ranges and runs `proto` on each. */
static int run_parallel(any_job proto, int64_t n, int t)
{
    any_job jobs[ORACLE_MAX_THREADS];
    pthread_t tids[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    for (int i = 0; i < t; ++i) {
        int64_t b = n * i / t, e = n * (i + 1) / t;
        jobs[i] = proto;
        if (proto.kind == JOB_ENCODE) { jobs[i].u.e.begin = b; jobs[i].u.e.end = e; }
        else if (proto.kind == JOB_DECODE) { jobs[i].u.d.begin = b; jobs[i].u.d.end = e; }
        else if (proto.kind == JOB_LINEAR) { jobs[i].u.l.begin = b; jobs[i].u.l.end = e; }
        else if (proto.kind == JOB_PROJECTED) { jobs[i].u.p.begin = b; jobs[i].u.p.end = e; }
        else { jobs[i].u.pd.begin = b; jobs[i].u.pd.end = e; }
        started[i] = (t > 1) && pthread_create(&tids[i], NULL, run_job, &jobs[i]) == 0;
        if (!started[i]) run_job(&jobs[i]);
    }
    for (int i = 0; i < t; ++i)
        if (started[i]) pthread_join(tids[i], NULL);
    return t;
}

/* ---- exported entry points --------------------------------------------- */

/* Encodes frames [0, n_frames). Returns the number of threads used. */
int oracle_encode(const float *x, int64_t n_frames, int32_t dim,
                  const float *books, int32_t n_stages, int32_t n_codes,
                  int32_t *codes, int32_t codes_ld, float *residual,
                  double *best, double *second, int threads)
{
    if (n_frames <= 0) return 0;
    any_job p;
    memset(&p, 0, sizeof p);
    p.kind = JOB_ENCODE;
    p.u.e.x = x; p.u.e.books = books; p.u.e.dim = dim;
    p.u.e.n_stages = n_stages; p.u.e.n_codes = n_codes;
    p.u.e.codes = codes; p.u.e.codes_ld = codes_ld; p.u.e.residual = residual;
    p.u.e.best = best; p.u.e.second = second;
    return run_parallel(p, n_frames, pick_threads(threads, n_frames));
}

/* Decodes frames [0, n_frames). Codes outside [0, K) give a NaN frame. */
int oracle_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                  const float *books, int32_t n_stages, int32_t n_codes,
                  int32_t dim, float *out, int threads)
{
    if (n_frames <= 0) return 0;
    any_job p;
    memset(&p, 0, sizeof p);
    p.kind = JOB_DECODE;
    p.u.d.codes = codes; p.u.d.codes_ld = codes_ld; p.u.d.books = books;
    p.u.d.n_stages = n_stages; p.u.d.n_codes = n_codes; p.u.d.dim = dim; p.u.d.out = out;
    return run_parallel(p, n_frames, pick_threads(threads, n_frames));
}

/* y[n, :] = W h[n, :] + b, W is [out_dim, in_dim] row-major. */
int oracle_linear(const float *h, int64_t n_rows, int32_t in_dim,
                  const float *w, const float *b, int32_t out_dim,
                  float *y, int threads)
{
    if (n_rows <= 0) return 0;
    any_job p;
    memset(&p, 0, sizeof p);
    p.kind = JOB_LINEAR;
    p.u.l.h = h; p.u.l.in_dim = in_dim; p.u.l.out_dim = out_dim;
    p.u.l.w = w; p.u.l.b = b; p.u.l.y = y;
    return run_parallel(p, n_rows, pick_threads(threads, n_rows));
}

/* Per-stage projected encode of frames [0, n_frames); see projected_frames.
 * e_given, e_out, residual, best and second are nullable. With `normalize`
 * set, every argmin is taken between the normalized encoding and the
 * normalized codewords (best / second are then those distances). */
int oracle_projected_encode(const float *h, int64_t n_frames, int32_t hidden,
                            const float *w_in, const float *b_in,
                            const float *books, int32_t n_stages, int32_t n_codes, int32_t dim,
                            const float *w_out, const float *b_out, const float *e_given,
                            int32_t *codes, int32_t codes_ld, float *e_out, float *residual,
                            double *best, double *second, int normalize, int threads)
{
    if (n_frames <= 0) return 0;
    double *units = NULL;
    if (normalize) {
        const int64_t rows = (int64_t)n_stages * n_codes;
        units = (double *)malloc(sizeof(double) * (size_t)(rows * dim));
        for (int64_t k = 0; k < rows; ++k) unit_vector(books + k * dim, dim, units + k * dim);
    }
    any_job p;
    memset(&p, 0, sizeof p);
    p.kind = JOB_PROJECTED;
    p.u.p.h = h; p.u.p.hidden = hidden; p.u.p.dim = dim;
    p.u.p.n_stages = n_stages; p.u.p.n_codes = n_codes;
    p.u.p.w_in = w_in; p.u.p.b_in = b_in; p.u.p.books = books;
    p.u.p.w_out = w_out; p.u.p.b_out = b_out; p.u.p.e_given = e_given;
    p.u.p.codes = codes; p.u.p.codes_ld = codes_ld; p.u.p.e_out = e_out;
    p.u.p.residual = residual; p.u.p.best = best; p.u.p.second = second;
    p.u.p.n_frames = n_frames;
    p.u.p.units = units;
    const int used = run_parallel(p, n_frames, pick_threads(threads, n_frames));
    free(units);
    return used;
}

/* Per-stage projected decode of frames [0, n_frames) into out [N, hidden]. */
int oracle_projected_decode(const int32_t *codes, int32_t codes_ld, int64_t n_frames,
                            const float *books, int32_t n_stages, int32_t n_codes, int32_t dim,
                            const float *w_out, const float *b_out, int32_t hidden,
                            float *out, int threads)
{
    if (n_frames <= 0) return 0;
    any_job p;
    memset(&p, 0, sizeof p);
    p.kind = JOB_PROJECTED_DECODE;
    p.u.pd.codes = codes; p.u.pd.codes_ld = codes_ld; p.u.pd.books = books;
    p.u.pd.w_out = w_out; p.u.pd.b_out = b_out;
    p.u.pd.n_stages = n_stages; p.u.pd.n_codes = n_codes; p.u.pd.dim = dim; p.u.pd.hidden = hidden;
    p.u.pd.out = out;
    return run_parallel(p, n_frames, pick_threads(threads, n_frames));
}
