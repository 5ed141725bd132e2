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
 *
 * Precision (the pages fix only that the codec is kept in F32):
 *   - distances: float64, direct form sum_j (r_j - c_j)^2, j ascending,
 *     one rounding per operation (built with -ffp-contract=off);
 *   - residual: float32, r_j <- fl32(r_j - c_j);
 *   - decode accumulator: float32, stage order ascending;
 *   - linear: float64 sum, i ascending, bias added last, rounded once.
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
            int32_t k1 = 0;
            double d1 = sq_dist(r, book, jb->dim);
            double d2 = INFINITY;
            for (int32_t k = 1; k < jb->n_codes; ++k) {
                double dk = sq_dist(r, book + (int64_t)k * jb->dim, jb->dim);
                if (dk < d1) {
                    d2 = d1;
                    d1 = dk;
                    k1 = k;
                } else if (dk < d2) {
                    d2 = dk;
                }
            }
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
    for (int64_t n = jb->begin; n < jb->end; ++n) {
        const float *hn = jb->h + n * jb->in_dim;
        for (int32_t o = 0; o < jb->out_dim; ++o) {
            const float *wo = jb->w + (int64_t)o * jb->in_dim;
            double s = 0.0;
            for (int32_t i = 0; i < jb->in_dim; ++i) s = s + (double)hn[i] * (double)wo[i];
            if (jb->b) s = s + (double)jb->b[o];
            jb->y[n * jb->out_dim + o] = (float)s;
        }
    }
}

/* ---- threading: contiguous frame ranges, one pthread each ------------- */

enum { JOB_ENCODE, JOB_DECODE, JOB_LINEAR };

typedef struct {
    int kind;
    union {
        encode_job e;
        decode_job d;
        linear_job l;
    } u;
} any_job;

static void *run_job(void *p)
{
    any_job *j = (any_job *)p;
    if (j->kind == JOB_ENCODE) encode_frames(&j->u.e);
    else if (j->kind == JOB_DECODE) decode_frames(&j->u.d);
    else linear_rows(&j->u.l);
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
        else { jobs[i].u.l.begin = b; jobs[i].u.l.end = e; }
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
