/*
 * synth.c - seeded synthetic inputs for the triangular solve A*X = alpha*B.
 *
 * This module only draws numbers. It holds none of the solve's arithmetic and
 * is the one piece of code that both the CPU oracle (oracle/) and the HIP
 * library's tests and benchmark use: each side receives the same arrays.
 *
 * Workload recipe (the pages test square, random-valued lower-triangular
 * systems; HSMA-TRSM news summary, "One framework, several paths"; the
 * distributions themselves are this project's choice, stated once here):
 *   - A, strictly below the diagonal:  (2u - 1) / offdiag_div
 *   - A, on the diagonal:               1 + u
 *   - A, above the diagonal:            a quiet NaN ("garbage"; a correct
 *                                       solver never reads it)
 *   - B:                                2u - 1
 * with u uniform on [0, 1). Complex elements draw real and imaginary parts
 * independently from the same law. Every value is computed in double and
 * rounded once to the storage type.
 *
 * Generator: SplitMix64's output mixing function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants
 * as in Vigna's public-domain reference splitmix64.c), applied to a counter
 * built from (seed, tag, batch, i, j, part). A value depends only on those
 * logical coordinates, never on the memory layout, leading dimension or
 * thread count that wrote it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

enum { SYNTH_F32 = 0, SYNTH_F64 = 1, SYNTH_C64 = 2, SYNTH_C128 = 3 };

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

#define GOLDEN 0x9e3779b97f4a7c15ULL

/* u in [0,1) with 53 random bits, for logical coordinates. */
static double unit(uint64_t seed, uint64_t tag, uint64_t b, uint64_t i, uint64_t j, uint64_t part)
{
    uint64_t h = mix64(seed + GOLDEN * (tag + 1));
    h = mix64(h + GOLDEN * (b + 1));
    h = mix64(h ^ (i * 0x100000001b3ULL + 0x51));
    h = mix64(h + GOLDEN * (j * 2 + part + 1));
    return (double)(h >> 11) * 0x1.0p-53;
}

static int is_complex(int dtype) { return dtype == SYNTH_C64 || dtype == SYNTH_C128; }

static void store(int dtype, void *out, int64_t off, double re, double im)
{
    switch (dtype) {
    case SYNTH_F32: ((float *)out)[off] = (float)re; break;
    case SYNTH_F64: ((double *)out)[off] = re; break;
    case SYNTH_C64: ((float *)out)[2 * off] = (float)re; ((float *)out)[2 * off + 1] = (float)im; break;
    case SYNTH_C128: ((double *)out)[2 * off] = re; ((double *)out)[2 * off + 1] = im; break;
    }
}

typedef struct {
    int kind; /* 0: triangular A, 1: right-hand side B */
    int dtype;
    int64_t m, n, batch;
    double offdiag_div;
    uint64_t seed, tag;
    void *out;
    int64_t rs, cs, bs; /* element strides: row, column, batch */
    const int64_t *cols;
    int upper_mode; /* 0: NaN above the diagonal, 1: zero, 2: leave untouched */
    int64_t lo, hi;  /* range of (batch * ncols) work items */
} job_t;

static void *run(void *arg)
{
    const job_t *J = (const job_t *)arg;
    const int cplx = is_complex(J->dtype);
    const int64_t ncols = J->kind == 0 ? J->m : J->n;
    for (int64_t w = J->lo; w < J->hi; ++w) {
        const int64_t b = w / ncols, c = w % ncols;
        const int64_t lc = (J->kind == 1 && J->cols) ? J->cols[c] : c; /* logical column */
        for (int64_t i = 0; i < J->m; ++i) {
            const int64_t off = b * J->bs + i * J->rs + c * J->cs;
            double re, im = 0.0;
            if (J->kind == 1) {
                re = 2.0 * unit(J->seed, J->tag, b, i, lc, 0) - 1.0;
                if (cplx) im = 2.0 * unit(J->seed, J->tag, b, i, lc, 1) - 1.0;
            } else if (i > c) {
                re = (2.0 * unit(J->seed, J->tag, b, i, c, 0) - 1.0) / J->offdiag_div;
                if (cplx) im = (2.0 * unit(J->seed, J->tag, b, i, c, 1) - 1.0) / J->offdiag_div;
            } else if (i == c) {
                re = 1.0 + unit(J->seed, J->tag, b, i, c, 0);
                if (cplx) im = 1.0 + unit(J->seed, J->tag, b, i, c, 1);
            } else {
                if (J->upper_mode == 2) continue;
                re = J->upper_mode == 0 ? NAN : 0.0;
                im = re;
            }
            store(J->dtype, J->out, off, re, im);
        }
    }
    return 0;
}

static void launch(job_t base, int64_t items, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (items < nthreads) nthreads = items > 0 ? (int)items : 1;
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].lo = items * t / nthreads;
        jobs[t].hi = items * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], 0, run, &jobs[t]);
    run(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], 0);
}

/* Lower-triangular A: batch problems of size m x m. Element (b, i, j) is
 * written at out[b*bs + i*rs + j*cs] (complex: that index in complex units). */
void synth_fill_tri(int dtype, int64_t m, int64_t batch, double offdiag_div, uint64_t seed,
                    uint64_t tag, void *out, int64_t rs, int64_t cs, int64_t bs, int upper_mode,
                    int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.kind = 0; J.dtype = dtype; J.m = m; J.n = m; J.batch = batch;
    J.offdiag_div = offdiag_div; J.seed = seed; J.tag = tag; J.out = out;
    J.rs = rs; J.cs = cs; J.bs = bs; J.upper_mode = upper_mode;
    launch(J, batch * m, nthreads);
}

/* Right-hand side B: batch blocks of m x n. Output column c holds logical
 * column cols[c] (or c when cols is NULL), so a column subset of a large B
 * can be drawn without drawing the rest. */
void synth_fill_rhs(int dtype, int64_t m, int64_t n, int64_t batch, uint64_t seed, uint64_t tag,
                    void *out, int64_t rs, int64_t cs, int64_t bs, const int64_t *cols,
                    int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.kind = 1; J.dtype = dtype; J.m = m; J.n = n; J.batch = batch;
    J.seed = seed; J.tag = tag; J.out = out; J.rs = rs; J.cs = cs; J.bs = bs; J.cols = cols;
    launch(J, batch * n, nthreads);
}

/* k distinct indices from [0, n), sorted ascending: a partial Fisher-Yates
 * shuffle driven by the same counter-based generator. work has n slots. */
void synth_pick(int64_t n, int64_t k, uint64_t seed, int64_t *work, int64_t *out)
{
    for (int64_t i = 0; i < n; ++i) work[i] = i;
    for (int64_t i = 0; i < k; ++i) {
        const double u = unit(seed, 0x636f6c73ULL /* "cols" */, 0, (uint64_t)i, 0, 0);
        int64_t r = i + (int64_t)(u * (double)(n - i));
        if (r >= n) r = n - 1;
        const int64_t t = work[i]; work[i] = work[r]; work[r] = t;
    }
    for (int64_t i = 0; i < k; ++i) out[i] = work[i];
    /* insertion sort: k is small */
    for (int64_t i = 1; i < k; ++i) {
        const int64_t v = out[i];
        int64_t j = i - 1;
        while (j >= 0 && out[j] > v) { out[j + 1] = out[j]; --j; }
        out[j + 1] = v;
    }
}

/* The raw 64-bit hash, exported so tests can check it against the published
 * SplitMix64 reference outputs. */
uint64_t synth_mix64(uint64_t z) { return mix64(z); }
