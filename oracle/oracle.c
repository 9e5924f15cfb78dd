/*
 * oracle.c - the CPU oracle for the lower-triangular solve.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may call,
 * link or load this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code with the HIP library.
 *
 * What it computes. The operation on the pages is the left-side,
 * lower-triangular, non-transposed, non-unit-diagonal TRSM on a square matrix
 * (HSMA-TRSM news summary, first paragraph: "left-side lower-triangular case";
 * llama.cpp PR #17457, the SOLVE_TRI kernel, which solves the same system by
 * substitution row after row). With A_L the lower triangle of the stored A,
 * diagonal included, the result is
 *
 *     X = A_L^{-1} (alpha * B),
 *
 * and the stored upper triangle is never read. The blocked method of the
 * HSMA-TRSM paper (inverted diagonal blocks, then GEMM updates of the
 * trailing rows) reaches the same X in exact arithmetic, so the oracle is the
 * plain definition: forward substitution,
 *
 *     x_i = (alpha*b_i - sum_{j<i} a_ij x_j) / a_ii,   i = 0 .. m-1,
 *
 * for each right-hand-side column, carried out in double precision (complex:
 * pairs of doubles) on inputs of any of the four storage types. Terms are
 * subtracted in increasing j. The pages call the same recurrence
 * "back-substitution" (HSMA-TRSM paper, the diagonal-block inversion
 * paragraphs); for a lower triangle it runs top to bottom.
 *
 * Conventions where the pages are silent (each is listed with the other
 * readings of the pages in the design notes):
 *   - alpha scales B before the solve; the pages never mention alpha.
 *   - no check for a zero diagonal: IEEE inf/NaN propagate (the SOLVE_TRI
 *     thread removed its division guard, PR #17457 review discussion).
 *   - complex division uses the textbook formula
 *       (w / d) = ((wr*dr + wi*di) + i(wi*dr - wr*di)) / (dr^2 + di^2).
 *   - built with -O2 -ffp-contract=off: no fused multiply-add, so results do
 *     not depend on the host compiler's contraction choices.
 *
 * Layout: element (i, j) of problem b of A is at A[b*sab + i*sai + j*saj],
 * in units of the storage element (a complex number counts as one). This
 * covers column-major BLAS storage (sai = 1, saj = lda) and the row-major
 * ggml storage (sai = row stride, saj = 1) with one routine. X is written in
 * double, column-major with leading dimension m, problems back to back;
 * complex X interleaves real and imaginary parts.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F64 = 1, OR_C64 = 2, OR_C128 = 3 };

static int cplx_of(int dtype) { return dtype == OR_C64 || dtype == OR_C128; }

/* Read element idx (in element units) of a typed array as a (re, im) double pair. */
static void get(int dtype, const void *p, int64_t idx, double *re, double *im)
{
    switch (dtype) {
    case OR_F32: *re = ((const float *)p)[idx]; *im = 0.0; break;
    case OR_F64: *re = ((const double *)p)[idx]; *im = 0.0; break;
    case OR_C64: *re = ((const float *)p)[2 * idx]; *im = ((const float *)p)[2 * idx + 1]; break;
    default: *re = ((const double *)p)[2 * idx]; *im = ((const double *)p)[2 * idx + 1]; break;
    }
}

typedef struct {
    int dtype;
    int64_t m, n;
    double ar, ai;
    const void *A; int64_t sai, saj, sab;
    const void *B; int64_t sbi, sbj, sbb;
    double *X;
    int64_t lo, hi; /* range of (problem * n + column) items */
} solve_job;

/* One column c of problem b, column-oriented forward substitution:
 * w := alpha*b; for j: x_j = w_j / a_jj; w_i -= a_ij * x_j for i > j.
 * Every w_i accumulates its terms in increasing j, the same order as the
 * row-oriented recurrence above. */
static void solve_column(const solve_job *J, int64_t b, int64_t c, double *w)
{
    const int cp = cplx_of(J->dtype);
    const int64_t m = J->m;
    for (int64_t i = 0; i < m; ++i) {
        double br, bi;
        get(J->dtype, J->B, b * J->sbb + i * J->sbi + c * J->sbj, &br, &bi);
        if (cp) {
            w[2 * i] = J->ar * br - J->ai * bi;
            w[2 * i + 1] = J->ar * bi + J->ai * br;
        } else {
            w[2 * i] = J->ar * br;
            w[2 * i + 1] = 0.0;
        }
    }
    for (int64_t j = 0; j < m; ++j) {
        double dr, di;
        get(J->dtype, J->A, b * J->sab + j * J->sai + j * J->saj, &dr, &di);
        double xr, xi;
        if (cp) {
            const double den = dr * dr + di * di;
            xr = (w[2 * j] * dr + w[2 * j + 1] * di) / den;
            xi = (w[2 * j + 1] * dr - w[2 * j] * di) / den;
        } else {
            xr = w[2 * j] / dr;
            xi = 0.0;
        }
        w[2 * j] = xr;
        w[2 * j + 1] = xi;
        for (int64_t i = j + 1; i < m; ++i) {
            double ar, ai;
            get(J->dtype, J->A, b * J->sab + i * J->sai + j * J->saj, &ar, &ai);
            if (cp) {
                w[2 * i] -= ar * xr - ai * xi;
                w[2 * i + 1] -= ar * xi + ai * xr;
            } else {
                w[2 * i] -= ar * xr;
            }
        }
    }
    double *x = J->X + (b * J->n + c) * m * (cp ? 2 : 1);
    for (int64_t i = 0; i < m; ++i) {
        if (cp) { x[2 * i] = w[2 * i]; x[2 * i + 1] = w[2 * i + 1]; }
        else x[i] = w[2 * i];
    }
}

static void *solve_run(void *arg)
{
    const solve_job *J = (const solve_job *)arg;
    double *w = (double *)malloc(sizeof(double) * 2 * (size_t)(J->m > 0 ? J->m : 1));
    if (!w) return (void *)1;
    for (int64_t it = J->lo; it < J->hi; ++it) solve_column(J, it / J->n, it % J->n, w);
    free(w);
    return 0;
}

/*
 * Solve batch independent problems A_b X_b = alpha B_b (see the header
 * comment for strides and the X layout). alpha is {re, im} (im ignored for
 * real types). Threads split the (problem, column) items into contiguous
 * ranges; a column's arithmetic never depends on the split, so the result
 * is bitwise the same for any thread count.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_trsm(int dtype, int64_t m, int64_t n, int64_t batch, const double *alpha,
                const void *A, int64_t sai, int64_t saj, int64_t sab,
                const void *B, int64_t sbi, int64_t sbj, int64_t sbb,
                double *X, int nthreads)
{
    if (dtype < 0 || dtype > 3 || m < 0 || n < 0 || batch < 0 || !alpha) return -1;
    const int64_t items = batch * n;
    if (m == 0 || items == 0) return 0;
    if (!A || !B || !X) return -1;
    solve_job base;
    memset(&base, 0, sizeof base);
    base.dtype = dtype; base.m = m; base.n = n;
    base.ar = alpha[0]; base.ai = cplx_of(dtype) ? alpha[1] : 0.0;
    base.A = A; base.sai = sai; base.saj = saj; base.sab = sab;
    base.B = B; base.sbi = sbi; base.sbj = sbj; base.sbb = sbb;
    base.X = X;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (items < nthreads) nthreads = (int)items;
    solve_job *jobs = (solve_job *)malloc(sizeof(solve_job) * (size_t)nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].lo = items * t / nthreads;
        jobs[t].hi = items * (t + 1) / nthreads;
    }
    int bad = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], 0, solve_run, &jobs[t]) != 0) { jobs[t].hi = jobs[t].lo; bad = 1; }
    if (solve_run(&jobs[0])) bad = 1;
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].hi == jobs[t].lo && bad) continue;
        void *r = 0;
        pthread_join(th[t], &r);
        if (r) bad = 1;
    }
    free(jobs); free(th);
    return bad ? -1 : 0;
}

/*
 * Plain product C = A * B in double, for checking the library's matrix-
 * multiply building block on its own. A is M x K, B is K x N, both typed and
 * addressed as (i, j) -> p[i*si + j*sj]; C is double, column-major M x N
 * (complex interleaved). Sums run over k in increasing order. This is not a
 * step of the solve's definition; it exists so the library's GEMM kernel can
 * be compared against an independent product.
 */
int oracle_gemm(int dtype, int64_t M, int64_t N, int64_t K,
                const void *A, int64_t sai, int64_t saj,
                const void *B, int64_t sbi, int64_t sbj, double *C)
{
    if (dtype < 0 || dtype > 3 || M < 0 || N < 0 || K < 0) return -1;
    const int cp = cplx_of(dtype);
    for (int64_t j = 0; j < N; ++j)
        for (int64_t i = 0; i < M; ++i) {
            double sr = 0.0, si = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double ar, ai, br, bi;
                get(dtype, A, i * sai + k * saj, &ar, &ai);
                get(dtype, B, k * sbi + j * sbj, &br, &bi);
                sr += ar * br - ai * bi;
                si += ar * bi + ai * br;
            }
            if (cp) { C[2 * (i + j * M)] = sr; C[2 * (i + j * M) + 1] = si; }
            else C[i + j * M] = sr;
        }
    return 0;
}

/*
 * The other TRSM variants (side, triangle, transpose, unit diagonal), by
 * definition. The HSMA-TRSM pages evaluate only the left-side lower case and
 * leave "other TRSM variants" open (news summary, "A result tied to a narrow
 * benchmark"); the variants here are the usual BLAS ones:
 *
 *   side left:   op(A) X = alpha B,  A is m x m
 *   side right:  X op(A) = alpha B,  A is n x n
 *   op(A) = A (trans 0), A^T (trans 1) or A^H (trans 2, conjugate transpose);
 *   uplo 0: A lower triangular, 1: upper (the other triangle is never read);
 *   diag 1: unit diagonal, op(A)(i, i) = 1 and the stored diagonal is never read.
 *
 * Each system is solved by substitution in the order its triangle allows:
 * left side, op(A) lower: x_i = (alpha b_i - sum_{j<i} op(A)(i,j) x_j) / op(A)(i,i)
 * for i = 0, 1, ...; op(A) upper: the same with j > i for i = m-1, m-2, ...
 * Right side, row r of B: sum_k x_k op(A)(k, j) = alpha b_j, so op(A) upper
 * gives x_j = (alpha b_j - sum_{k<j} x_k op(A)(k,j)) / op(A)(j,j) for
 * j = 0, 1, ..., and op(A) lower the same with k > j, j descending. Sums run
 * over the already solved unknowns in the order they were solved. Complex
 * products and the textbook complex division in double, as above.
 *
 * X is written in double, column-major m x n per problem (leading dimension
 * m), problems back to back, as for oracle_trsm.
 */
typedef struct {
    int dtype, side, uplo, trans, diag;
    int64_t m, n, k; /* k = order of A: m (left) or n (right) */
    double ar, ai;
    const void *A; int64_t sai, saj, sab;
    const void *B; int64_t sbi, sbj, sbb;
    double *X;
    int64_t lo, hi; /* range of (problem * vectors + vector) items */
} general_job;

/* op(A)(i, j) of problem b as a (re, im) pair. */
static void op_a(const general_job *J, int64_t b, int64_t i, int64_t j, double *re, double *im)
{
    if (J->diag == 1 && i == j) { *re = 1.0; *im = 0.0; return; }
    const int64_t r = J->trans ? j : i;   /* element of the stored A */
    const int64_t c = J->trans ? i : j;
    get(J->dtype, J->A, b * J->sab + r * J->sai + c * J->saj, re, im);
    if (J->trans == 2) *im = -*im;
}

/* (pr, pi) = (ar, ai) * (br, bi) */
static void cprod(double ar, double ai, double br, double bi, double *pr, double *pi)
{
    *pr = ar * br - ai * bi;
    *pi = ar * bi + ai * br;
}

/* One right-hand-side vector: column c (left side) or row c (right side). */
static void solve_vector(const general_job *J, int64_t b, int64_t c, double *x)
{
    const int left = J->side == 0;
    const int64_t k = J->k;
    /* op(A) lower iff (A lower and not transposed) or (A upper and transposed) */
    const int op_lower = (J->uplo == 0) == (J->trans == 0);
    /* substitution runs forward when the unknown of step s only needs earlier ones */
    const int forward = left ? op_lower : !op_lower;
    for (int64_t s = 0; s < k; ++s) {
        const int64_t i = forward ? s : k - 1 - s;
        double br, bi;
        const int64_t row = left ? i : c, col = left ? c : i;
        get(J->dtype, J->B, b * J->sbb + row * J->sbi + col * J->sbj, &br, &bi);
        double accr, acci;
        cprod(J->ar, cplx_of(J->dtype) ? J->ai : 0.0, br, bi, &accr, &acci);
        for (int64_t t = 0; t < s; ++t) {
            const int64_t j = forward ? t : k - 1 - t;   /* solved unknowns, in solve order */
            double opr, opi, pr, pi;
            if (left) op_a(J, b, i, j, &opr, &opi);      /* op(A)(i, j) x_j */
            else op_a(J, b, j, i, &opr, &opi);           /* x_j op(A)(j, i) */
            cprod(opr, opi, x[2 * j], x[2 * j + 1], &pr, &pi);
            accr -= pr;
            acci -= pi;
        }
        double dr, di;
        op_a(J, b, i, i, &dr, &di);
        if (cplx_of(J->dtype)) {
            const double den = dr * dr + di * di;
            x[2 * i] = (accr * dr + acci * di) / den;
            x[2 * i + 1] = (acci * dr - accr * di) / den;
        } else {
            x[2 * i] = accr / dr;
            x[2 * i + 1] = 0.0;
        }
    }
    /* store: X(row, col) of problem b, column-major with leading dimension m */
    const int cp = cplx_of(J->dtype);
    double *Xb = J->X + b * J->m * J->n * (cp ? 2 : 1);
    for (int64_t i = 0; i < k; ++i) {
        const int64_t row = left ? i : c, col = left ? c : i;
        const int64_t at = row + col * J->m;
        if (cp) { Xb[2 * at] = x[2 * i]; Xb[2 * at + 1] = x[2 * i + 1]; }
        else Xb[at] = x[2 * i];
    }
}

static void *general_run(void *arg)
{
    const general_job *J = (const general_job *)arg;
    double *x = (double *)malloc(sizeof(double) * 2 * (size_t)(J->k > 0 ? J->k : 1));
    if (!x) return (void *)1;
    const int64_t per = J->side == 0 ? J->n : J->m;
    for (int64_t it = J->lo; it < J->hi; ++it) solve_vector(J, it / per, it % per, x);
    free(x);
    return 0;
}

/*
 * Solve batch problems of one variant (codes above). A: element (i, j) of
 * problem b at A[b*sab + i*sai + j*saj], order m (left) or n (right); B and
 * X as for oracle_trsm. Returns 0, or -1 on a bad argument or allocation
 * failure. Bitwise independent of the thread count.
 */
int oracle_trsm_general(int dtype, int side, int uplo, int trans, int diag, int64_t m, int64_t n,
                        int64_t batch, const double *alpha,
                        const void *A, int64_t sai, int64_t saj, int64_t sab,
                        const void *B, int64_t sbi, int64_t sbj, int64_t sbb,
                        double *X, int nthreads)
{
    if (dtype < 0 || dtype > 3 || side < 0 || side > 1 || uplo < 0 || uplo > 1 || trans < 0 ||
        trans > 2 || diag < 0 || diag > 1 || m < 0 || n < 0 || batch < 0 || !alpha)
        return -1;
    const int64_t per = side == 0 ? n : m;
    const int64_t items = batch * per;
    if (m == 0 || n == 0 || items == 0) return 0;
    if (!A || !B || !X) return -1;
    general_job base;
    memset(&base, 0, sizeof base);
    base.dtype = dtype; base.side = side; base.uplo = uplo; base.trans = trans; base.diag = diag;
    base.m = m; base.n = n; base.k = side == 0 ? m : n;
    base.ar = alpha[0]; base.ai = cplx_of(dtype) ? alpha[1] : 0.0;
    base.A = A; base.sai = sai; base.saj = saj; base.sab = sab;
    base.B = B; base.sbi = sbi; base.sbj = sbj; base.sbb = sbb;
    base.X = X;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (items < nthreads) nthreads = (int)items;
    general_job *jobs = (general_job *)malloc(sizeof(general_job) * (size_t)nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int *started = (int *)calloc((size_t)nthreads, sizeof(int));
    if (!jobs || !th || !started) { free(jobs); free(th); free(started); return -1; }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].lo = items * t / nthreads;
        jobs[t].hi = items * (t + 1) / nthreads;
    }
    int bad = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], 0, general_run, &jobs[t]) == 0) started[t] = 1;
        else bad = 1;
    }
    if (general_run(&jobs[0])) bad = 1;
    for (int t = 1; t < nthreads; ++t) {
        if (!started[t]) continue;
        void *r = 0;
        pthread_join(th[t], &r);
        if (r) bad = 1;
    }
    free(jobs); free(th); free(started);
    return bad ? -1 : 0;
}
