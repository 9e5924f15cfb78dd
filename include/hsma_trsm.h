/*
 * hsma_trsm.h - C ABI of the MI355X (gfx950) triangular-solve library.
 *
 * The operation is the left-side, lower-triangular, non-transposed,
 * non-unit-diagonal TRSM on a square matrix (HSMA-TRSM news summary, first
 * paragraph: "the left-side lower-triangular case, run with square matrices"):
 *
 *     solve  A * X = alpha * B   for X,  X overwrites B,
 *
 * where only the lower triangle of A, diagonal included, is read; the stored
 * upper triangle may hold anything (NaN included) and is never read.
 * Two regimes follow the HSMA-TRSM paper: m <= 64 is solved directly on chip
 * (the paper's small-scale section), larger m by blocked TRSM whose diagonal
 * blocks are inverted in parallel and applied with matrix-multiply updates
 * (the paper's blocked section and its adaptive block size).
 *
 * Conventions for every entry point:
 *   - Storage is column-major unless stated: element (i, j) of A is at
 *     A[i + j*lda]. Sizes and strides are counted in elements (a complex
 *     number is one element), never in bytes.
 *   - Pointers are device pointers (HBM). The caller owns all of A, B and X;
 *     the library never keeps them after the call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream). They return once the work is enqueued. A kernel fault surfaces
 *     at the caller's next synchronisation.
 *   - Workspace for the blocked path is allocated stream-ordered on `stream`
 *     (hipMallocFromPoolAsync / hipFreeAsync), so calls on different streams
 *     do not share memory. It comes from a memory pool the library creates
 *     once per device and keeps until the process ends; freed workspace stays
 *     in that pool for the next call (its size is at most the largest
 *     workspace used so far) instead of being returned to the driver.
 *   - The blocked path also runs some copies on a second stream the library
 *     creates once per device (non-blocking, default priority, kept until
 *     the process ends), ordered against `stream` with events: `stream`
 *     waits for them before the call's work on it ends, so a call remains
 *     one ordered piece of work on `stream`.
 *   - No singularity check: a zero or NaN diagonal entry produces inf/NaN
 *     under IEEE rules (the SOLVE_TRI review in llama.cpp PR #17457 dropped
 *     its zero-pivot guard for the same reason). Pivots are applied as
 *     reciprocals, x_j = w_j * (1/a_jj): a zero pivot gives +-inf (NaN where
 *     w_j is 0 or the pivot is complex) in its row and non-finite values in
 *     every row below it, in every path. A pivot whose reciprocal overflows
 *     (|a_jj| < 2^-1024 in double; subnormal float pivots) acts like a zero
 *     pivot. Complex reciprocals are scaled (Smith's method), so they hold
 *     over the whole exponent range.
 *   - The environment variable HSMA_TEST_FAIL_ALLOC=1 makes every workspace
 *     allocation fail: such calls return ALLOC_FAILED before any GPU work
 *     (for tests of that error path).
 *   - m == 0, n == 0 or batch_count == 0: success, no memory touched.
 *     alpha == 0: B is set to zero and A is not read.
 *   - No C++ exception crosses this interface.
 */
#ifndef HSMA_TRSM_H
#define HSMA_TRSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int hsma_status;
#define HSMA_STATUS_SUCCESS 0
#define HSMA_STATUS_INVALID_SIZE 1    /* negative size, leading dimension too small, overlapping outputs */
#define HSMA_STATUS_INVALID_POINTER 2 /* NULL A, B or X where data must be read or written */
#define HSMA_STATUS_NOT_SUPPORTED 3   /* shape outside what this entry point handles */
#define HSMA_STATUS_ALLOC_FAILED 4    /* workspace allocation failed */
#define HSMA_STATUS_HIP_ERROR 5       /* a HIP runtime call or kernel launch failed */
#define HSMA_STATUS_INVALID_VALUE 6   /* bad option value */
#define HSMA_STATUS_SCRATCH_TOO_SMALL 7 /* hsma_trsm_noalloc: problem exceeds its fixed scratch */

typedef struct { float re, im; } hsma_float_complex;
typedef struct { double re, im; } hsma_double_complex;

/* Element-type codes used by the helpers below. */
#define HSMA_DTYPE_F32 0
#define HSMA_DTYPE_F64 1
#define HSMA_DTYPE_C64 2
#define HSMA_DTYPE_C128 3

/*
 * hsma_trsm_{s,d,c,z}: one m x m system with n right-hand sides.
 *   m     order of A (m >= 0); n: number of columns of B (n >= 0)
 *   alpha scalar applied to B before the solve
 *   A     device pointer, lda >= max(1, m); read-only, lower triangle only
 *   B     device pointer, ldb >= max(1, m); on return holds X
 * Route: m <= 64 the small regime (one launch); 64 < m <= 192 with n <= 16
 * block rows of 64 (as the strided-batched entry points below, no
 * workspace); otherwise the blocked solver.
 * Errors: INVALID_SIZE, INVALID_POINTER (A or B NULL with m*n > 0),
 *         ALLOC_FAILED, HIP_ERROR.
 */
hsma_status hsma_trsm_s(int64_t m, int64_t n, float alpha, const float *A, int64_t lda,
                        float *B, int64_t ldb, void *stream);
hsma_status hsma_trsm_d(int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                        double *B, int64_t ldb, void *stream);
hsma_status hsma_trsm_c(int64_t m, int64_t n, hsma_float_complex alpha,
                        const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                        int64_t ldb, void *stream);
hsma_status hsma_trsm_z(int64_t m, int64_t n, hsma_double_complex alpha,
                        const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                        int64_t ldb, void *stream);

/*
 * hsma_trsm_strided_batched_{s,d,c,z}: batch_count independent systems;
 * problem b uses A + b*strideA and B + b*strideB (strides in elements).
 * The batched use case is llama.cpp's SOLVE_TRI (PR #17457, "SOLVE_TRI CUDA
 * kernel for small matrices": one small system per batch index, solved by one
 * thread block each); the HSMA-TRSM paper's small-scale section gives the
 * per-problem method (the triangle on chip, direct solve).
 * strideA == 0 shares one A across the batch. B blocks must not overlap:
 * strideB >= ldb*n when batch_count > 1 (else INVALID_SIZE).
 * m <= 64 runs as one launch over the whole batch (the pages' small regime);
 * 64 < m <= 512 runs in block rows of 64 over the whole batch (per block row
 * one batched GEMM update with the finished rows and one batched small-regime
 * solve of the diagonal blocks); larger m runs the blocked solver once per
 * problem.
 * Errors: as hsma_trsm_*; ALLOC_FAILED only for m > 512.
 */
hsma_status hsma_trsm_strided_batched_s(int64_t m, int64_t n, float alpha, const float *A,
                                        int64_t lda, int64_t strideA, float *B, int64_t ldb,
                                        int64_t strideB, int64_t batch_count, void *stream);
hsma_status hsma_trsm_strided_batched_d(int64_t m, int64_t n, double alpha, const double *A,
                                        int64_t lda, int64_t strideA, double *B, int64_t ldb,
                                        int64_t strideB, int64_t batch_count, void *stream);
hsma_status hsma_trsm_strided_batched_c(int64_t m, int64_t n, hsma_float_complex alpha,
                                        const hsma_float_complex *A, int64_t lda, int64_t strideA,
                                        hsma_float_complex *B, int64_t ldb, int64_t strideB,
                                        int64_t batch_count, void *stream);
hsma_status hsma_trsm_strided_batched_z(int64_t m, int64_t n, hsma_double_complex alpha,
                                        const hsma_double_complex *A, int64_t lda, int64_t strideA,
                                        hsma_double_complex *B, int64_t ldb, int64_t strideB,
                                        int64_t batch_count, void *stream);

/*
 * hsma_trsm_general_{s,d,c,z} and hsma_trsm_strided_batched_general_{s,d,c,z}:
 * the other TRSM variants, which the HSMA-TRSM pages leave untested (news
 * summary, "A result tied to a narrow benchmark": nonsquare shapes and
 * other TRSM variants remain unresolved), with the usual BLAS meaning:
 *   side HSMA_SIDE_LEFT:   op(A) X = alpha B,  A is m x m
 *   side HSMA_SIDE_RIGHT:  X op(A) = alpha B,  A is n x n
 *   uplo HSMA_FILL_LOWER / HSMA_FILL_UPPER: the triangle of A that is used
 *        (the other one is never read)
 *   trans HSMA_OP_N: op(A) = A; HSMA_OP_T: A^T; HSMA_OP_C: A^H (conjugate
 *        transpose; the same as HSMA_OP_T for real types)
 *   diag HSMA_DIAG_UNIT: a unit diagonal is assumed and the stored diagonal
 *        is never read; HSMA_DIAG_NON_UNIT: the stored diagonal is used
 * B is m x n with ldb >= max(1, m); lda >= max(1, order of A). X overwrites
 * B; m != n is allowed everywhere. side LEFT, uplo LOWER, trans N, diag
 * NON_UNIT is exactly hsma_trsm_* (hsma_trsm_strided_batched_*).
 * Every variant is solved as the canonical left-side lower-triangular
 * system C Y = alpha Bhat, with C = op(A) (left) or op(A)^T (right), taken
 * in reverse index order when it is upper triangular, and Bhat = B or B^T
 * (rows reversed with C). For an order of at most 64 the small regime
 * reads these as strided views (lane-per-row kernel); batches of order
 * 64 < k <= 256 gather the triangles and right-hand sides of the whole batch
 * into workspace and run in block rows of 64; larger orders gather one
 * problem at a time and run the blocked solver on the copy, then X is
 * scattered back. The gathers take workspace (k*k, plus m*n unless Bhat is
 * B itself); ALLOC_FAILED if it cannot be had.
 * Errors: INVALID_VALUE (bad side/uplo/trans/diag code), INVALID_SIZE,
 *         INVALID_POINTER, ALLOC_FAILED, HIP_ERROR.
 */
#define HSMA_SIDE_LEFT 0
#define HSMA_SIDE_RIGHT 1
#define HSMA_FILL_LOWER 0
#define HSMA_FILL_UPPER 1
#define HSMA_OP_N 0
#define HSMA_OP_T 1
#define HSMA_OP_C 2
#define HSMA_DIAG_NON_UNIT 0
#define HSMA_DIAG_UNIT 1

hsma_status hsma_trsm_general_s(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, float alpha, const float *A, int64_t lda,
                                float *B, int64_t ldb, void *stream);
hsma_status hsma_trsm_general_d(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                                double *B, int64_t ldb, void *stream);
hsma_status hsma_trsm_general_c(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, hsma_float_complex alpha,
                                const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                                int64_t ldb, void *stream);
hsma_status hsma_trsm_general_z(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, hsma_double_complex alpha,
                                const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                                int64_t ldb, void *stream);
hsma_status hsma_trsm_strided_batched_general_s(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n, float alpha,
                                                const float *A, int64_t lda, int64_t strideA,
                                                float *B, int64_t ldb, int64_t strideB,
                                                int64_t batch_count, void *stream);
hsma_status hsma_trsm_strided_batched_general_d(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n, double alpha,
                                                const double *A, int64_t lda, int64_t strideA,
                                                double *B, int64_t ldb, int64_t strideB,
                                                int64_t batch_count, void *stream);
hsma_status hsma_trsm_strided_batched_general_c(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n,
                                                hsma_float_complex alpha,
                                                const hsma_float_complex *A, int64_t lda,
                                                int64_t strideA, hsma_float_complex *B,
                                                int64_t ldb, int64_t strideB, int64_t batch_count,
                                                void *stream);
hsma_status hsma_trsm_strided_batched_general_z(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n,
                                                hsma_double_complex alpha,
                                                const hsma_double_complex *A, int64_t lda,
                                                int64_t strideA, hsma_double_complex *B,
                                                int64_t ldb, int64_t strideB, int64_t batch_count,
                                                void *stream);

/*
 * hsma_solve_tri_f32: the ggml SOLVE_TRI operation (llama.cpp PR #17457,
 * "SOLVE_TRI CUDA kernel for small matrices"): for every batch index
 * (i2, i3) in [0, ne02) x [0, ne03), solve A X = B with A n x n lower
 * triangular and B, X n x k, out of place.
 * Layout is ggml's, row-major with the column index fastest:
 *   A(i, j) = A[i*sA1 + j + i2*sA2 + i3*sA3]
 *   B(i, c) = B[i*sB1 + c + i2*sB2 + i3*sB3]
 *   X(i, c) = X[i*sX1 + c + i2*sX2 + i3*sX3]
 * Strides are in elements (floats), as the PR's reviewers asked. B is
 * read-only; X must not overlap A or B.
 * n <= 256 (any k). One launch solves every batch entry on chip: up to 64
 * rows one wave per group of right-hand sides; above that one wave per block
 * of 64 rows (two, three or four), each block solved after the earlier ones
 * have passed their finished rows through LDS -- covering the [128,128,4,1]
 * case the PR's kernel reports as not supported.
 * n > 256 returns NOT_SUPPORTED.
 */
hsma_status hsma_solve_tri_f32(int64_t n, int64_t k, const float *A, const float *B, float *X,
                               int64_t ne02, int64_t ne03, int64_t sA1, int64_t sA2, int64_t sA3,
                               int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1, int64_t sX2,
                               int64_t sX3, void *stream);

/*
 * Options for the *_ex entry points (a NULL opts means all defaults). They
 * exist for the offline block-size sweep of the HSMA-TRSM paper's adaptive
 * blocking section (every candidate block size is run and timed on the
 * target GPU) and for tests of each route.
 *   nb    outer block size N_B of the blocked path (0: from the built-in
 *         table); must be a multiple of 16 in [16, 2048]; above 1024 (above
 *         512 for double complex) m must also be a multiple of nb, since
 *         such blocks are inverted only by the blocked-inverse formula
 *   ib    inner block I_B of the diagonal inversion (0: nb/8; must divide nb,
 *         nb/ib <= 64). The paper's I_B is the width of the identity tile a
 *         work unit substitutes against (blocked section). Here it only
 *         applies to the column-substitution route (m not a multiple of nb,
 *         or nb < 128): a work unit takes the largest power of two G <= 16
 *         (<= 8 for double and float complex, <= 4 for double complex; the
 *         register budget) that divides both ib and nb. The blocked-inverse
 *         route always starts from 64 x 64 sub-blocks (the small-regime
 *         solver's size) and ignores ib.
 *   path  HSMA_PATH_AUTO, HSMA_PATH_SMALL (requires m <= 64),
 *         HSMA_PATH_BLOCKED (any m >= 1) or HSMA_PATH_ROWS64 (m <= 512:
 *         block rows of 64, each updated by one matrix-core GEMM with the
 *         finished rows and solved by the small regime, no inversion and no
 *         workspace; what AUTO takes for batches with 64 < m <= 512
 *         and for single problems with 64 < m <= 192 and n <= 16)
 *   inv   route of the diagonal-block inversion (blocked path):
 *         HSMA_INV_AUTO: BLOCKED where it applies (for f64 and c64 only
 *           when nb > 128, for c128 when nb > 256), else COLUMN;
 *         HSMA_INV_BLOCKED: 64 x 64 sub-blocks by substitution against
 *           identity columns, merged by the block-inverse formula in batched
 *           matrix-core products (m a multiple of nb, nb a multiple of 64,
 *           nb >= 128);
 *         HSMA_INV_FUSED: the "traditional" fused kernel the paper's
 *           blocked section describes and replaces: each 2*ib x 2*ib
 *           diagonal block inverted whole in LDS (4*ib^2 elements), then the
 *           same merges up to nb (ib 32 or 64, 32 for double complex; m a
 *           multiple of nb, nb a multiple of 2*ib); an A/B alternative;
 *         HSMA_INV_COLUMN: column-level substitution against identity
 *           tiles (nb <= 1024).
 *         A route that does not apply to (m, nb, ib) gives INVALID_VALUE.
 *   Timing of the blocked path's phases (the paper's Table 3 splits the
 *   run time into diagonal inversion and GEMM update): when n_events > 0,
 *   events[0 .. n_events) are hipEvent_t handles created by the caller, and
 *   the library records events[k] on the stream at the start of each phase
 *   and once more at the end, writing the phase code (HSMA_PHASE_*) of the
 *   interval that starts at events[k] to event_phase[k] (HSMA_PHASE_END for
 *   the last event) and the number of events recorded to *events_used. The
 *   interval between events[k] and events[k+1] is then the time of phase
 *   event_phase[k]. A blocked solve records 3*ceil(m/nb) + 1 events, one
 *   more when alpha != 1; if n_events is smaller the call returns
 *   INVALID_VALUE before any work, with the number needed in *events_used.
 *   Events are recorded only by the blocked path (*events_used = 0 on the
 *   others). event_phase and events_used must be valid when n_events > 0.
 * Bad values return INVALID_VALUE.
 */
#define HSMA_PATH_AUTO 0
#define HSMA_PATH_SMALL 1
#define HSMA_PATH_BLOCKED 2
#define HSMA_PATH_ROWS64 3
#define HSMA_INV_AUTO 0
#define HSMA_INV_BLOCKED 1
#define HSMA_INV_FUSED 2
#define HSMA_INV_COLUMN 3
#define HSMA_PHASE_END (-1)
#define HSMA_PHASE_SCALE 0      /* B := alpha * B */
#define HSMA_PHASE_DIAG_INV 1   /* inversion of all diagonal blocks */
#define HSMA_PHASE_INV_GEMM 2   /* W = D_t^{-1} B_t */
#define HSMA_PHASE_COPY 3       /* W -> B_t */
#define HSMA_PHASE_TRAILING 4   /* B[below] -= A[below, t] X_t */
typedef struct {
    int32_t nb;
    int32_t ib;
    int32_t path;
    int32_t inv;
    int32_t n_events;
    void **events;
    int32_t *event_phase;
    int32_t *events_used;
} hsma_trsm_opts;

hsma_status hsma_trsm_ex_s(int64_t m, int64_t n, float alpha, const float *A, int64_t lda,
                           float *B, int64_t ldb, const hsma_trsm_opts *opts, void *stream);
hsma_status hsma_trsm_ex_d(int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                           double *B, int64_t ldb, const hsma_trsm_opts *opts, void *stream);
hsma_status hsma_trsm_ex_c(int64_t m, int64_t n, hsma_float_complex alpha,
                           const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                           int64_t ldb, const hsma_trsm_opts *opts, void *stream);
hsma_status hsma_trsm_ex_z(int64_t m, int64_t n, hsma_double_complex alpha,
                           const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                           int64_t ldb, const hsma_trsm_opts *opts, void *stream);

/*
 * Building blocks of the blocked path, exported so that each step can be
 * checked on its own.
 *
 * hsma_diag_inv_{s,d,c,z}: inverts every diagonal block of the lower
 * triangle of A (HSMA-TRSM paper, blocked section: the diagonal blocks D_t
 * are independent and are inverted in parallel, by substitution against
 * identity tiles). Block t covers rows/columns [t*nb, min(m, (t+1)*nb)).
 * invA receives ceil(m/nb) blocks of nb x nb, block t at invA + t*nb*nb,
 * column-major with leading dimension nb; entries above the diagonal, and
 * rows/columns beyond m in the last block, are written as exact zeros (the
 * padded part of the last block holds the identity on its diagonal).
 * nb, ib as in hsma_trsm_opts (0 = defaults). When m is a multiple of nb and
 * nb a multiple of 64 with nb >= 128 (f64 and c64: nb > 128; c128: nb > 256;
 * where this measured faster than the column route), 64 x 64 sub-blocks are inverted by
 * substitution against identity columns and merged by the block-inverse
 * formula with matrix-core products (ib unused; a temporary of nb*nb/4
 * elements per block comes from the library's workspace pool); otherwise
 * column-level substitution, one work unit per (diagonal block, group of G
 * identity columns) with G chosen from ib as described for hsma_trsm_opts
 * (nb <= 1024).
 * Either way the result is the block inverses up to rounding.
 */
hsma_status hsma_diag_inv_s(int64_t m, int32_t nb, int32_t ib, const float *A, int64_t lda,
                            float *invA, void *stream);
hsma_status hsma_diag_inv_d(int64_t m, int32_t nb, int32_t ib, const double *A, int64_t lda,
                            double *invA, void *stream);
hsma_status hsma_diag_inv_c(int64_t m, int32_t nb, int32_t ib, const hsma_float_complex *A,
                            int64_t lda, hsma_float_complex *invA, void *stream);
hsma_status hsma_diag_inv_z(int64_t m, int32_t nb, int32_t ib, const hsma_double_complex *A,
                            int64_t lda, hsma_double_complex *invA, void *stream);

/*
 * hsma_diag_inv_ex_{s,d,c,z}: hsma_diag_inv_* with the block size, inner
 * block and inversion route taken from opts (nb, ib, inv; NULL = defaults;
 * path and the event fields are ignored), for checking each route on its
 * own. Errors as hsma_diag_inv_*; INVALID_VALUE if the route does not apply.
 */
hsma_status hsma_diag_inv_ex_s(int64_t m, const hsma_trsm_opts *opts, const float *A, int64_t lda,
                               float *invA, void *stream);
hsma_status hsma_diag_inv_ex_d(int64_t m, const hsma_trsm_opts *opts, const double *A,
                               int64_t lda, double *invA, void *stream);
hsma_status hsma_diag_inv_ex_c(int64_t m, const hsma_trsm_opts *opts,
                               const hsma_float_complex *A, int64_t lda,
                               hsma_float_complex *invA, void *stream);
hsma_status hsma_diag_inv_ex_z(int64_t m, const hsma_trsm_opts *opts,
                               const hsma_double_complex *A, int64_t lda,
                               hsma_double_complex *invA, void *stream);

/*
 * hsma_gemm_{s,d,c,z}: C = beta*C + alpha*A*B with A M x K, B K x N,
 * C M x N, all column-major, on the matrix cores (the update of the trailing
 * rows and the multiply by an inverted diagonal block in the blocked path).
 * alpha and beta are real, beta must be 0 or 1 (beta == 0: C is not read).
 * a_lower == 1 declares A lower triangular with M == K: the kernel then skips
 * the zero tiles above the diagonal and treats those entries as exact zeros
 * (it never reads them). a_lower == 2 (hsma_gemm_s and hsma_gemm_d only, M
 * even) declares A lower triangular in 2 x 2 blocks, the real form of a
 * complex lower-triangular matrix (complex entry (i, k) as the block
 * [[re, -im], [im, re]] at rows 2i, 2i+1 and columns 2k, 2k+1): entries with
 * k > i | 1 are treated as zeros. Other values of a_lower:
 * HSMA_STATUS_INVALID_VALUE. C must not overlap A or B.
 */
hsma_status hsma_gemm_s(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                        const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                        int32_t a_lower, void *stream);
hsma_status hsma_gemm_d(int64_t M, int64_t N, int64_t K, double alpha, const double *A,
                        int64_t lda, const double *B, int64_t ldb, double beta, double *C,
                        int64_t ldc, int32_t a_lower, void *stream);
hsma_status hsma_gemm_c(int64_t M, int64_t N, int64_t K, float alpha, const hsma_float_complex *A,
                        int64_t lda, const hsma_float_complex *B, int64_t ldb, float beta,
                        hsma_float_complex *C, int64_t ldc, int32_t a_lower, void *stream);
hsma_status hsma_gemm_z(int64_t M, int64_t N, int64_t K, double alpha,
                        const hsma_double_complex *A, int64_t lda, const hsma_double_complex *B,
                        int64_t ldb, double beta, hsma_double_complex *C, int64_t ldc,
                        int32_t a_lower, void *stream);

/*
 * hsma_trsm_noalloc: the solve of hsma_trsm_{s,d,c,z} (same operation,
 * layout and semantics; dtype is an HSMA_DTYPE_* code and alpha points to
 * one host value of that element type) without any device allocation, for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It calls no hipMalloc, hipFree or
 * other allocating routine. The blocked path's workspace comes from a fixed
 * 64 MiB device array in the library, one per GPU, held from the library's
 * first use on that GPU until the process ends. The block size is the
 * table's, halved until the inverted diagonal blocks fill at most half of
 * it, and B is solved in column chunks that fit the rest (so large problems
 * may run with a smaller N_B than hsma_trsm_*). Limit: roughly
 * 16 * m * sizeof(element) <= 32 MiB, i.e. m <= 524288 (f32), 262144 (f64,
 * c64), 131072 (c128); larger m returns SCRATCH_TOO_SMALL before any GPU
 * work. m <= 64 uses no scratch. All calls on one GPU share its array:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and must be serialised by the caller; the array keeps the last
 * call's contents, and nothing in it needs to start at zero.
 * Errors: INVALID_SIZE, INVALID_POINTER (alpha NULL, or A/B NULL as for
 * hsma_trsm_*), INVALID_VALUE (bad dtype), SCRATCH_TOO_SMALL, HIP_ERROR.
 */
hsma_status hsma_trsm_noalloc(int32_t dtype, int64_t m, int64_t n, const void *alpha,
                              const void *A, int64_t lda, void *B, int64_t ldb, void *stream);

/*
 * hsma_trsm_block_size: the outer block size N_B the blocked path uses for
 * an m x m system with n right-hand sides of the given dtype (HSMA_DTYPE_*),
 * from the built-in "scale x dtype -> block" table (HSMA-TRSM paper,
 * adaptive blocking section), here keyed on the shape (m, n): the nearest
 * tested shape by |log2 m - log2 m_i| + |log2 n - log2 n_i|. Returns 0 for
 * m <= 64 (small path) and -1 for a bad dtype; n < 1 counts as 1. The
 * environment variable HSMA_NB, read once, overrides the table when set to
 * a valid block size.
 */
int32_t hsma_trsm_block_size(int32_t dtype, int64_t m, int64_t n);

/* Static, human-readable name of a status code. */
const char *hsma_status_string(hsma_status status);

#ifdef __cplusplus
}
#endif

#endif /* HSMA_TRSM_H */
