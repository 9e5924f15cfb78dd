// internal.hpp - launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsma_trsm.h"
#include "common.hpp"

namespace hsma {

// Small regime, lane = row (any m <= 64, any strides, negative ones
// included; X may alias B). unit: unit diagonal, the stored diagonal is not
// read.
template <typename T>
hipError_t small_rowlane(const T *A, int64_t sai, int64_t saj, int64_t sa2, int64_t sa3,
                         const T *B, int64_t sbi, int64_t sbj, int64_t sb2, int64_t sb3,
                         T *X, int64_t sxi, int64_t sxj, int64_t sx2, int64_t sx3,
                         int64_t m, int64_t n, int64_t ne02, int64_t ne03, T alpha, hipStream_t s,
                         bool unit = false);

// Small regime, lane = right-hand-side column (m == 64, column-major, in place).
template <typename T>
hipError_t small_colane(int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA, T *B,
                        int64_t ldb, int64_t strideB, int64_t batch, hipStream_t s);

// Same with a two-level batch: problem z = g * per + k uses A + g*strideA2 +
// k*strideA and B + g*strideB2 + k*strideB.
template <typename T>
hipError_t small_colane2(int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA,
                         int64_t strideA2, T *B, int64_t ldb, int64_t strideB, int64_t strideB2,
                         int64_t per, int64_t batch, hipStream_t s);

// SOLVE_TRI (ggml row-major layout, f32) for 64 < n <= 256: block rows of 64,
// one wave each, in one launch (hipErrorInvalidValue outside that range).
hipError_t solve_tri_medium(int64_t n, int64_t k, const float *A, const float *B, float *X,
                            int64_t ne02, int64_t ne03, int64_t sA1, int64_t sA2, int64_t sA3,
                            int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1, int64_t sX2,
                            int64_t sX3, hipStream_t s);

// B := alpha*B, or B := 0 when set_zero (column-major, batched).
template <typename T>
hipError_t scale_matrix(T *B, int64_t m, int64_t n, int64_t ldb, int64_t strideB, int64_t batch,
                        T alpha, bool set_zero, hipStream_t s);

// Stream-ordered workspace from the library's memory pool of the current
// device (created on first use; freed memory is kept for reuse). Returns
// hipErrorOutOfMemory without any HIP call when HSMA_TEST_FAIL_ALLOC=1.
hipError_t workspace_alloc(void **p, size_t bytes, hipStream_t s);
hipError_t workspace_free(void *p, hipStream_t s);

// Blocked regime: inversion of all diagonal blocks of size nb (inner block ib).
template <typename T>
hipError_t diag_invert(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA,
                       hipStream_t s);

// Same, by route (HSMA_INV_*): AUTO takes the blocked-inverse formula (small
// solver + batched GEMMs) when m is a multiple of nb and nb of 64 (nb >= 128;
// nb > 128 for f64 and c64, nb > 256 for c128), else the column
// substitution; FUSED inverts 2*ib
// blocks in LDS and merges.
// A route that does not apply to (m, nb, ib) gives hipErrorInvalidValue.
template <typename T>
hipError_t diag_invert_any(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA,
                           hipStream_t s, int route = 0);
template <typename T>
bool invert_route_applies(int64_t m, int nb, int ib, int route);

// C = beta*C + alpha*A*B on the matrix cores (beta in {0, 1}); a_lower 1: A
// is lower triangular (M == K) and its upper tiles are skipped; 2 (real
// types): A is lower triangular in 2 x 2 blocks, the real form of a complex
// lower-triangular matrix (entry (i, k) is used when k <= i | 1).
template <typename T>
hipError_t gemm(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha, const T *A,
                int64_t lda, const T *B, int64_t ldb, typename traits<T>::real beta, T *C,
                int64_t ldc, int a_lower, hipStream_t s);

// Strided-batched C_z = beta*C_z + alpha*A_z*B_z, z < batch (A_z = A + z*strideA,
// alike for B and C; strideA may be 0).
template <typename T>
hipError_t gemm_strided(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha,
                        const T *A, int64_t lda, int64_t strideA, const T *B, int64_t ldb,
                        int64_t strideB, typename traits<T>::real beta, T *C, int64_t ldc,
                        int64_t strideC, int64_t batch, hipStream_t s);

// Phase events of the blocked path: mark(phase) records the caller's next
// event on the stream and notes which phase starts there.
struct PhaseRec {
    hipEvent_t *ev = nullptr;
    int32_t *phase = nullptr;
    int cap = 0;
    int used = 0;
    hipError_t mark(int ph, hipStream_t s)
    {
        if (used >= cap) return hipErrorInvalidValue;
        phase[used] = ph;
        return hipEventRecord(ev[used++], s);
    }
};
// Events a blocked solve with nt diagonal blocks records (excluding scaling):
// inversion, then per block row the inverse multiply, the copy and (all but
// the last) the trailing update, then the end.
inline int blocked_phase_events(int64_t nt) { return (int)(3 * nt + 1); }

// Whole blocked solve of one problem (B already scaled by alpha), with a
// caller-provided workspace of blocked_workspace_elems<T>(m, n, nb) elements.
// rec (nullable) records the phase events.
template <typename T>
int64_t blocked_workspace_elems(int64_t m, int64_t n, int nb);
template <typename T>
hipError_t blocked_solve(int64_t m, int64_t n, int nb, int ib, const T *A, int64_t lda, T *B,
                         int64_t ldb, T *work, hipStream_t s, PhaseRec *rec = nullptr,
                         int route = 0);

// The two halves of blocked_solve. blocked_invert: all diagonal blocks into
// invA (ceil(m/nb) blocks of nb x nb), using temp (blocked_inverse_temp_elems
// elements) for the blocked-inverse merges. blocked_apply: the block-row
// loop for n columns of B with the inverted blocks, W holding nb x n.
int64_t blocked_inverse_temp_elems(int64_t m, int nb);
template <typename T>
hipError_t blocked_invert(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA, T *temp,
                          hipStream_t s, int route = 0);
// part (part_elems elements, may be NULL) holds split-K partial products
// for products with few output tiles. With ov, each W -> B_t copy runs on
// ov->aux beside the trailing product on s (both only read W), and s waits
// for it before W is written again.
struct CopyOverlap {
    hipStream_t aux;
    hipEvent_t ready, copied;
};
template <typename T>
hipError_t blocked_apply(int64_t m, int64_t n, int nb, const T *A, int64_t lda, const T *invA,
                         T *B, int64_t ldb, T *W, hipStream_t s, PhaseRec *rec = nullptr,
                         T *part = nullptr, int64_t part_elems = 0,
                         const CopyOverlap *ov = nullptr, T *expand = nullptr);

// The second stream of the current device for the blocked path's copies
// (created on first use, default priority, kept until the process ends).
hipError_t aux_stream(hipStream_t *out);

// Small-regime dispatch on column-major storage, in place (m <= 64): the
// lane-per-column kernel needs the full 64 rows, enough columns to fill a
// wavefront and 16-byte aligned columns of B; otherwise the lane-per-row
// kernel.
template <typename T>
hipError_t small_path(int64_t m, int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA,
                      T *B, int64_t ldb, int64_t strideB, int64_t batch, hipStream_t s)
{
    const int64_t sb = batch > 1 ? strideB : 0;
    const bool aligned = ((uintptr_t)B & 15) == 0 && ((ldb * (int64_t)sizeof(T)) & 15) == 0 &&
                         ((sb * (int64_t)sizeof(T)) & 15) == 0;
    if (m == 64 && n >= 32 && aligned)
        return small_colane<T>(n, alpha, A, lda, strideA, B, ldb, sb, batch, s);
    return small_rowlane<T>(A, 1, lda, strideA, 0, B, 1, ldb, strideB, 0, B, 1, ldb, strideB, 0,
                            m, n, batch, 1, alpha, s);
}

// dst(i, j) = f(src(i, j)) for i < rows, j < cols (only j <= i when lower)
// of batch problems: element (i, j) of problem b at src[b*ssb + i*ssi +
// j*ssj], dst alike (strides of either sign). f conjugates (conj), puts 1 on
// the diagonal without reading it (unit) and multiplies by *alpha (when
// alpha is not NULL).
template <typename T>
hipError_t tile_copy(const T *src, int64_t ssi, int64_t ssj, int64_t ssb, T *dst, int64_t dsi,
                     int64_t dsj, int64_t dsb, int64_t rows, int64_t cols, int64_t batch,
                     bool lower, bool conj, bool unit, const T *alpha, hipStream_t s);

// Outer block size for an m x m system with n right-hand sides of the given
// dtype code: the table by nearest shape, or the HSMA_NB override (api.cpp).
int choose_nb(int dtype, int64_t m, int64_t n);

}  // namespace hsma
