// api.cpp - the C ABI (include/hsma_trsm.h): argument checks, quick returns,
// path dispatch and the blocked path's workspace.
//
// Dispatch follows the HSMA-TRSM pages' size x dtype strategy (news summary,
// "One framework, several paths"; paper, small-scale section): m <= 64 is
// solved directly on chip, larger m by the blocked solver whose outer block
// N_B comes from a "size x dtype -> block" table with nearest-size lookup
// (paper, adaptive blocking section).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <mutex>

#include "hsma_trsm.h"
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

// ---------------------------------------------------------------------------
// Workspace pool: one stream-ordered memory pool per device, owned by the
// library for the life of the process. Its release threshold is unlimited,
// so memory freed at the end of a call stays mapped for the next one; with
// the default pool (threshold 0) every synchronisation hands it back to the
// driver and the next call maps it again.

namespace {
constexpr int kMaxDevices = 64;
hipMemPool_t g_pool[kMaxDevices] = {};
std::mutex g_pool_mutex;

hipError_t device_pool(int dev, hipMemPool_t *out)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (!g_pool[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        g_pool[dev] = pool;
    }
    *out = g_pool[dev];
    return hipSuccess;
}
}  // namespace

hipError_t workspace_alloc(void **p, size_t bytes, hipStream_t s)
{
    // Allocation-failure injection for tests of the error path: read on
    // every call, before any HIP call.
    const char *fail = std::getenv("HSMA_TEST_FAIL_ALLOC");
    if (fail && fail[0] == '1' && fail[1] == 0) return hipErrorOutOfMemory;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipMemPool_t pool = nullptr;
    e = device_pool(dev, &pool);
    if (e != hipSuccess) return e;
    return hipMallocFromPoolAsync(p, bytes, pool, s);
}

hipError_t workspace_free(void *p, hipStream_t s) { return hipFreeAsync(p, s); }

namespace {
hipStream_t g_aux[kMaxDevices] = {};
std::mutex g_aux_mutex;
}  // namespace

hipError_t aux_stream(hipStream_t *out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_aux_mutex);
    if (!g_aux[dev]) {
        hipStream_t st = nullptr;
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e != hipSuccess) return e;
        g_aux[dev] = st;
    }
    *out = g_aux[dev];
    return hipSuccess;
}

namespace {

// ---------------------------------------------------------------------------
// Block-size table: tested shapes (m_i, n_i) and the best N_B at each, per
// dtype. Lookup takes the tested shape nearest to (m, n) by
// |log2 m - log2 m_i| + |log2 n - log2 n_i| (ties go to the earlier entry,
// which the table lists by increasing m, then n), then clamps N_B to m
// rounded up to a multiple of 16.

struct NbEntry {
    int64_t m, n;
    int nb;
};

#include "nb_table.inc"

int table_lookup(int dtype, int64_t m, int64_t n)
{
    const NbEntry *tab = nullptr;
    int len = 0;
    switch (dtype) {
    case 0: tab = kNbF32; len = (int)(sizeof(kNbF32) / sizeof(kNbF32[0])); break;
    case 1: tab = kNbF64; len = (int)(sizeof(kNbF64) / sizeof(kNbF64[0])); break;
    case 2: tab = kNbC64; len = (int)(sizeof(kNbC64) / sizeof(kNbC64[0])); break;
    case 3: tab = kNbC128; len = (int)(sizeof(kNbC128) / sizeof(kNbC128[0])); break;
    default: return -1;
    }
    const double lm = std::log2((double)m), ln = std::log2((double)(n > 0 ? n : 1));
    int best = 0;
    double bd = 1e300;
    for (int i = 0; i < len; ++i) {
        const double d = std::fabs(lm - std::log2((double)tab[i].m)) +
                         std::fabs(ln - std::log2((double)tab[i].n));
        if (d < bd - 1e-12) { bd = d; best = i; }
    }
    return tab[best].nb;
}

constexpr int kMaxNb = 2048;
constexpr int64_t kSolveTriMaxN = 256;  // SOLVE_TRI sizes handled (block rows of 64 above 64)

bool valid_nb(int64_t nb) { return nb >= 16 && nb <= kMaxNb && nb % 16 == 0; }

// Large blocks are inverted only by the blocked-inverse formula, which needs
// m to be a multiple of N_B: above 1024 rows (the column-substitution kernel
// holds at most 1024 rows of an identity tile in registers), and above 512
// for double complex.
bool nb_fits(int64_t nb, int64_t m, int dtype)
{
    return nb <= (dtype == 3 ? 512 : 1024) || m % nb == 0;
}

int env_nb()
{
    static int value = -1;
    static std::once_flag once;
    std::call_once(once, [] {
        const char *s = std::getenv("HSMA_NB");
        if (s) {
            char *end = nullptr;
            const long v = std::strtol(s, &end, 10);
            if (end != s && valid_nb(v)) value = (int)v;
        }
    });
    return value;
}


}  // namespace

int choose_nb(int dtype, int64_t m, int64_t n)
{
    int nb = env_nb();
    if (nb <= 0) nb = table_lookup(dtype, m, n);
    if (nb > kMaxNb) nb = kMaxNb;
    while (!nb_fits(nb, m, dtype)) nb /= 2;
    const int64_t cap = ((m + 15) / 16) * 16;
    if (nb > cap) nb = (int)(cap < 16 ? 16 : cap);
    return nb;
}

namespace {

// ---------------------------------------------------------------------------

template <typename T>
T from_abi(T v) { return v; }
inline c32 from_abi(hsma_float_complex v) { return {v.re, v.im}; }
inline c64 from_abi(hsma_double_complex v) { return {v.re, v.im}; }

hsma_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return HSMA_STATUS_SUCCESS;
    // Only workspace allocations report out-of-memory.
    if (e == hipErrorOutOfMemory) return HSMA_STATUS_ALLOC_FAILED;
    return HSMA_STATUS_HIP_ERROR;
}

int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// Largest m of the block-rows-of-64 route for batches: against one blocked
// solve per problem it measured 1.1-15x faster on MI355X up to m = 512
// (batches of 2 to 32) and mixed to 4x slower at m = 768 and above.
constexpr int64_t kMediumMaxM = 512;

hsma_status check_opts(const hsma_trsm_opts *o, int dtype, int64_t m)
{
    if (!o) return HSMA_STATUS_SUCCESS;
    if (o->path < HSMA_PATH_AUTO || o->path > HSMA_PATH_ROWS64) return HSMA_STATUS_INVALID_VALUE;
    if (o->inv < HSMA_INV_AUTO || o->inv > HSMA_INV_COLUMN) return HSMA_STATUS_INVALID_VALUE;
    if (o->path == HSMA_PATH_SMALL && m > 64) return HSMA_STATUS_INVALID_VALUE;
    if (o->path == HSMA_PATH_ROWS64 && m > kMediumMaxM) return HSMA_STATUS_INVALID_VALUE;
    if (o->nb != 0 && (!valid_nb(o->nb) || !nb_fits(o->nb, m, dtype)))
        return HSMA_STATUS_INVALID_VALUE;
    if (o->ib != 0) {
        const int nb = o->nb != 0 ? o->nb : 0;
        if (o->ib < 1) return HSMA_STATUS_INVALID_VALUE;
        if (nb != 0 && (nb % o->ib != 0 || nb / o->ib > 64)) return HSMA_STATUS_INVALID_VALUE;
    }
    if (o->n_events < 0) return HSMA_STATUS_INVALID_VALUE;
    if (o->n_events > 0 && (!o->events || !o->event_phase || !o->events_used))
        return HSMA_STATUS_INVALID_POINTER;
    return HSMA_STATUS_SUCCESS;
}

// Batches of 64 < m <= 512: block rows of 64 for the whole batch at once
// (X_r = A_rr^{-1} (B_r - A[r, <r] X_<r)), the update by one strided-batched
// matrix-core GEMM and the diagonal solve by the small regime, both over all
// problems; 2 * ceil(m/64) launches instead of a blocked solve per problem.
// A single problem takes this route too when m <= kRows64SingleMaxM and it
// has at most kRows64MaxRhs right-hand sides: there the blocked path's
// inversion costs more than the substitution it replaces (measured on
// MI355X: 1.03-2.2x for n <= 16, m <= 192, in all four types); with more
// columns or rows the inverse-times-block products of the blocked path win.
constexpr int64_t kRows64MaxRhs = 16;
constexpr int64_t kRows64SingleMaxM = 192;

template <typename T>
hipError_t medium_batched(int64_t m, int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA,
                          T *B, int64_t ldb, int64_t strideB, int64_t batch, hipStream_t s)
{
    using R = typename traits<T>::real;
    hipError_t e = hipSuccess;
    if (!is_one(alpha)) {
        e = scale_matrix<T>(B, m, n, ldb, strideB, batch, alpha, false, s);
        if (e != hipSuccess) return e;
    }
    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    for (int64_t r0 = 0; r0 < m; r0 += 64) {
        const int64_t rows = m - r0 < 64 ? m - r0 : 64;
        if (r0 > 0) {
            e = gemm_strided<T>(rows, n, r0, R(-1), A + r0, lda, strideA, B, ldb, strideB, R(1),
                                B + r0, ldb, strideB, batch, s);
            if (e != hipSuccess) return e;
        }
        e = small_path<T>(rows, n, one, A + r0 + r0 * lda, lda, strideA, B + r0, ldb, strideB,
                          batch, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hsma_status trsm_impl(int64_t m, int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA,
                      T *B, int64_t ldb, int64_t strideB, int64_t batch,
                      const hsma_trsm_opts *opts, void *stream)
{
    constexpr int dt = traits<T>::dtype;
    if (m < 0 || n < 0 || batch < 0) return HSMA_STATUS_INVALID_SIZE;
    if (lda < imax(1, m) || ldb < imax(1, m)) return HSMA_STATUS_INVALID_SIZE;
    if (strideA < 0 || strideB < 0) return HSMA_STATUS_INVALID_SIZE;
    if (batch > 1 && strideB < ldb * n) return HSMA_STATUS_INVALID_SIZE;
    const hsma_status os = check_opts(opts, dt, m);
    if (os != HSMA_STATUS_SUCCESS) return os;
    const bool timed = opts && opts->n_events > 0;
    if (timed) *opts->events_used = 0;
    if (m == 0 || n == 0 || batch == 0) return HSMA_STATUS_SUCCESS;
    if (!B) return HSMA_STATUS_INVALID_POINTER;
    hipStream_t s = (hipStream_t)stream;
    if (is_zero(alpha)) return hip_status(scale_matrix<T>(B, m, n, ldb, strideB, batch, alpha, true, s));
    if (!A) return HSMA_STATUS_INVALID_POINTER;

    const int path = opts ? opts->path : HSMA_PATH_AUTO;
    const bool small = path == HSMA_PATH_SMALL || (path == HSMA_PATH_AUTO && m <= 64);
    if (small) return hip_status(small_path<T>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, s));
    if (path == HSMA_PATH_ROWS64 ||
        (path == HSMA_PATH_AUTO && m <= kMediumMaxM &&
         (batch > 1 || (m <= kRows64SingleMaxM && n <= kRows64MaxRhs))))
        return hip_status(medium_batched<T>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, s));

    // Blocked path.
    int nb = (opts && opts->nb) ? opts->nb : choose_nb(dt, m, n);
    if (!(opts && opts->nb)) {
        const int64_t cap = ((m + 15) / 16) * 16;
        if (nb > cap) nb = (int)cap;
    }
    int ib = (opts && opts->ib) ? opts->ib : (nb / 8 > 0 ? nb / 8 : 1);
    if (nb % ib != 0 || nb / ib > 64) return HSMA_STATUS_INVALID_VALUE;
    const int route = opts ? opts->inv : HSMA_INV_AUTO;
    if (!invert_route_applies<T>(m, nb, ib, route)) return HSMA_STATUS_INVALID_VALUE;

    // Phase events (single problems only: the *_ex entry points).
    PhaseRec rec;
    if (timed) {
        const int need = blocked_phase_events((m + nb - 1) / nb) + (is_one(alpha) ? 0 : 1);
        if (batch != 1 || opts->n_events < need) {
            *opts->events_used = need;
            return HSMA_STATUS_INVALID_VALUE;
        }
        rec.ev = (hipEvent_t *)opts->events;
        rec.phase = opts->event_phase;
        rec.cap = opts->n_events;
    }

    const int64_t welems = blocked_workspace_elems<T>(m, n, nb);
    void *work = nullptr;
    if (workspace_alloc(&work, (size_t)welems * sizeof(T), s) != hipSuccess || !work) {
        (void)hipGetLastError();
        return HSMA_STATUS_ALLOC_FAILED;
    }
    hipError_t e = hipSuccess;
    if (!is_one(alpha)) {
        if (timed) e = rec.mark(HSMA_PHASE_SCALE, s);
        if (e == hipSuccess) e = scale_matrix<T>(B, m, n, ldb, strideB, batch, alpha, false, s);
    }
    for (int64_t b = 0; b < batch && e == hipSuccess; ++b)
        e = blocked_solve<T>(m, n, nb, ib, A + b * strideA, lda, B + b * strideB, ldb, (T *)work, s,
                             timed ? &rec : nullptr, route);
    if (timed) *opts->events_used = rec.used;
    const hipError_t ef = workspace_free(work, s);
    if (e != hipSuccess || ef != hipSuccess) return HSMA_STATUS_HIP_ERROR;
    return HSMA_STATUS_SUCCESS;
}

// ---------------------------------------------------------------------------
// Other TRSM variants (side, triangle, op, unit diagonal) through the
// canonical left-side lower-triangular solve.
//
// With C = op(A) for the left side and C = op(A)^T for the right side
// (X op(A) = alpha B <=> op(A)^T X^T = alpha B^T), every variant solves
// C Y = alpha Bhat with Bhat = B (left) or B^T (right). C is lower
// triangular as it stands, or after reversing the order of its rows and
// columns (then Bhat's rows are reversed too). Both become strided views:
// Ahat(i, j) = conj?(A[aoff + i*sai + j*saj]) lower triangular of order M,
// Bhat(i, c) = B[boff + i*sbi + c*sbj], M x N.

struct VariantView {
    int64_t M, N;
    int64_t aoff, sai, saj;
    int64_t boff, sbi, sbj;
    bool conj, unit;
};

VariantView variant_view(int side, int uplo, int trans, int diag, int64_t m, int64_t n,
                         int64_t lda, int64_t ldb)
{
    VariantView v;
    const bool left = side == HSMA_SIDE_LEFT;
    const int64_t k = left ? m : n;
    v.M = k;
    v.N = left ? n : m;
    v.conj = trans == HSMA_OP_C;
    v.unit = diag == HSMA_DIAG_UNIT;
    // C(i, j) is A(j, i) (conjugated for op C) when C "stores transposed"
    const bool st = left ? trans != HSMA_OP_N : trans == HSMA_OP_N;
    const bool op_lower = (uplo == HSMA_FILL_LOWER) == (trans == HSMA_OP_N);
    const bool c_lower = left ? op_lower : !op_lower;
    int64_t si = st ? lda : 1, sj = st ? 1 : lda;
    v.aoff = 0;
    if (!c_lower) {   // reverse the index order: Ahat(i, j) = C(k-1-i, k-1-j)
        v.aoff = (k - 1) * (1 + lda);
        si = -si;
        sj = -sj;
    }
    v.sai = si;
    v.saj = sj;
    v.sbi = left ? 1 : ldb;
    v.sbj = left ? ldb : 1;
    v.boff = 0;
    if (!c_lower) {
        v.boff = (k - 1) * v.sbi;
        v.sbi = -v.sbi;
    }
    return v;
}

template <typename T>
hsma_status trsm_variant_impl(int side, int uplo, int trans, int diag, int64_t m, int64_t n,
                              T alpha, const T *A, int64_t lda, int64_t strideA, T *B,
                              int64_t ldb, int64_t strideB, int64_t batch, void *stream)
{
    constexpr int dt = traits<T>::dtype;
    if (side < 0 || side > 1 || uplo < 0 || uplo > 1 || trans < 0 || trans > 2 || diag < 0 ||
        diag > 1)
        return HSMA_STATUS_INVALID_VALUE;
    if (!traits<T>::is_complex && trans == HSMA_OP_C) trans = HSMA_OP_T;  // conj(a) = a
    const int64_t k = side == HSMA_SIDE_LEFT ? m : n;
    if (m < 0 || n < 0 || batch < 0) return HSMA_STATUS_INVALID_SIZE;
    if (lda < imax(1, k) || ldb < imax(1, m)) return HSMA_STATUS_INVALID_SIZE;
    if (strideA < 0 || strideB < 0) return HSMA_STATUS_INVALID_SIZE;
    if (batch > 1 && strideB < ldb * n) return HSMA_STATUS_INVALID_SIZE;
    if (side == HSMA_SIDE_LEFT && uplo == HSMA_FILL_LOWER && trans == HSMA_OP_N &&
        diag == HSMA_DIAG_NON_UNIT)
        return trsm_impl<T>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, nullptr, stream);
    if (m == 0 || n == 0 || batch == 0) return HSMA_STATUS_SUCCESS;
    if (!B) return HSMA_STATUS_INVALID_POINTER;
    hipStream_t s = (hipStream_t)stream;
    if (is_zero(alpha)) return hip_status(scale_matrix<T>(B, m, n, ldb, strideB, batch, alpha, true, s));
    if (!A) return HSMA_STATUS_INVALID_POINTER;

    const VariantView v = variant_view(side, uplo, trans, diag, m, n, lda, ldb);
    const T *Ah = A + v.aoff;
    T *Bh = B + v.boff;
    const int64_t M = v.M, N = v.N;
    if (M <= 64) {
        // The lane-per-row kernel reads the views directly. A conjugated
        // system conj(C) Y = alpha Bhat is solved as C conj(Y) =
        // conj(alpha) conj(Bhat): Bhat is conjugated in place before and
        // after the solve.
        T a = alpha;
        hipError_t e = hipSuccess;
        if constexpr (traits<T>::is_complex) {
            if (v.conj) {
                a.im = -a.im;
                e = tile_copy<T>(Bh, v.sbi, v.sbj, strideB, Bh, v.sbi, v.sbj, strideB, M, N, batch,
                                 false, true, false, nullptr, s);
            }
        }
        if (e == hipSuccess)
            e = small_rowlane<T>(Ah, v.sai, v.saj, strideA, 0, Bh, v.sbi, v.sbj, strideB, 0, Bh, v.sbi,
                                 v.sbj, strideB, 0, M, N, batch, 1, a, s, v.unit);
        if constexpr (traits<T>::is_complex) {
            if (v.conj && e == hipSuccess)
                e = tile_copy<T>(Bh, v.sbi, v.sbj, strideB, Bh, v.sbi, v.sbj, strideB, M, N, batch,
                                 false, true, false, nullptr, s);
        }
        return hip_status(e);
    }

    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    hipError_t e = hipSuccess;
    void *work = nullptr;
    if (batch > 1 && M <= kMediumMaxM) {
        // gather every problem's Ahat triangle and alpha*Bhat, block rows of
        // 64 over the whole batch, scatter X back
        const size_t elems = (size_t)batch * (size_t)(M * M + M * N);
        if (workspace_alloc(&work, elems * sizeof(T), s) != hipSuccess || !work) {
            (void)hipGetLastError();
            return HSMA_STATUS_ALLOC_FAILED;
        }
        T *Aw = (T *)work, *Bw = Aw + batch * M * M;
        e = tile_copy<T>(Ah, v.sai, v.saj, strideA, Aw, 1, M, M * M, M, M, batch, true, v.conj,
                         v.unit, nullptr, s);
        if (e == hipSuccess)
            e = tile_copy<T>(Bh, v.sbi, v.sbj, strideB, Bw, 1, M, M * N, M, N, batch, false, false,
                             false, is_one(alpha) ? nullptr : &alpha, s);
        if (e == hipSuccess) e = medium_batched<T>(M, N, one, Aw, M, M * M, Bw, M, M * N, batch, s);
        if (e == hipSuccess)
            e = tile_copy<T>(Bw, 1, M, M * N, Bh, v.sbi, v.sbj, strideB, M, N, batch, false, false,
                             false, nullptr, s);
    } else {
        // one problem at a time: the triangle of Ahat into an M x M
        // column-major copy, Bhat into an M x N one unless it is B itself
        // (left side, no reversal), then the canonical blocked solve
        const bool b_direct = v.sbi == 1 && v.boff == 0;
        const int nb = choose_nb(dt, M, N);
        const int64_t wblk = blocked_workspace_elems<T>(M, N, nb);
        const size_t elems = (size_t)(M * M + (b_direct ? 0 : M * N) + wblk);
        if (workspace_alloc(&work, elems * sizeof(T), s) != hipSuccess || !work) {
            (void)hipGetLastError();
            return HSMA_STATUS_ALLOC_FAILED;
        }
        T *Aw = (T *)work;
        T *Bw = b_direct ? nullptr : Aw + M * M;
        T *Wk = Aw + M * M + (b_direct ? 0 : M * N);
        for (int64_t b = 0; b < batch && e == hipSuccess; ++b) {
            const T *Ab = Ah + b * strideA;
            T *Bb = Bh + b * strideB;
            e = tile_copy<T>(Ab, v.sai, v.saj, 0, Aw, 1, M, 0, M, M, 1, true, v.conj, v.unit,
                             nullptr, s);
            if (e != hipSuccess) break;
            if (b_direct) {
                if (!is_one(alpha)) e = scale_matrix<T>(Bb, M, N, ldb, 0, 1, alpha, false, s);
                if (e == hipSuccess)
                    e = blocked_solve<T>(M, N, nb, nb / 8 > 0 ? nb / 8 : 1, Aw, M, Bb, ldb, Wk, s);
            } else {
                e = tile_copy<T>(Bb, v.sbi, v.sbj, 0, Bw, 1, M, 0, M, N, 1, false, false, false,
                                 is_one(alpha) ? nullptr : &alpha, s);
                if (e == hipSuccess)
                    e = blocked_solve<T>(M, N, nb, nb / 8 > 0 ? nb / 8 : 1, Aw, M, Bw, M, Wk, s);
                if (e == hipSuccess)
                    e = tile_copy<T>(Bw, 1, M, 0, Bb, v.sbi, v.sbj, 0, M, N, 1, false, false, false,
                                     nullptr, s);
            }
        }
    }
    const hipError_t ef = workspace_free(work, s);
    if (e != hipSuccess || ef != hipSuccess) return HSMA_STATUS_HIP_ERROR;
    return HSMA_STATUS_SUCCESS;
}

template <typename T>
hsma_status diag_inv_impl(int64_t m, int32_t nb, int32_t ib, const T *A, int64_t lda, T *invA,
                          void *stream, int route = HSMA_INV_AUTO)
{
    constexpr int dt = traits<T>::dtype;
    if (m < 0 || lda < imax(1, m)) return HSMA_STATUS_INVALID_SIZE;
    if (nb == 0) nb = choose_nb(dt, m > 64 ? m : 65, m > 64 ? m : 65);
    if (!valid_nb(nb) || !nb_fits(nb, m, dt)) return HSMA_STATUS_INVALID_VALUE;
    if (ib == 0) ib = nb / 8;
    if (ib < 1 || nb % ib != 0 || nb / ib > 64) return HSMA_STATUS_INVALID_VALUE;
    if (route < HSMA_INV_AUTO || route > HSMA_INV_COLUMN) return HSMA_STATUS_INVALID_VALUE;
    if (m == 0) return HSMA_STATUS_SUCCESS;
    if (!invert_route_applies<T>(m, nb, ib, route)) return HSMA_STATUS_INVALID_VALUE;
    if (!A || !invA) return HSMA_STATUS_INVALID_POINTER;
    return hip_status(diag_invert_any<T>(m, nb, ib, A, lda, invA, (hipStream_t)stream, route));
}

template <typename T>
hsma_status diag_inv_ex_impl(int64_t m, const hsma_trsm_opts *o, const T *A, int64_t lda, T *invA,
                             void *stream)
{
    return diag_inv_impl<T>(m, o ? o->nb : 0, o ? o->ib : 0, A, lda, invA, stream,
                            o ? o->inv : HSMA_INV_AUTO);
}

template <typename T>
hsma_status gemm_impl(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha, const T *A,
                      int64_t lda, const T *B, int64_t ldb, typename traits<T>::real beta, T *C,
                      int64_t ldc, int32_t a_lower, void *stream)
{
    if (M < 0 || N < 0 || K < 0) return HSMA_STATUS_INVALID_SIZE;
    if (lda < imax(1, M) || ldb < imax(1, K) || ldc < imax(1, M)) return HSMA_STATUS_INVALID_SIZE;
    if (a_lower < 0 || a_lower > 2 || (a_lower == 2 && traits<T>::is_complex)) return HSMA_STATUS_INVALID_VALUE;
    if (a_lower && M != K) return HSMA_STATUS_INVALID_SIZE;
    if (a_lower == 2 && M % 2 != 0) return HSMA_STATUS_INVALID_SIZE;
    if (!(beta == 0 || beta == 1)) return HSMA_STATUS_INVALID_VALUE;
    if (M == 0 || N == 0) return HSMA_STATUS_SUCCESS;
    if (!C || (K > 0 && (!A || !B))) return HSMA_STATUS_INVALID_POINTER;
    return hip_status(gemm<T>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, a_lower,
                              (hipStream_t)stream));
}

}  // namespace
}  // namespace hsma

using namespace hsma;

#define HSMA_NOEXCEPT(expr)                                                                        \
    try {                                                                                          \
        return expr;                                                                               \
    } catch (...) {                                                                                \
        return HSMA_STATUS_HIP_ERROR;                                                              \
    }

extern "C" {

hsma_status hsma_trsm_s(int64_t m, int64_t n, float alpha, const float *A, int64_t lda, float *B,
                        int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<float>(m, n, alpha, A, lda, 0, B, ldb, 0, 1, nullptr, stream))
}
hsma_status hsma_trsm_d(int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                        double *B, int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<double>(m, n, alpha, A, lda, 0, B, ldb, 0, 1, nullptr, stream))
}
hsma_status hsma_trsm_c(int64_t m, int64_t n, hsma_float_complex alpha,
                        const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                        int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c32>(m, n, from_abi(alpha), (const c32 *)A, lda, 0, (c32 *)B, ldb, 0,
                                 1, nullptr, stream))
}
hsma_status hsma_trsm_z(int64_t m, int64_t n, hsma_double_complex alpha,
                        const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                        int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c64>(m, n, from_abi(alpha), (const c64 *)A, lda, 0, (c64 *)B, ldb, 0,
                                 1, nullptr, stream))
}

hsma_status hsma_trsm_strided_batched_s(int64_t m, int64_t n, float alpha, const float *A,
                                        int64_t lda, int64_t strideA, float *B, int64_t ldb,
                                        int64_t strideB, int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<float>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch_count,
                                   nullptr, stream))
}
hsma_status hsma_trsm_strided_batched_d(int64_t m, int64_t n, double alpha, const double *A,
                                        int64_t lda, int64_t strideA, double *B, int64_t ldb,
                                        int64_t strideB, int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<double>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch_count,
                                    nullptr, stream))
}
hsma_status hsma_trsm_strided_batched_c(int64_t m, int64_t n, hsma_float_complex alpha,
                                        const hsma_float_complex *A, int64_t lda, int64_t strideA,
                                        hsma_float_complex *B, int64_t ldb, int64_t strideB,
                                        int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c32>(m, n, from_abi(alpha), (const c32 *)A, lda, strideA, (c32 *)B,
                                 ldb, strideB, batch_count, nullptr, stream))
}
hsma_status hsma_trsm_strided_batched_z(int64_t m, int64_t n, hsma_double_complex alpha,
                                        const hsma_double_complex *A, int64_t lda, int64_t strideA,
                                        hsma_double_complex *B, int64_t ldb, int64_t strideB,
                                        int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c64>(m, n, from_abi(alpha), (const c64 *)A, lda, strideA, (c64 *)B,
                                 ldb, strideB, batch_count, nullptr, stream))
}

hsma_status hsma_trsm_ex_s(int64_t m, int64_t n, float alpha, const float *A, int64_t lda,
                           float *B, int64_t ldb, const hsma_trsm_opts *opts, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<float>(m, n, alpha, A, lda, 0, B, ldb, 0, 1, opts, stream))
}
hsma_status hsma_trsm_ex_d(int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                           double *B, int64_t ldb, const hsma_trsm_opts *opts, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<double>(m, n, alpha, A, lda, 0, B, ldb, 0, 1, opts, stream))
}
hsma_status hsma_trsm_ex_c(int64_t m, int64_t n, hsma_float_complex alpha,
                           const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                           int64_t ldb, const hsma_trsm_opts *opts, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c32>(m, n, from_abi(alpha), (const c32 *)A, lda, 0, (c32 *)B, ldb, 0,
                                 1, opts, stream))
}
hsma_status hsma_trsm_ex_z(int64_t m, int64_t n, hsma_double_complex alpha,
                           const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                           int64_t ldb, const hsma_trsm_opts *opts, void *stream)
{
    HSMA_NOEXCEPT(trsm_impl<c64>(m, n, from_abi(alpha), (const c64 *)A, lda, 0, (c64 *)B, ldb, 0,
                                 1, opts, stream))
}

hsma_status hsma_solve_tri_f32(int64_t n, int64_t k, const float *A, const float *B, float *X,
                               int64_t ne02, int64_t ne03, int64_t sA1, int64_t sA2, int64_t sA3,
                               int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1, int64_t sX2,
                               int64_t sX3, void *stream)
{
    try {
        if (n < 0 || k < 0 || ne02 < 0 || ne03 < 0) return HSMA_STATUS_INVALID_SIZE;
        if (n == 0 || k == 0 || ne02 == 0 || ne03 == 0) return HSMA_STATUS_SUCCESS;
        if (n > kSolveTriMaxN) return HSMA_STATUS_NOT_SUPPORTED;
        if (sA1 < n || sB1 < k || sX1 < k) return HSMA_STATUS_INVALID_SIZE;
        if (sA2 < 0 || sA3 < 0 || sB2 < 0 || sB3 < 0 || sX2 < 0 || sX3 < 0)
            return HSMA_STATUS_INVALID_SIZE;
        if (!A || !B || !X) return HSMA_STATUS_INVALID_POINTER;
        if (n > 64)
            return hip_status(solve_tri_medium(n, k, A, B, X, ne02, ne03, sA1, sA2, sA3, sB1, sB2,
                                               sB3, sX1, sX2, sX3, (hipStream_t)stream));
        return hip_status(small_rowlane<float>(A, sA1, 1, sA2, sA3, B, sB1, 1, sB2, sB3, X, sX1, 1,
                                               sX2, sX3, n, k, ne02, ne03, 1.0f,
                                               (hipStream_t)stream));
    } catch (...) {
        return HSMA_STATUS_HIP_ERROR;
    }
}

hsma_status hsma_diag_inv_s(int64_t m, int32_t nb, int32_t ib, const float *A, int64_t lda,
                            float *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_impl<float>(m, nb, ib, A, lda, invA, stream))
}
hsma_status hsma_diag_inv_d(int64_t m, int32_t nb, int32_t ib, const double *A, int64_t lda,
                            double *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_impl<double>(m, nb, ib, A, lda, invA, stream))
}
hsma_status hsma_diag_inv_c(int64_t m, int32_t nb, int32_t ib, const hsma_float_complex *A,
                            int64_t lda, hsma_float_complex *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_impl<c32>(m, nb, ib, (const c32 *)A, lda, (c32 *)invA, stream))
}
hsma_status hsma_diag_inv_z(int64_t m, int32_t nb, int32_t ib, const hsma_double_complex *A,
                            int64_t lda, hsma_double_complex *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_impl<c64>(m, nb, ib, (const c64 *)A, lda, (c64 *)invA, stream))
}

hsma_status hsma_diag_inv_ex_s(int64_t m, const hsma_trsm_opts *opts, const float *A, int64_t lda,
                               float *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_ex_impl<float>(m, opts, A, lda, invA, stream))
}
hsma_status hsma_diag_inv_ex_d(int64_t m, const hsma_trsm_opts *opts, const double *A,
                               int64_t lda, double *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_ex_impl<double>(m, opts, A, lda, invA, stream))
}
hsma_status hsma_diag_inv_ex_c(int64_t m, const hsma_trsm_opts *opts,
                               const hsma_float_complex *A, int64_t lda,
                               hsma_float_complex *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_ex_impl<c32>(m, opts, (const c32 *)A, lda, (c32 *)invA, stream))
}
hsma_status hsma_diag_inv_ex_z(int64_t m, const hsma_trsm_opts *opts,
                               const hsma_double_complex *A, int64_t lda,
                               hsma_double_complex *invA, void *stream)
{
    HSMA_NOEXCEPT(diag_inv_ex_impl<c64>(m, opts, (const c64 *)A, lda, (c64 *)invA, stream))
}

hsma_status hsma_gemm_s(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                        const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                        int32_t a_lower, void *stream)
{
    HSMA_NOEXCEPT(gemm_impl<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, a_lower, stream))
}
hsma_status hsma_gemm_d(int64_t M, int64_t N, int64_t K, double alpha, const double *A,
                        int64_t lda, const double *B, int64_t ldb, double beta, double *C,
                        int64_t ldc, int32_t a_lower, void *stream)
{
    HSMA_NOEXCEPT(gemm_impl<double>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, a_lower, stream))
}
hsma_status hsma_gemm_c(int64_t M, int64_t N, int64_t K, float alpha, const hsma_float_complex *A,
                        int64_t lda, const hsma_float_complex *B, int64_t ldb, float beta,
                        hsma_float_complex *C, int64_t ldc, int32_t a_lower, void *stream)
{
    HSMA_NOEXCEPT(gemm_impl<c32>(M, N, K, alpha, (const c32 *)A, lda, (const c32 *)B, ldb, beta,
                                 (c32 *)C, ldc, a_lower, stream))
}
hsma_status hsma_gemm_z(int64_t M, int64_t N, int64_t K, double alpha,
                        const hsma_double_complex *A, int64_t lda, const hsma_double_complex *B,
                        int64_t ldb, double beta, hsma_double_complex *C, int64_t ldc,
                        int32_t a_lower, void *stream)
{
    HSMA_NOEXCEPT(gemm_impl<c64>(M, N, K, alpha, (const c64 *)A, lda, (const c64 *)B, ldb, beta,
                                 (c64 *)C, ldc, a_lower, stream))
}

hsma_status hsma_trsm_general_s(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, float alpha, const float *A, int64_t lda,
                                float *B, int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<float>(side, uplo, trans, diag, m, n, alpha, A, lda, 0, B, ldb,
                                           0, 1, stream))
}
hsma_status hsma_trsm_general_d(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, double alpha, const double *A, int64_t lda,
                                double *B, int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<double>(side, uplo, trans, diag, m, n, alpha, A, lda, 0, B, ldb,
                                            0, 1, stream))
}
hsma_status hsma_trsm_general_c(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, hsma_float_complex alpha,
                                const hsma_float_complex *A, int64_t lda, hsma_float_complex *B,
                                int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<c32>(side, uplo, trans, diag, m, n, from_abi(alpha),
                                         (const c32 *)A, lda, 0, (c32 *)B, ldb, 0, 1, stream))
}
hsma_status hsma_trsm_general_z(int32_t side, int32_t uplo, int32_t trans, int32_t diag,
                                int64_t m, int64_t n, hsma_double_complex alpha,
                                const hsma_double_complex *A, int64_t lda, hsma_double_complex *B,
                                int64_t ldb, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<c64>(side, uplo, trans, diag, m, n, from_abi(alpha),
                                         (const c64 *)A, lda, 0, (c64 *)B, ldb, 0, 1, stream))
}

hsma_status hsma_trsm_strided_batched_general_s(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n, float alpha,
                                                const float *A, int64_t lda, int64_t strideA,
                                                float *B, int64_t ldb, int64_t strideB,
                                                int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<float>(side, uplo, trans, diag, m, n, alpha, A, lda, strideA, B,
                                           ldb, strideB, batch_count, stream))
}
hsma_status hsma_trsm_strided_batched_general_d(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n, double alpha,
                                                const double *A, int64_t lda, int64_t strideA,
                                                double *B, int64_t ldb, int64_t strideB,
                                                int64_t batch_count, void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<double>(side, uplo, trans, diag, m, n, alpha, A, lda, strideA,
                                            B, ldb, strideB, batch_count, stream))
}
hsma_status hsma_trsm_strided_batched_general_c(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n,
                                                hsma_float_complex alpha,
                                                const hsma_float_complex *A, int64_t lda,
                                                int64_t strideA, hsma_float_complex *B,
                                                int64_t ldb, int64_t strideB, int64_t batch_count,
                                                void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<c32>(side, uplo, trans, diag, m, n, from_abi(alpha),
                                         (const c32 *)A, lda, strideA, (c32 *)B, ldb, strideB,
                                         batch_count, stream))
}
hsma_status hsma_trsm_strided_batched_general_z(int32_t side, int32_t uplo, int32_t trans,
                                                int32_t diag, int64_t m, int64_t n,
                                                hsma_double_complex alpha,
                                                const hsma_double_complex *A, int64_t lda,
                                                int64_t strideA, hsma_double_complex *B,
                                                int64_t ldb, int64_t strideB, int64_t batch_count,
                                                void *stream)
{
    HSMA_NOEXCEPT(trsm_variant_impl<c64>(side, uplo, trans, diag, m, n, from_abi(alpha),
                                         (const c64 *)A, lda, strideA, (c64 *)B, ldb, strideB,
                                         batch_count, stream))
}

int32_t hsma_trsm_block_size(int32_t dtype, int64_t m, int64_t n)
{
    if (dtype < 0 || dtype > 3) return -1;
    if (m <= 64) return 0;
    return choose_nb(dtype, m, n > 0 ? n : 1);
}

const char *hsma_status_string(hsma_status status)
{
    switch (status) {
    case HSMA_STATUS_SUCCESS: return "success";
    case HSMA_STATUS_INVALID_SIZE: return "invalid size";
    case HSMA_STATUS_INVALID_POINTER: return "invalid pointer";
    case HSMA_STATUS_NOT_SUPPORTED: return "not supported";
    case HSMA_STATUS_ALLOC_FAILED: return "workspace allocation failed";
    case HSMA_STATUS_HIP_ERROR: return "HIP error";
    case HSMA_STATUS_INVALID_VALUE: return "invalid value";
    case HSMA_STATUS_SCRATCH_TOO_SMALL: return "problem exceeds the no-allocation scratch";
    default: return "unknown status";
    }
}

}  // extern "C"
