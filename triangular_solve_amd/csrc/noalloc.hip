// noalloc.hip - hsma_trsm_noalloc: the solve of hsma_trsm_{s,d,c,z} without
// any device allocation, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The blocked path's workspace (inverted diagonal blocks, the solved block
// row W and the blocked-inverse merge temporaries) comes from `scratch`, a
// fixed device array of kScratchBytes that every GPU the library runs on
// holds until the process ends. Its device address is taken once per device
// with hipGetSymbolAddress; host code uses that address, never the array's
// name (which on the host is only a stand-in for the symbol).
//
// The scratch bounds the block size: N_B is the table's choice, halved until
// the inverted blocks take at most half of the scratch; the rest holds W for
// as many right-hand-side columns as fit, and B is solved in column chunks
// of that width after one inversion. All calls on one GPU share its scratch,
// so calls that overlap in time on one GPU (different streams or threads)
// race; nothing in the scratch needs to start at zero.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>

#include "hsma_trsm.h"
#include "common.hpp"
#include "internal.hpp"

namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
}

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace hsma {
namespace {

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// Device address of this device's scratch, looked up on the first call on
// the device (with the device current).
hipError_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Usable scratch bytes: kScratchBytes, or less when HSMA_NOALLOC_LIMIT (a
// byte count, for tests of the chunked and too-large cases) asks for less.
size_t usable_bytes()
{
    size_t b = kScratchBytes;
    if (const char *s = std::getenv("HSMA_NOALLOC_LIMIT")) {
        char *end = nullptr;
        const unsigned long long v = std::strtoull(s, &end, 10);
        if (end != s && v < b) b = (size_t)v;
    }
    return b;
}

struct Plan {
    int nb;
    int64_t nc;   // right-hand-side columns per chunk
};

// Block size and column chunk that fit the scratch; false if none does.
bool make_plan(int dtype, int64_t m, int64_t n, size_t elem, Plan *out)
{
    const int64_t budget = (int64_t)(usable_bytes() / elem);
    int nb = choose_nb(dtype, m, n);
    while (true) {
        const int64_t nt = (m + nb - 1) / nb;
        const int64_t inv = nt * (int64_t)nb * nb;
        const int64_t rest = budget - inv;
        if (inv <= budget / 2 && rest >= blocked_inverse_temp_elems(m, nb) && rest >= nb) {
            out->nb = nb;
            out->nc = rest / nb < n ? rest / nb : n;
            return true;
        }
        if (nb <= 16) return false;
        nb = (nb / 2) & ~15;
        if (nb < 16) nb = 16;
    }
}

template <typename T>
hsma_status noalloc_impl(int64_t m, int64_t n, T alpha, const T *A, int64_t lda, T *B,
                         int64_t ldb, void *stream)
{
    constexpr int dt = traits<T>::dtype;
    if (m < 0 || n < 0) return HSMA_STATUS_INVALID_SIZE;
    if (lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1)) return HSMA_STATUS_INVALID_SIZE;
    if (m == 0 || n == 0) return HSMA_STATUS_SUCCESS;
    if (!B) return HSMA_STATUS_INVALID_POINTER;
    hipStream_t s = (hipStream_t)stream;
    if (is_zero(alpha))
        return scale_matrix<T>(B, m, n, ldb, 0, 1, alpha, true, s) == hipSuccess
                   ? HSMA_STATUS_SUCCESS : HSMA_STATUS_HIP_ERROR;
    if (!A) return HSMA_STATUS_INVALID_POINTER;
    if (m <= 64)   // the small regime uses no workspace
        return small_path<T>(m, n, alpha, A, lda, 0, B, ldb, 0, 1, s) == hipSuccess
                   ? HSMA_STATUS_SUCCESS : HSMA_STATUS_HIP_ERROR;

    Plan pl;
    if (!make_plan(dt, m, n, sizeof(T), &pl)) return HSMA_STATUS_SCRATCH_TOO_SMALL;
    void *base = nullptr;
    if (scratch_address(&base) != hipSuccess) return HSMA_STATUS_HIP_ERROR;
    const int64_t nt = (m + pl.nb - 1) / pl.nb;
    T *invA = (T *)base;
    T *W = invA + nt * (int64_t)pl.nb * pl.nb;   // also the inversion's temporary
    hipError_t e = hipSuccess;
    if (!is_one(alpha)) e = scale_matrix<T>(B, m, n, ldb, 0, 1, alpha, false, s);
    if (e == hipSuccess) e = blocked_invert<T>(m, pl.nb, pl.nb / 8 > 0 ? pl.nb / 8 : 1, A, lda, invA, W, s);
    for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += pl.nc) {
        const int64_t nc = n - c0 < pl.nc ? n - c0 : pl.nc;
        e = blocked_apply<T>(m, nc, pl.nb, A, lda, invA, B + c0 * ldb, ldb, W, s);
    }
    return e == hipSuccess ? HSMA_STATUS_SUCCESS : HSMA_STATUS_HIP_ERROR;
}

}  // namespace
}  // namespace hsma

using namespace hsma;

extern "C" hsma_status hsma_trsm_noalloc(int32_t dtype, int64_t m, int64_t n, const void *alpha,
                                         const void *A, int64_t lda, void *B, int64_t ldb,
                                         void *stream)
{
    try {
        if (!alpha) return HSMA_STATUS_INVALID_POINTER;
        switch (dtype) {
        case HSMA_DTYPE_F32:
            return noalloc_impl<float>(m, n, *(const float *)alpha, (const float *)A, lda,
                                       (float *)B, ldb, stream);
        case HSMA_DTYPE_F64:
            return noalloc_impl<double>(m, n, *(const double *)alpha, (const double *)A, lda,
                                        (double *)B, ldb, stream);
        case HSMA_DTYPE_C64: {
            const hsma_float_complex a = *(const hsma_float_complex *)alpha;
            return noalloc_impl<c32>(m, n, c32{a.re, a.im}, (const c32 *)A, lda, (c32 *)B, ldb,
                                     stream);
        }
        case HSMA_DTYPE_C128: {
            const hsma_double_complex a = *(const hsma_double_complex *)alpha;
            return noalloc_impl<c64>(m, n, c64{a.re, a.im}, (const c64 *)A, lda, (c64 *)B, ldb,
                                     stream);
        }
        default: return HSMA_STATUS_INVALID_VALUE;
        }
    } catch (...) {
        return HSMA_STATUS_HIP_ERROR;
    }
}
