// variants.hip - strided tile copies that bring the other TRSM variants to the
// canonical left-side lower-triangular form.
//
// The pages' method is the left-side lower-triangular solve; the variants
// (right side, upper triangle, transposed or conjugate-transposed A, unit
// diagonal) are the usual BLAS ones, which the news summary of the
// HSMA-TRSM paper lists as untested ("A result tied to a narrow
// benchmark"). Each variant is the canonical solve of Ahat Y = alpha Bhat
// for strided views Ahat (A, A^T, A^H or their index-reversed forms) and
// Bhat (B, B with reversed rows, B^T or B^T with reversed rows). The small
// regime reads those views directly; the blocked regime gathers the lower
// triangle of Ahat and all of Bhat into column-major workspace with
// tile_copy, runs the canonical blocked solve there and scatters X back.
//
// tile_copy moves 32 x 32 tiles through LDS, so that both the source and
// the destination are accessed along their contiguous dimension (for a
// transposing copy one side is contiguous along rows, the other along
// columns).
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

template <typename T>
struct CopyArgs {
    const T *src;
    int64_t ssi, ssj, ssb;
    T *dst;
    int64_t dsi, dsj, dsb;
    int64_t rows, cols;
    T alpha;
    int scale, conj, unit, lower;
};

constexpr int kTile = 32;

// SRC_I / DST_I: the source / destination is contiguous along i (else along j).
template <typename T, bool SRC_I, bool DST_I>
__global__ void __launch_bounds__(256) tile_copy_kernel(CopyArgs<T> p)
{
    __shared__ T tile[kTile][kTile + 1];
    const int64_t i0 = (int64_t)blockIdx.x * kTile, j0 = (int64_t)blockIdx.y * kTile;
    if (p.lower && j0 > i0 + kTile - 1) return;   // tile wholly above the diagonal
    const T *src = p.src + (int64_t)blockIdx.z * p.ssb;
    T *dst = p.dst + (int64_t)blockIdx.z * p.dsb;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;

    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    auto inside = [&](int64_t i, int64_t j) {
        return i < p.rows && j < p.cols && (!p.lower || j <= i);
    };
#pragma unroll
    for (int r = 0; r < kTile / 8; ++r) {
        const int a = SRC_I ? tx : ty + 8 * r;   // tile row (i - i0)
        const int b = SRC_I ? ty + 8 * r : tx;   // tile column (j - j0)
        const int64_t i = i0 + a, j = j0 + b;
        if (inside(i, j)) {
            T v;
            if (p.unit && i == j) {
                v = one;
            } else {
                v = src[i * p.ssi + j * p.ssj];
                if constexpr (traits<T>::is_complex) {
                    if (p.conj) v.im = -v.im;
                }
                if (p.scale) v = mul(p.alpha, v);
            }
            tile[a][b] = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kTile / 8; ++r) {
        const int a = DST_I ? tx : ty + 8 * r;
        const int b = DST_I ? ty + 8 * r : tx;
        const int64_t i = i0 + a, j = j0 + b;
        if (inside(i, j)) dst[i * p.dsi + j * p.dsj] = tile[a][b];
    }
}

template <typename T>
hipError_t tile_copy(const T *src, int64_t ssi, int64_t ssj, int64_t ssb, T *dst, int64_t dsi,
                     int64_t dsj, int64_t dsb, int64_t rows, int64_t cols, int64_t batch,
                     bool lower, bool conj, bool unit, const T *alpha, hipStream_t s)
{
    if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
    CopyArgs<T> p;
    p.src = src; p.ssi = ssi; p.ssj = ssj; p.ssb = ssb;
    p.dst = dst; p.dsi = dsi; p.dsj = dsj; p.dsb = dsb;
    p.rows = rows; p.cols = cols;
    p.alpha = alpha ? *alpha : zero_of(T());
    p.scale = alpha ? 1 : 0;
    p.conj = conj ? 1 : 0;
    p.unit = unit ? 1 : 0;
    p.lower = lower ? 1 : 0;
    const int64_t gx = (rows + kTile - 1) / kTile, gy = (cols + kTile - 1) / kTile;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
    // contiguous dimension of each side (a unit stride, either sign)
    const bool si = ssi == 1 || ssi == -1 || !(ssj == 1 || ssj == -1);
    const bool di = dsi == 1 || dsi == -1 || !(dsj == 1 || dsj == -1);
    const int64_t kMaxZ = 65535;
    for (int64_t b0 = 0; b0 < batch; b0 += kMaxZ) {
        const int64_t nb = batch - b0 < kMaxZ ? batch - b0 : kMaxZ;
        CopyArgs<T> q = p;
        q.src = src + b0 * ssb;
        q.dst = dst + b0 * dsb;
        const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)nb);
        if (si && di) hipLaunchKernelGGL((tile_copy_kernel<T, true, true>), grid, dim3(256), 0, s, q);
        else if (si) hipLaunchKernelGGL((tile_copy_kernel<T, true, false>), grid, dim3(256), 0, s, q);
        else if (di) hipLaunchKernelGGL((tile_copy_kernel<T, false, true>), grid, dim3(256), 0, s, q);
        else hipLaunchKernelGGL((tile_copy_kernel<T, false, false>), grid, dim3(256), 0, s, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

#define HSMA_INST(T)                                                                              \
    template hipError_t tile_copy<T>(const T *, int64_t, int64_t, int64_t, T *, int64_t, int64_t,  \
                                     int64_t, int64_t, int64_t, int64_t, bool, bool, bool,         \
                                     const T *, hipStream_t);
HSMA_INST(float)
HSMA_INST(double)
HSMA_INST(c32)
HSMA_INST(c64)
#undef HSMA_INST

}  // namespace hsma
