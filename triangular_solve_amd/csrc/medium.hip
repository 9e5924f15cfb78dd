// medium.hip - SOLVE_TRI (ggml layout, f32) for 64 < n <= 256.
//
// llama.cpp PR #17457 ("SOLVE_TRI CUDA kernel for small matrices") keeps the
// whole system in one thread block and reports n = 128 ([128,128,4,1]) as
// not supported. Here the rows are cut into blocks of 64 and solved in
// block-row order, the forward substitution applied blockwise:
//
//   X_r = A_rr^{-1} (B_r - sum_{c < r} A_rc X_c),
//
// the update by update_kernel (lane = row, all finished rows above at once)
// and the diagonal solve by the lane-per-row small-regime kernel, in place
// on X. Each block row is two launches on the caller's stream.
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

constexpr int kUpdCols = 8;  // right-hand-side columns per update workgroup

// X[r0 + i][c] = B[r0 + i][c] - sum_{j < r0} A[r0 + i][j] X[j][c] for the rows
// i < rows of the block row starting at r0 and columns c of this workgroup.
// One wave per (problem, group of kUpdCols columns); row-major ggml strides in
// elements (row stride s*1, batch strides s*2, s*3).
__global__ void __launch_bounds__(64) update_kernel(const float *__restrict__ A, int64_t sA1,
                                                    int64_t sA2, int64_t sA3,
                                                    const float *__restrict__ B, int64_t sB1,
                                                    int64_t sB2, int64_t sB3, float *X,
                                                    int64_t sX1, int64_t sX2, int64_t sX3,
                                                    int r0, int rows, int64_t k, int64_t ne02)
{
    const int64_t b = blockIdx.x;
    const int64_t i2 = b % ne02, i3 = b / ne02;
    const int lane = threadIdx.x;
    const bool live = lane < rows;
    const int64_t i = r0 + (live ? lane : 0);
    const int64_t c0 = (int64_t)blockIdx.y * kUpdCols;
    const float *Ar = A + i2 * sA2 + i3 * sA3 + i * sA1;
    const float *Bb = B + i2 * sB2 + i3 * sB3;
    float *Xb = X + i2 * sX2 + i3 * sX3;

    float acc[kUpdCols];
#pragma unroll
    for (int c = 0; c < kUpdCols; ++c) {
        const int64_t cc = c0 + c < k ? c0 + c : k - 1;  // columns past k repeat a valid one
        acc[c] = Bb[i * sB1 + cc];
    }
    for (int j = 0; j < r0; ++j) {
        const float a = Ar[j];
        const float *xr = Xb + (int64_t)j * sX1;
#pragma unroll
        for (int c = 0; c < kUpdCols; ++c) {
            const int64_t cc = c0 + c < k ? c0 + c : k - 1;
            acc[c] = __builtin_fmaf(-a, xr[cc], acc[c]);
        }
    }
    if (live) {
#pragma unroll
        for (int c = 0; c < kUpdCols; ++c)
            if (c0 + c < k) Xb[i * sX1 + c0 + c] = acc[c];
    }
}

hipError_t solve_tri_medium(int64_t n, int64_t k, const float *A, const float *B, float *X,
                            int64_t ne02, int64_t ne03, int64_t sA1, int64_t sA2, int64_t sA3,
                            int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1, int64_t sX2,
                            int64_t sX3, hipStream_t s)
{
    const int64_t nprob = ne02 * ne03;
    const int64_t ychunks = (k + kUpdCols - 1) / kUpdCols;
    if (nprob > 0x7fffffff || ychunks > 65535) return hipErrorInvalidConfiguration;
    for (int64_t r0 = 0; r0 < n; r0 += 64) {
        const int64_t rows = n - r0 < 64 ? n - r0 : 64;
        const float *Brow = B + r0 * sB1;
        int64_t sb1 = sB1, sb2 = sB2, sb3 = sB3;
        if (r0 > 0) {
            hipLaunchKernelGGL(update_kernel, dim3((unsigned)nprob, (unsigned)ychunks), dim3(64), 0, s,
                               A, sA1, sA2, sA3, B, sB1, sB2, sB3, X, sX1, sX2, sX3, (int)r0,
                               (int)rows, k, ne02);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            // the diagonal solve then runs in place on the updated rows of X
            Brow = X + r0 * sX1;
            sb1 = sX1; sb2 = sX2; sb3 = sX3;
        }
        hipError_t e = small_rowlane<float>(A + r0 * sA1 + r0, sA1, 1, sA2, sA3, Brow, sb1, 1, sb2,
                                            sb3, X + r0 * sX1, sX1, 1, sX2, sX3, rows, k, ne02,
                                            ne03, 1.0f, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hsma
