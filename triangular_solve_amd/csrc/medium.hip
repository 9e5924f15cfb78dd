// medium.hip - SOLVE_TRI (ggml layout, f32) for 64 < n <= 256.
//
// llama.cpp PR #17457 ("SOLVE_TRI CUDA kernel for small matrices") keeps the
// whole system in one thread block and reports n = 128 ([128,128,4,1]) as
// not supported. Here the rows are cut into blocks of 64, one wave per block
// row in one workgroup per (problem, group of right-hand sides), and solved
// in block-row order, the forward substitution applied blockwise:
//
//   X_r = A_rr^{-1} (B_r - sum_{c < r} A_rc X_c),
//
// one launch for any n <= 256 (solve_tri_128_kernel for two block rows,
// solve_tri_256_kernel for three or four).
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

// Forward substitution of one wave's 64 rows (lane = row), coefficients
// a[j] = a_ij / a_ii below the diagonal and 0 elsewhere, w = b / a_ii. Step j
// updates only the rows below j, so finished rows keep their values even
// when a later x_j is inf or NaN.
template <int KW>
__device__ __forceinline__ void wave_substitute(const float (&a)[64], float (&w)[KW])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
        const bool below = j < lane;
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const float u = __builtin_fmaf(-a[j], readlane(w[q], j), w[q]);
            w[q] = below ? u : w[q];
        }
    }
}

// 64 < n <= 128 in one launch: two waves per (problem, group of KW columns),
// lane = row. Every lane first loads its row of A into registers (16-byte
// loads when VEC: rows 16-byte aligned), all before the barrier. Wave 0
// solves rows 0..63 (x_j broadcast with v_readlane) and publishes them in LDS;
// after the barrier wave 1 subtracts A21 X1 (the finished rows read as LDS
// broadcasts) and solves rows 64..n-1 the same way. Coefficients are scaled
// by the row's 1/a_ii, as in the small regime.
template <int KW, bool VEC>
__global__ void __launch_bounds__(128) solve_tri_128_kernel(
    const float *__restrict__ A, int64_t sA1, int64_t sA2, int64_t sA3, const float *__restrict__ B,
    int64_t sB1, int64_t sB2, int64_t sB3, float *__restrict__ X, int64_t sX1, int64_t sX2,
    int64_t sX3, int n, int64_t k, int64_t ne02)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ float xs[64 * KW];
    const int64_t b = blockIdx.x;
    const int64_t i2 = b % ne02, i3 = b / ne02;
    const int64_t c0 = (int64_t)blockIdx.y * KW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = wave * 64 + lane;          // row of this lane
    const bool live = i < n;
    const float *Ar = A + i2 * sA2 + i3 * sA3 + (int64_t)(live ? i : 0) * sA1;
    const float *Bb = B + i2 * sB2 + i3 * sB3;
    float *Xb = X + i2 * sX2 + i3 * sX3;

    // columns 0..63 of the row (wave 0: its diagonal block; wave 1: A21) and,
    // for wave 1, columns 64..127 (its diagonal block); columns past n are 0
    float lo[64], hi[64];
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
        if (VEC) {
            const f4 v = *(const f4 *)(Ar + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) lo[c + e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) lo[c + e] = Ar[c + e];
        }
    }
#pragma unroll
    for (int c = 0; c < 64; ++c) hi[c] = 0.0f;
    if (wave == 1) {
#pragma unroll
        for (int c = 0; c < 64; c += 4) {
            if (VEC && 64 + c + 4 <= n) {
                const f4 v = *(const f4 *)(Ar + 64 + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[c + e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[c + e] = 64 + c + e < n ? Ar[64 + c + e] : 0.0f;
            }
        }
    }
    const float inv = live ? 1.0f / Ar[i] : 1.0f;
    float w[KW];
#pragma unroll
    for (int q = 0; q < KW; ++q)
        w[q] = (live && c0 + q < k) ? Bb[(int64_t)i * sB1 + c0 + q] : 0.0f;

    // coefficients of this wave's diagonal block: columns wave*64 + j
    float a[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) {
        const float v = wave == 0 ? lo[j] : hi[j];
        a[j] = (live && wave * 64 + j < i) ? v * inv : 0.0f;
    }

    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < KW; ++q) w[q] *= inv;
        wave_substitute<KW>(a, w);
#pragma unroll
        for (int q = 0; q < KW; ++q) xs[lane * KW + q] = w[q];
    }
    __syncthreads();
    if (wave == 1) {
        // rows 64..n-1: subtract A21 X1, then solve with the diagonal block
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const float aij = live ? lo[j] : 0.0f;
#pragma unroll
            for (int q = 0; q < KW; ++q) w[q] = __builtin_fmaf(-aij, xs[j * KW + q], w[q]);
        }
#pragma unroll
        for (int q = 0; q < KW; ++q) w[q] *= inv;
        wave_substitute<KW>(a, w);
    }
    if (live) {
#pragma unroll
        for (int q = 0; q < KW; ++q)
            if (c0 + q < k) Xb[(int64_t)i * sX1 + c0 + q] = w[q];
    }
}

template <int KW>
static hipError_t launch_128(bool vec, int64_t n, int64_t k, const float *A, const float *B,
                             float *X, int64_t nprob, int64_t ne02, int64_t sA1, int64_t sA2,
                             int64_t sA3, int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1,
                             int64_t sX2, int64_t sX3, hipStream_t s)
{
    const int64_t chunks = (k + KW - 1) / KW;
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nprob, (unsigned)chunks);
    if (vec)
        hipLaunchKernelGGL((solve_tri_128_kernel<KW, true>), grid, dim3(128), 0, s, A, sA1, sA2, sA3,
                           B, sB1, sB2, sB3, X, sX1, sX2, sX3, (int)n, k, ne02);
    else
        hipLaunchKernelGGL((solve_tri_128_kernel<KW, false>), grid, dim3(128), 0, s, A, sA1, sA2,
                           sA3, B, sB1, sB2, sB3, X, sX1, sX2, sX3, (int)n, k, ne02);
    return hipGetLastError();
}

// 128 < n <= 256 in one launch: four waves per (problem, group of KW
// columns), lane = row, wave w owning rows 64w .. 64w+63. At stage s wave s
// solves its diagonal block (its rows already hold B_s - sum_{c<s} A_sc X_c)
// and publishes X_s in LDS; after the barrier every later wave subtracts
// A_ws X_s, reading its row's 64 coefficients of block s from memory (16-byte
// loads when VEC) and X_s as LDS broadcasts. Coefficients of the diagonal
// block are scaled by the row's 1/a_ii, as in the small regime.
template <int KW, bool VEC>
__global__ void __launch_bounds__(256) solve_tri_256_kernel(
    const float *__restrict__ A, int64_t sA1, int64_t sA2, int64_t sA3, const float *__restrict__ B,
    int64_t sB1, int64_t sB2, int64_t sB3, float *__restrict__ X, int64_t sX1, int64_t sX2,
    int64_t sX3, int n, int64_t k, int64_t ne02)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ float xs[256 * KW];
    const int64_t b = blockIdx.x;
    const int64_t i2 = b % ne02, i3 = b / ne02;
    const int64_t c0 = (int64_t)blockIdx.y * KW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = wave * 64 + lane;          // row of this lane
    const bool live = i < n;
    const int nblk = (n + 63) / 64;          // 3 or 4, the same for every wave
    const float *Ar = A + i2 * sA2 + i3 * sA3 + (int64_t)(live ? i : 0) * sA1;
    const float *Bb = B + i2 * sB2 + i3 * sB3;
    float *Xb = X + i2 * sX2 + i3 * sX3;

    // the row's coefficients in columns 64c .. 64c+63 (0 past n)
    auto load_block = [&](int c, float (&v)[64]) {
        const int base = 64 * c;
#pragma unroll
        for (int t = 0; t < 64; t += 4) {
            if (VEC && base + t + 4 <= n) {
                const f4 x = *(const f4 *)(Ar + base + t);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[t + e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[t + e] = base + t + e < n ? Ar[base + t + e] : 0.0f;
            }
        }
    };

    const float inv = live ? 1.0f / Ar[i] : 1.0f;
    float w[KW];
#pragma unroll
    for (int q = 0; q < KW; ++q)
        w[q] = (live && c0 + q < k) ? Bb[(int64_t)i * sB1 + c0 + q] : 0.0f;
    float a[64];
    if (wave < nblk) {
        float v[64];
        load_block(wave, v);
#pragma unroll
        for (int j = 0; j < 64; ++j) a[j] = (live && j < lane) ? v[j] * inv : 0.0f;
    } else {
#pragma unroll
        for (int j = 0; j < 64; ++j) a[j] = 0.0f;
    }

    for (int s = 0; s < nblk; ++s) {
        if (wave == s) {
#pragma unroll
            for (int q = 0; q < KW; ++q) w[q] *= inv;
            wave_substitute<KW>(a, w);
#pragma unroll
            for (int q = 0; q < KW; ++q) xs[(64 * s + lane) * KW + q] = w[q];
        }
        __syncthreads();
        if (wave > s && wave < nblk) {
            float v[64];
            load_block(s, v);
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                const float aij = live ? v[j] : 0.0f;
#pragma unroll
                for (int q = 0; q < KW; ++q)
                    w[q] = __builtin_fmaf(-aij, xs[(64 * s + j) * KW + q], w[q]);
            }
        }
    }
    if (live) {
#pragma unroll
        for (int q = 0; q < KW; ++q)
            if (c0 + q < k) Xb[(int64_t)i * sX1 + c0 + q] = w[q];
    }
}

template <int KW>
static hipError_t launch_256(bool vec, int64_t n, int64_t k, const float *A, const float *B,
                             float *X, int64_t nprob, int64_t ne02, int64_t sA1, int64_t sA2,
                             int64_t sA3, int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1,
                             int64_t sX2, int64_t sX3, hipStream_t s)
{
    const int64_t chunks = (k + KW - 1) / KW;
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nprob, (unsigned)chunks);
    if (vec)
        hipLaunchKernelGGL((solve_tri_256_kernel<KW, true>), grid, dim3(256), 0, s, A, sA1, sA2, sA3,
                           B, sB1, sB2, sB3, X, sX1, sX2, sX3, (int)n, k, ne02);
    else
        hipLaunchKernelGGL((solve_tri_256_kernel<KW, false>), grid, dim3(256), 0, s, A, sA1, sA2,
                           sA3, B, sB1, sB2, sB3, X, sX1, sX2, sX3, (int)n, k, ne02);
    return hipGetLastError();
}

hipError_t solve_tri_medium(int64_t n, int64_t k, const float *A, const float *B, float *X,
                            int64_t ne02, int64_t ne03, int64_t sA1, int64_t sA2, int64_t sA3,
                            int64_t sB1, int64_t sB2, int64_t sB3, int64_t sX1, int64_t sX2,
                            int64_t sX3, hipStream_t s)
{
    const int64_t nprob = ne02 * ne03;
    if (nprob > 0x7fffffff || n <= 64 || n > 256) return hipErrorInvalidValue;
    // fewer columns per workgroup shorten each wave's dependent chain; more
    // share the row loads of A
    const bool vec = (uintptr_t)A % 16 == 0 && (sA1 * 4) % 16 == 0 && (sA2 * 4) % 16 == 0 &&
                     (sA3 * 4) % 16 == 0;
    if (n <= 128) {
        if (k <= 8) return launch_128<2>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
        if (k <= 32) return launch_128<4>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
        return launch_128<8>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
    }
    if (k <= 8) return launch_256<2>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
    if (k <= 32) return launch_256<4>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
    return launch_256<8>(vec, n, k, A, B, X, nprob, ne02, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3, s);
}

}  // namespace hsma
