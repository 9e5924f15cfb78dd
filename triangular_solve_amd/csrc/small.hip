// small.hip - the small regime (m <= 64): direct forward substitution on chip.
//
// HSMA-TRSM paper, small-scale section: for m, n <= 64 the whole triangle is
// kept on chip and the system is solved directly, overlapping memory traffic
// with arithmetic. Its 64 KB / 48 KB shared-memory partitioning (and the
// dual thread-group pipeline it needs for double complex at m = 64) comes
// from DCU and NVIDIA budgets; on gfx950 a 64 x 64 double-complex A and B fit
// together, so this file keeps the on-chip direct solve and re-derives the
// layout for 64-wide wavefronts instead.
//
// Two kernels:
//
//  * colane  - one wavefront per (problem, group of 64 right-hand sides),
//    lane = right-hand-side column. The column lives in VGPRs, so the
//    substitution needs no cross-lane traffic at all: every coefficient a_ij
//    is wave-uniform and is read with scalar loads straight into SGPRs, and
//    each one feeds one FMA per lane. This is the throughput kernel for
//    batches of 64 x 64 column-major problems. For double complex the 64-row
//    column does not fit the register file, so the column is processed as
//    row panels: a later panel first subtracts the contributions of earlier
//    panels, reading their finished x values back from the output (the
//    2 x 2 block step of the paper's double-complex scheme: solve with A11,
//    update with A21, solve with A22).
//
//  * rowlane - one workgroup per problem, lane = row. The diagonal-scaled
//    triangle is staged in LDS (transposed so step j reads one contiguous
//    LDS column), each wave owns a few right-hand-side columns in VGPRs, and
//    step j broadcasts x_j from lane j with v_readlane. No barrier inside the
//    substitution, any m <= 64, any strides (column-major or the row-major
//    ggml layout), in place or out of place. This is the latency kernel for
//    few right-hand sides (the SOLVE_TRI shape) and the general fallback.
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

// ---------------------------------------------------------------------------
// rowlane

template <typename T>
struct RowlaneArgs {
    const T *A;
    const T *B;
    T *X;
    int m, n;
    int64_t sai, saj, sbi, sbj, sxi, sxj;
    int64_t ne02;
    int64_t sa2, sa3, sb2, sb3, sx2, sx3;
    T alpha;
};

constexpr int kLdsStride = 65;  // padded LDS column stride of the staged triangle

template <typename T, int KW>
__global__ void __launch_bounds__(256) rowlane_kernel(RowlaneArgs<T> p)
{
    __shared__ T AT[64 * kLdsStride];
    __shared__ T sinv[64];

    const int64_t b = blockIdx.x;
    const int64_t i2 = b % p.ne02, i3 = b / p.ne02;
    const T *Ab = p.A + i2 * p.sa2 + i3 * p.sa3;
    const T *Bb = p.B + i2 * p.sb2 + i3 * p.sb3;
    T *Xb = p.X + i2 * p.sx2 + i3 * p.sx3;
    const int m = p.m;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nthr = blockDim.x;

    if (tid < 64) {
        T one = zero_of(T());
        if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
        const T d = tid < m ? Ab[tid * (p.sai + p.saj)] : one;
        sinv[tid] = recip(d);
    }
    __syncthreads();

    // Stage tril(A) scaled by its row's inverse diagonal, strictly lower part
    // only (diagonal and above are zero), transposed: AT[j][i] = a_ij / a_ii.
    // The walk order follows the storage so global reads coalesce.
    const bool colmajor = p.sai == 1;
    for (int idx = tid; idx < 64 * 64; idx += nthr) {
        const int i = colmajor ? (idx & 63) : (idx >> 6);
        const int j = colmajor ? (idx >> 6) : (idx & 63);
        T v = zero_of(T());
        if (i < m && j < i) v = mul(Ab[i * p.sai + j * p.saj], sinv[i]);
        AT[j * kLdsStride + i] = v;
    }

    // This wave's right-hand-side columns, one row per lane, pre-scaled the
    // same way: w_i = alpha * b_i / a_ii.
    const int c0 = (blockIdx.y * (nthr >> 6) + wave) * KW;
    const T inv = sinv[lane];
    T w[KW];
#pragma unroll
    for (int q = 0; q < KW; ++q) {
        const int c = c0 + q;
        w[q] = zero_of(T());
        if (lane < m && c < p.n) w[q] = mul(mul(p.alpha, Bb[lane * p.sbi + c * p.sbj]), inv);
    }
    __syncthreads();

    // Forward substitution. After step j-1, lane j holds the finished x_j;
    // every lane below subtracts its (scaled) a_ij * x_j. Lanes at or above
    // j read a zero coefficient and keep their value.
    for (int j = 0; j < m; ++j) {
        const T a = AT[j * kLdsStride + lane];
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const T x = readlane(w[q], j);
            w[q] = fms(w[q], a, x);
        }
    }

#pragma unroll
    for (int q = 0; q < KW; ++q) {
        const int c = c0 + q;
        if (lane < m && c < p.n) Xb[lane * p.sxi + c * p.sxj] = w[q];
    }
}

template <typename T, int KW>
static hipError_t rowlane_launch(const RowlaneArgs<T> &p, int64_t nprob, int nwaves,
                                 hipStream_t s)
{
    const int per_block = nwaves * KW;
    const int64_t ychunks = (p.n + per_block - 1) / per_block;
    if (ychunks > 65535) return hipErrorInvalidConfiguration;
    if (nprob > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rowlane_kernel<T, KW>), dim3((unsigned)nprob, (unsigned)ychunks),
                       dim3(64 * nwaves), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t small_rowlane(const T *A, int64_t sai, int64_t saj, int64_t sa2, int64_t sa3,
                         const T *B, int64_t sbi, int64_t sbj, int64_t sb2, int64_t sb3,
                         T *X, int64_t sxi, int64_t sxj, int64_t sx2, int64_t sx3,
                         int64_t m, int64_t n, int64_t ne02, int64_t ne03, T alpha, hipStream_t s)
{
    RowlaneArgs<T> p;
    p.A = A; p.B = B; p.X = X;
    p.m = (int)m; p.n = (int)n;
    p.sai = sai; p.saj = saj; p.sbi = sbi; p.sbj = sbj; p.sxi = sxi; p.sxj = sxj;
    p.ne02 = ne02;
    p.sa2 = sa2; p.sa3 = sa3; p.sb2 = sb2; p.sb3 = sb3; p.sx2 = sx2; p.sx3 = sx3;
    p.alpha = alpha;
    const int64_t nprob = ne02 * ne03;
    // Columns per wave and waves per workgroup: spread few right-hand sides
    // over several waves (latency), more of them into registers (throughput).
    if (n <= 1) return rowlane_launch<T, 1>(p, nprob, 1, s);
    if (n <= 4) return rowlane_launch<T, 1>(p, nprob, (int)n, s);
    if (n <= 8) return rowlane_launch<T, 2>(p, nprob, (int)((n + 1) / 2), s);
    if (n <= 16) return rowlane_launch<T, 4>(p, nprob, (int)((n + 3) / 4), s);
    if (traits<T>::is_complex && sizeof(T) == 16) return rowlane_launch<T, 4>(p, nprob, 4, s);
    if (n <= 32) return rowlane_launch<T, 8>(p, nprob, (int)((n + 7) / 8), s);
    return rowlane_launch<T, 16>(p, nprob, 4, s);
}

// ---------------------------------------------------------------------------
// colane

template <typename T>
using cptr = const __attribute__((address_space(4))) T *;

// Wave-uniform read through the constant address space (scalar loads).
template <typename T>
__device__ __forceinline__ T ld_uniform(cptr<T> p, int idx)
{
    if constexpr (traits<T>::is_complex) {
        using R = typename traits<T>::real;
        const cptr<R> q = (cptr<R>)p;
        return T{q[2 * idx], q[2 * idx + 1]};
    } else {
        return p[idx];
    }
}

// Number of coefficients read per scalar-load group: 16 dwords.
template <typename T>
constexpr int kGroup = (int)(64 / sizeof(T));

// w[r] -= a(row0 + r, col) * x for r in [RLO, P): one column segment of A,
// read as wave-uniform scalars in groups of kGroup so that the SGPR working
// set stays bounded (a scheduling barrier separates the groups).
// Empty asm that makes v look modified after `dep` is available: values
// derived from v cannot be computed before dep. Emits no instruction.
template <typename V, typename T>
__device__ __forceinline__ void order_after(V &v, const T &dep)
{
    if constexpr (traits<T>::is_complex) asm volatile("" : "+s"(v) : "v"(dep.re));
    else asm volatile("" : "+s"(v) : "v"(dep));
}

template <typename T, int P, int RLO>
__device__ __forceinline__ void seg_update(T (&w)[P], cptr<T> acol, T x)
{
    constexpr int G = kGroup<T>;
    static_for<RLO / G, (P + G - 1) / G>([&](auto gi) {
        constexpr int g0 = decltype(gi)::value * G;
        constexpr int lo = g0 > RLO ? g0 : RLO;
        constexpr int hi = g0 + G < P ? g0 + G : P;
        // issue this group's scalar loads only once x exists
        cptr<T> ap = acol;
        order_after(ap, x);
        T a[hi - lo];
        static_for<lo, hi>([&](auto r) { a[r - lo] = ld_uniform<T>(ap, r); });
        static_for<lo, hi>([&](auto r) { w[r] = fms(w[r], a[r - lo], x); });
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <typename T, int NPANEL>
__global__ void __launch_bounds__(256) colane_kernel(const T *__restrict__ A, int64_t lda,
                                                      int64_t strideA, T *__restrict__ B,
                                                      int64_t ldb, int64_t strideB, int64_t n,
                                                      int64_t nchunks, int64_t items, T alpha,
                                                      T alpha_inv)
{
    constexpr int M = 64;
    constexpr int P = M / NPANEL;
    const int lane = threadIdx.x & 63;
    // The wave index is uniform across the wave; readfirstlane tells the
    // compiler so, which keeps the problem's A pointer in SGPRs.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (item >= items) return;  // whole wave leaves together; no barriers below
    const int64_t prob = item / nchunks;
    const int64_t cfirst = (item % nchunks) * 64;
    const int64_t c = cfirst + lane;
    const bool live = c < n;

    const T *Ap = A + prob * strideA;
    const cptr<T> a4 = (cptr<T>)Ap;
    // Lanes past n work on a copy of the wave's first column (always valid)
    // and never store, so loads need no guard.
    T *Bc = B + prob * strideB + (live ? c : cfirst) * ldb;

    // 1/a_ll for this lane's row index l; step j broadcasts lane j's value.
    const T myinv = recip(Ap[lane + lane * lda]);

    static_for<0, NPANEL>([&](auto pi) {
        constexpr int r0 = decltype(pi)::value * P;
        // The solve runs on B itself; alpha is applied to X on the way out
        // (A (alpha^{-1} X) = B has the same substitution with alpha factored out).
        T w[P];
        static_for<0, P>([&](auto r) { w[r] = Bc[r0 + r]; });

        // Contributions of the finished rows above this panel.
        static_for<0, r0>([&](auto k) {
            // reload the finished x_k only after the previous update is issued
            T *bk = Bc + k;
            if constexpr (traits<T>::is_complex) asm volatile("" : "+v"(bk) : "v"(w[P - 1].re));
            else asm volatile("" : "+v"(bk) : "v"(w[P - 1]));
            const T x = mul(*bk, alpha_inv);
            seg_update<T, P, 0>(w, a4 + (r0 + k * lda), x);
        });
        // Substitution inside the panel.
        static_for<0, P>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            // Tie the broadcast of 1/a_jj to w[j] so the compiler cannot hoist
            // all 64 broadcasts to the top (that would exhaust the SGPRs).
            T inv = myinv;
            if constexpr (traits<T>::is_complex) {
                asm volatile("" : "+v"(inv.re), "+v"(inv.im) : "v"(w[j].re), "v"(w[j].im));
            } else {
                asm volatile("" : "+v"(inv) : "v"(w[j]));
            }
            const T x = mul(w[j], readlane(inv, r0 + j));
            w[j] = x;
            if constexpr (j + 1 < P) seg_update<T, P, j + 1>(w, a4 + (r0 + (int64_t)(r0 + j) * lda), x);
        });
        if (live) static_for<0, P>([&](auto r) { Bc[r0 + r] = mul(alpha, w[r]); });
    });
}

template <typename T>
hipError_t small_colane(int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA, T *B,
                        int64_t ldb, int64_t strideB, int64_t batch, hipStream_t s)
{
    const int64_t nchunks = (n + 63) / 64;
    const int64_t items = nchunks * batch;
    const int64_t blocks = (items + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int NP = sizeof(T) == 16 ? 2 : 1;
    // Earlier panels' rows are read back from B already scaled by alpha.
    const T alpha_inv = host_recip(alpha);
    hipLaunchKernelGGL((colane_kernel<T, NP>), dim3((unsigned)blocks), dim3(256), 0, s, A, lda,
                       strideA, B, ldb, strideB, n, nchunks, items, alpha, alpha_inv);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Elementwise helpers on an m x n column-major block (batched):
// B := 0 (alpha == 0) and B := alpha * B (blocked path).

template <typename T>
__global__ void __launch_bounds__(256) scale_kernel(T *B, int64_t m, int64_t n, int64_t ldb,
                                                    int64_t strideB, T alpha, int set_zero)
{
    const int64_t col = blockIdx.y;
    T *Bc = B + (int64_t)blockIdx.z * strideB + col * ldb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m;
         i += (int64_t)gridDim.x * blockDim.x)
        Bc[i] = set_zero ? zero_of(T()) : mul(alpha, Bc[i]);
}

template <typename T>
hipError_t scale_matrix(T *B, int64_t m, int64_t n, int64_t ldb, int64_t strideB, int64_t batch,
                        T alpha, bool set_zero, hipStream_t s)
{
    const int64_t kMaxYZ = 65535;
    const unsigned gx = (unsigned)((m + 255) / 256 < 64 ? (m + 255) / 256 : 64);
    for (int64_t b0 = 0; b0 < batch; b0 += kMaxYZ)
        for (int64_t c0 = 0; c0 < n; c0 += kMaxYZ) {
            const int64_t nb = batch - b0 < kMaxYZ ? batch - b0 : kMaxYZ;
            const int64_t nc = n - c0 < kMaxYZ ? n - c0 : kMaxYZ;
            hipLaunchKernelGGL(scale_kernel<T>, dim3(gx, (unsigned)nc, (unsigned)nb), dim3(256), 0,
                               s, B + b0 * strideB + c0 * ldb, m, nc, ldb, strideB, alpha,
                               set_zero ? 1 : 0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

#define HSMA_INST(T)                                                                              \
    template hipError_t small_rowlane<T>(const T *, int64_t, int64_t, int64_t, int64_t, const T *, \
                                         int64_t, int64_t, int64_t, int64_t, T *, int64_t, int64_t, \
                                         int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, T,   \
                                         hipStream_t);                                             \
    template hipError_t small_colane<T>(int64_t, T, const T *, int64_t, int64_t, T *, int64_t,     \
                                        int64_t, int64_t, hipStream_t);                            \
    template hipError_t scale_matrix<T>(T *, int64_t, int64_t, int64_t, int64_t, int64_t, T, bool, \
                                        hipStream_t);
HSMA_INST(float)
HSMA_INST(double)
HSMA_INST(c32)
HSMA_INST(c64)
#undef HSMA_INST

}  // namespace hsma
