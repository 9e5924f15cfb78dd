// blocked.hip - the large regime: blocked TRSM on the matrix cores.
//
// HSMA-TRSM paper, blocked section: the diagonal blocks D_t (size N_B) of A
// are independent, so they are inverted in parallel first; then, block row
// by block row, X_t = D_t^{-1} B_t and the trailing rows are updated by a
// matrix multiply, B[below] -= A[below, t] X_t. Table 3 of the paper shows
// the multiply taking most of the time as m grows, so the multiply is the
// kernel that has to run near the matrix-core peak here.
//
// Kernels:
//  * diag_inv_kernel - one workgroup per (diagonal block t, identity tile of
//    G columns). It solves D_t Y = E by column-level forward substitution
//    (the paper's decoupled diagonal inversion: only the current column of
//    D_t is needed at each step, and the next columns are fetched while the
//    current one is used). Y stays in registers, one group of rows per
//    thread; the solved row is broadcast through a double-buffered LDS slot.
//  * gemm_kernel - C = beta*C + alpha*A*B with FP32 or FP64 MFMA, 128 x 128
//    output tile per 256-thread workgroup. Complex matrices run as real ones:
//    B and C are read as real matrices with twice the rows, and each complex
//    a of A is expanded on its way into LDS to the real 2 x 2 block
//    [[re, -im], [im, re]], so one complex multiply-add costs exactly the four
//    real ones the flop count assumes.
//  * copy_kernel - places the solved block row W into B.
#include "common.hpp"
#include "internal.hpp"

namespace hsma {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Diagonal-block inversion

template <typename T> struct dinv_cfg;  // columns per work unit G, prefetch chunk CK
template <> struct dinv_cfg<float> { static constexpr int G = 16, CK = 8; };
template <> struct dinv_cfg<double> { static constexpr int G = 8, CK = 8; };
template <> struct dinv_cfg<c32> { static constexpr int G = 8, CK = 8; };
template <> struct dinv_cfg<c64> { static constexpr int G = 4, CK = 4; };

template <typename T, int R, int G>
__global__ void __launch_bounds__(256) diag_inv_kernel(const T *__restrict__ A, int64_t lda,
                                                        int64_t m, int nb, T *__restrict__ invA)
{
    constexpr int CK = dinv_cfg<T>::CK;
    static_assert(CK % R == 0, "chunk must be a multiple of rows per thread");
    __shared__ T ybuf[2][G];

    const int t = blockIdx.y;             // diagonal block
    const int cstart = blockIdx.x * G;    // first identity column of this unit
    if (cstart >= nb) return;
    const int64_t r0 = (int64_t)t * nb;
    const int rb = (int)((m - r0) < nb ? (m - r0) : nb);  // rows of this block inside A
    const int tid = threadIdx.x;
    const T *D = A + r0 + r0 * lda;

    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;

    // Rows tid*R .. tid*R+R-1 of the unit's columns; start from the identity tile.
    T w[R][G];
    T inv[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int i = tid * R + q;
        inv[q] = (i < rb) ? recip(D[i + (int64_t)i * lda]) : one;
#pragma unroll
        for (int c = 0; c < G; ++c) w[q][c] = (i == cstart + c) ? one : zero_of(T());
    }

    // Column k of D_t below the diagonal, as this thread's rows see it;
    // everything else (diagonal, upper part, padding) reads as zero.
    auto dcol = [&](int k, int q) -> T {
        const int i = tid * R + q;
        if (k < rb && i > k && i < rb) return D[i + (int64_t)k * lda];
        return zero_of(T());
    };

    // Steps start at a multiple of R so that the owner of row k is always
    // register row k % R; steps before cstart only move zeros.
    const int kbeg = cstart - cstart % R;
    T dcur[R][CK], dnxt[R][CK];
#pragma unroll
    for (int kk = 0; kk < CK; ++kk)
#pragma unroll
        for (int q = 0; q < R; ++q) dcur[q][kk] = dcol(kbeg + kk, q);

    for (int k0 = kbeg; k0 < rb; k0 += CK) {
        // fetch the next chunk of columns while this one is used
#pragma unroll
        for (int kk = 0; kk < CK; ++kk)
#pragma unroll
            for (int q = 0; q < R; ++q) dnxt[q][kk] = dcol(k0 + CK + kk, q);
#pragma unroll
        for (int kk = 0; kk < CK; ++kk) {
            const int k = k0 + kk;
            if (k >= rb) break;
            const int qo = kk % R;  // row k is register row qo of thread k / R
            if (tid == k / R) {
#pragma unroll
                for (int c = 0; c < G; ++c) {
                    const T y = mul(w[qo][c], inv[qo]);
                    w[qo][c] = y;
                    ybuf[k & 1][c] = y;
                }
            }
            __syncthreads();
            T y[G];
#pragma unroll
            for (int c = 0; c < G; ++c) y[c] = ybuf[k & 1][c];
#pragma unroll
            for (int q = 0; q < R; ++q)
#pragma unroll
                for (int c = 0; c < G; ++c) w[q][c] = fms(w[q][c], dcur[q][kk], y[c]);
        }
#pragma unroll
        for (int kk = 0; kk < CK; ++kk)
#pragma unroll
            for (int q = 0; q < R; ++q) dcur[q][kk] = dnxt[q][kk];
    }

    T *out = invA + (int64_t)t * nb * nb;
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int i = tid * R + q;
            if (i < nb) out[i + (int64_t)(cstart + c) * nb] = w[q][c];
        }
}

template <typename T, int G>
static hipError_t diag_inv_launch(int64_t m, int nb, const T *A, int64_t lda, T *invA,
                                  hipStream_t s)
{
    const int64_t nt = (m + nb - 1) / nb;
    if (nt > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((nb + G - 1) / G), (unsigned)nt);
    if (nb <= 256)
        hipLaunchKernelGGL((diag_inv_kernel<T, 1, G>), grid, dim3(256), 0, s, A, lda, m, nb, invA);
    else if (nb <= 512)
        hipLaunchKernelGGL((diag_inv_kernel<T, 2, G>), grid, dim3(256), 0, s, A, lda, m, nb, invA);
    else if constexpr (dinv_cfg<T>::CK % 4 == 0)
        hipLaunchKernelGGL((diag_inv_kernel<T, 4, G>), grid, dim3(256), 0, s, A, lda, m, nb, invA);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename T>
hipError_t diag_invert(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA, hipStream_t s)
{
    // The identity tile of width ib is split into register-resident groups of
    // at most dinv_cfg<T>::G columns, each its own workgroup.
    constexpr int GM = dinv_cfg<T>::G;
    int g = 1;
    for (int cand = GM; cand >= 1; cand /= 2)
        if (ib % cand == 0 && nb % cand == 0) { g = cand; break; }
    switch (g) {
    case 16: if constexpr (GM >= 16) return diag_inv_launch<T, 16>(m, nb, A, lda, invA, s); break;
    case 8: if constexpr (GM >= 8) return diag_inv_launch<T, 8>(m, nb, A, lda, invA, s); break;
    case 4: return diag_inv_launch<T, 4>(m, nb, A, lda, invA, s);
    case 2: return diag_inv_launch<T, 2>(m, nb, A, lda, invA, s);
    default: return diag_inv_launch<T, 1>(m, nb, A, lda, invA, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Matrix-core GEMM

template <typename R> struct mfma_cfg;
// FP32: v_mfma_f32_32x32x2f32, a wave owns 64 x 64 outputs as 2 x 2 blocks.
template <> struct mfma_cfg<float> {
    static constexpr int BLK = 32, KSTEP = 2, NB = 2;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
};
// FP64: v_mfma_f64_16x16x4f64, a wave owns 64 x 64 outputs as 4 x 4 blocks.
template <> struct mfma_cfg<double> {
    static constexpr int BLK = 16, KSTEP = 4, NB = 4;
    using acc_t = f64x4;
    static constexpr int NACC = 4;
};

__device__ inline f32x16 mfma_op(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ inline f64x4 mfma_op(double a, double b, f64x4 c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

constexpr int kBM = 128, kBN = 128, kBK = 16;
constexpr int kPadA = 4;  // As[k][i] row padding (elements)
constexpr int kPadB = 1;  // Bs[j][k] row padding (elements)

// Real view of the product: Mr x N output from an Mr x Kr "A" and a Kr x N
// "B". For complex T, Mr = 2M, Kr = 2K, and B, C are the complex arrays read
// as real ones (leading dimension doubled); A is expanded on load.
template <typename T>
struct GemmArgs {
    using R = typename traits<T>::real;
    const T *A;
    int64_t lda;
    const R *B;
    int64_t ldb;  // real units
    R *C;
    int64_t ldc;  // real units
    int64_t Mr, N, Kr;
    R alpha, beta;
    int a_lower;
};

// The MFMA "row" operand runs over output columns j (from Bs) and the MFMA
// "column" operand over output rows i (from As). That makes consecutive lanes
// touch consecutive rows of the column-major C, so C reads and writes
// coalesce.
template <typename T>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs<T> p)
{
    using R = typename traits<T>::real;
    using cfg = mfma_cfg<R>;
    constexpr bool CPX = traits<T>::is_complex;
    constexpr int BLK = cfg::BLK, KS = cfg::KSTEP, NBK = cfg::NB;
    constexpr int LDA_S = kBM + kPadA, LDB_S = kBK + kPadB;
    __shared__ R As[kBK * LDA_S];
    __shared__ R Bs[kBN * LDB_S];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = (wave & 1) * 64;   // wave's row offset inside the tile (i)
    const int wj = (wave >> 1) * 64;  // wave's column offset (j)
    const int64_t i0 = (int64_t)blockIdx.x * kBM;
    const int64_t j0 = (int64_t)blockIdx.y * kBN;

    int64_t kend = p.Kr;
    if (p.a_lower && i0 + kBM < kend) kend = i0 + kBM;  // A is zero right of the diagonal

    // ---- global -> register staging of one K tile ----
    constexpr int A_PER = CPX ? (kBM / 2) * (kBK / 2) / 256 : kBM * kBK / 256;
    constexpr int B_PER = kBK * kBN / 256;
    T ra[A_PER];
    R rbv[B_PER];

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < A_PER; ++e) {
            const int idx = tid + 256 * e;
            if constexpr (CPX) {
                const int il = idx % (kBM / 2), kl = idx / (kBM / 2);
                const int64_t ic = i0 / 2 + il, kc = k0 / 2 + kl;
                const bool ok = ic < p.Mr / 2 && kc < p.Kr / 2 && (!p.a_lower || kc <= ic);
                ra[e] = ok ? p.A[ic + kc * p.lda] : zero_of(T());
            } else {
                const int il = idx % kBM, kl = idx / kBM;
                const int64_t i = i0 + il, k = k0 + kl;
                const bool ok = i < p.Mr && k < p.Kr && (!p.a_lower || k <= i);
                ra[e] = ok ? p.A[i + k * p.lda] : R(0);
            }
        }
#pragma unroll
        for (int e = 0; e < B_PER; ++e) {
            const int idx = tid + 256 * e;
            const int kl = idx % kBK, jl = idx / kBK;
            const int64_t k = k0 + kl, j = j0 + jl;
            rbv[e] = (k < p.Kr && j < p.N) ? p.B[k + j * p.ldb] : R(0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int e = 0; e < A_PER; ++e) {
            const int idx = tid + 256 * e;
            if constexpr (CPX) {
                const int il = idx % (kBM / 2), kl = idx / (kBM / 2);
                const T a = ra[e];
                // real 2 x 2 block of a complex entry: [[re, -im], [im, re]]
                As[(2 * kl) * LDA_S + 2 * il] = a.re;
                As[(2 * kl) * LDA_S + 2 * il + 1] = a.im;
                As[(2 * kl + 1) * LDA_S + 2 * il] = -a.im;
                As[(2 * kl + 1) * LDA_S + 2 * il + 1] = a.re;
            } else {
                const int il = idx % kBM, kl = idx / kBM;
                As[kl * LDA_S + il] = ra[e];
            }
        }
#pragma unroll
        for (int e = 0; e < B_PER; ++e) {
            const int idx = tid + 256 * e;
            const int kl = idx % kBK, jl = idx / kBK;
            Bs[jl * LDB_S + kl] = rbv[e];
        }
    };

    typename cfg::acc_t acc[NBK][NBK];
#pragma unroll
    for (int a = 0; a < NBK; ++a)
#pragma unroll
        for (int b = 0; b < NBK; ++b)
#pragma unroll
            for (int r = 0; r < cfg::NACC; ++r) acc[a][b][r] = 0;

    const int lrow = lane % BLK;   // MFMA operand row / output column inside a block
    const int lk = lane / BLK;     // MFMA k sub-index

    if (kend > 0) load_tile(0);
    for (int64_t k0 = 0; k0 < kend; k0 += kBK) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (k0 + kBK < kend) load_tile(k0 + kBK);
#pragma unroll
        for (int kk = 0; kk < kBK; kk += KS) {
            R bj[NBK], ai[NBK];
#pragma unroll
            for (int b = 0; b < NBK; ++b) bj[b] = Bs[(wj + b * BLK + lrow) * LDB_S + kk + lk];
#pragma unroll
            for (int a = 0; a < NBK; ++a) ai[a] = As[(kk + lk) * LDA_S + wi + a * BLK + lrow];
#pragma unroll
            for (int b = 0; b < NBK; ++b)
#pragma unroll
                for (int a = 0; a < NBK; ++a) acc[b][a] = mfma_op(bj[b], ai[a], acc[b][a]);
        }
    }

    // ---- epilogue: acc[b][a] holds D[j][i] for j in block b, i in block a ----
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
        for (int a = 0; a < NBK; ++a)
#pragma unroll
            for (int r = 0; r < cfg::NACC; ++r) {
                int jr;
                // output-row index of register r (lane layouts of the two MFMA forms)
                if constexpr (BLK == 32) jr = 8 * (r / 4) + 4 * lk + (r % 4);
                else jr = lk + 4 * r;
                const int64_t i = i0 + wi + a * BLK + lrow;
                const int64_t j = j0 + wj + b * BLK + jr;
                if (i < p.Mr && j < p.N) {
                    R v = p.alpha * acc[b][a][r];
                    R *cp = p.C + i + j * p.ldc;
                    if (p.beta != R(0)) v += *cp;
                    *cp = v;
                }
            }
}

template <typename T>
hipError_t gemm(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha, const T *A,
                int64_t lda, const T *B, int64_t ldb, typename traits<T>::real beta, T *C,
                int64_t ldc, bool a_lower, hipStream_t s)
{
    using R = typename traits<T>::real;
    constexpr int f = traits<T>::is_complex ? 2 : 1;
    GemmArgs<T> p;
    p.A = A;
    p.lda = lda;
    p.B = (const R *)B;
    p.ldb = ldb * f;
    p.C = (R *)C;
    p.ldc = ldc * f;
    p.Mr = M * f;
    p.N = N;
    p.Kr = K * f;
    p.alpha = alpha;
    p.beta = beta;
    p.a_lower = a_lower ? 1 : 0;
    const int64_t gx = (p.Mr + kBM - 1) / kBM, gy = (N + kBN - 1) / kBN;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemm_kernel<T>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Blocked driver

template <typename T>
__global__ void __launch_bounds__(256) copy_kernel(const T *__restrict__ W, int64_t ldw, int64_t rows,
                                                   T *__restrict__ B, int64_t ldb)
{
    const int64_t col = blockIdx.y;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows;
         i += (int64_t)gridDim.x * blockDim.x)
        B[i + col * ldb] = W[i + col * ldw];
}

int64_t blocked_workspace_elems(int64_t m, int64_t n, int nb)
{
    const int64_t nt = (m + nb - 1) / nb;
    return nt * nb * nb + (int64_t)nb * n;
}

template <typename T>
hipError_t blocked_solve(int64_t m, int64_t n, int nb, int ib, const T *A, int64_t lda, T *B,
                         int64_t ldb, T *work, hipStream_t s)
{
    using R = typename traits<T>::real;
    const int64_t nt = (m + nb - 1) / nb;
    T *invA = work;
    T *W = work + nt * nb * nb;
    hipError_t e = diag_invert<T>(m, nb, ib, A, lda, invA, s);
    for (int64_t t = 0; t < nt && e == hipSuccess; ++t) {
        const int64_t r0 = t * nb;
        const int64_t rb = m - r0 < nb ? m - r0 : nb;
        // X_t = D_t^{-1} B_t (D_t^{-1} is lower triangular: upper tiles skipped)
        e = gemm<T>(rb, n, rb, R(1), invA + t * nb * nb, nb, B + r0, ldb, R(0), W, nb, true, s);
        if (e != hipSuccess) break;
        for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += 65535) {
            const int64_t nc = n - c0 < 65535 ? n - c0 : 65535;
            hipLaunchKernelGGL(copy_kernel<T>, dim3((unsigned)((rb + 255) / 256), (unsigned)nc),
                               dim3(256), 0, s, W + c0 * nb, (int64_t)nb, rb, B + r0 + c0 * ldb, ldb);
            e = hipGetLastError();
        }
        if (e != hipSuccess) break;
        // B[below] -= A[below, t] X_t
        if (r0 + rb < m)
            e = gemm<T>(m - r0 - rb, n, rb, R(-1), A + (r0 + rb) + r0 * lda, lda, W, nb, R(1),
                        B + r0 + rb, ldb, false, s);
    }
    return e;
}

#define HSMA_INST(T)                                                                              \
    template hipError_t diag_invert<T>(int64_t, int, int, const T *, int64_t, T *, hipStream_t);  \
    template hipError_t gemm<T>(int64_t, int64_t, int64_t, typename traits<T>::real, const T *,    \
                                int64_t, const T *, int64_t, typename traits<T>::real, T *,       \
                                int64_t, bool, hipStream_t);                                      \
    template hipError_t blocked_solve<T>(int64_t, int64_t, int, int, const T *, int64_t, T *,     \
                                         int64_t, T *, hipStream_t);
HSMA_INST(float)
HSMA_INST(double)
HSMA_INST(c32)
HSMA_INST(c64)
#undef HSMA_INST

}  // namespace hsma
