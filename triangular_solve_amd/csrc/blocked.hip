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
#include <type_traits>

#include "hsma_trsm.h"
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
        T d = one;
        if (i < rb) d = D[i + (int64_t)i * lda];
        inv[q] = recip(d);
#pragma unroll
        for (int c = 0; c < G; ++c) w[q][c] = pick(i == cstart + c, one, zero_of(T()));
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
            // only the rows below k change: row k and the rows above keep
            // their values also when y is inf or NaN (a zero pivot)
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const bool below = tid * R + q > k;
#pragma unroll
                for (int c = 0; c < G; ++c) {
                    const T u = fms(w[q][c], dcur[q][kk], y[c]);
                    w[q][c] = pick(below, u, w[q][c]);
                }
            }
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
    if (nb > 1024) return hipErrorInvalidValue;  // 256 threads x at most 4 rows
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
static hipError_t blocked_inverse(int64_t m, int nb, const T *A, int64_t lda, T *invA, T *temp,
                                  hipStream_t s);
template <typename T>
static bool blocked_inverse_applies(int64_t m, int nb);
template <typename T>
static bool auto_merges(int64_t m, int nb);
template <typename T>
bool invert_route_applies(int64_t m, int nb, int ib, int route);
// Inversion of all diagonal blocks by route: with merge products
// (temporaries allocated stream-ordered) or by diag_inv_kernel alone.
template <typename T>
hipError_t diag_invert_any(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA,
                           hipStream_t s, int route)
{
    if (!invert_route_applies<T>(m, nb, ib, route)) return hipErrorInvalidValue;
    const bool merges = route == HSMA_INV_FUSED || route == HSMA_INV_BLOCKED ||
                        (route == HSMA_INV_AUTO && auto_merges<T>(m, nb));
    if (!merges) return diag_invert<T>(m, nb, ib, A, lda, invA, s);
    void *tmp = nullptr;
    hipError_t e = workspace_alloc(&tmp, (size_t)blocked_inverse_temp_elems(m, nb) * sizeof(T), s);
    if (e != hipSuccess) return e;
    e = blocked_invert<T>(m, nb, ib, A, lda, invA, (T *)tmp, s, route);
    const hipError_t ef = workspace_free(tmp, s);
    return e != hipSuccess ? e : ef;
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
//
// C = beta*C + alpha*A*B. A 256-thread workgroup owns a 128 x 128 tile of C
// (four waves, 64 x 64 each). K advances in steps of BK through two LDS
// buffers: the next step's tiles are fetched from HBM into registers while
// the matrix cores work on the current one, then written to the other
// buffer; one barrier per step. Global loads are 16 bytes wide along the
// contiguous dimension of each column-major operand.
//
// Operand roles: the MFMA "row" operand runs over output columns j (from the
// B tile) and the MFMA "column" operand over output rows i (from the A tile),
// so consecutive lanes own consecutive rows of the column-major C and C
// traffic coalesces. Inside a step the k index is permuted: lane group h
// handles k = KS*h + s at MFMA sub-step s, so each lane's B fragment for KS
// sub-steps is one contiguous 16-byte LDS read (the same permutation is used
// for A, so every k is still summed exactly once).

// NI x NJ blocks of BLK x BLK outputs per wave (NI along the rows i of C, NJ
// along its columns j), WI x WJ waves, so a workgroup tile is BM = WI*NI*BLK
// rows by BN = WJ*NJ*BLK columns; K steps of BK. TILE selects the standard
// tile, the large f32 tiles for large products or the 64 x 64 tile for
// products with few standard tiles.
constexpr int kTileStd = 0, kTileWide = 1, kTileSmall = 2, kTileBig = 3, kTileStd8 = 4;
template <typename R, int TILE = kTileStd> struct mfma_cfg;
// FP32: v_mfma_f32_32x32x2f32, a wave owns 64 x 64 outputs as 2 x 2 blocks.
template <> struct mfma_cfg<float, kTileStd> {
    static constexpr int WI = 2, WJ = 2;
    static constexpr int BLK = 32, LG = 2, NI = 2, NJ = 2, BK = 32;  // LG: lane groups along k
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP32, wide: a wave owns 128 x 64 outputs as 4 x 2 blocks, a 256 x 128
// workgroup tile with K steps of 16: a third fewer LDS bytes per MFMA and
// more flops per byte of L2 traffic. It wins on large products (the trailing
// updates, K >= 2048) and loses where its coarser tiles leave CUs idle.
template <> struct mfma_cfg<float, kTileWide> {
    static constexpr int WI = 2, WJ = 2;
    static constexpr int BLK = 32, LG = 2, NI = 4, NJ = 2, BK = 16;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP32, big: the wide tile's waves, eight of them, as a 256 x 256 workgroup
// tile (232 VGPRs: one workgroup per CU): half the A and B bytes fetched per
// output. For real f32 products it replaces the wide tile (MI355X:
// 6144 x 8192 x 2048 1.93 -> 1.88 ms, 4096 x 8192 x 2048 1.16 -> 1.12 ms,
// 2048 x 8192 x 2048 0.575 -> 0.56 ms); complex products, whose A is expanded
// on its way into LDS, lose with it (c64 6144 x 8192 x 2048 6.94 -> 7.14 ms)
// and keep the wide tile.
template <> struct mfma_cfg<float, kTileBig> {
    static constexpr int WI = 2, WJ = 4;
    static constexpr int BLK = 32, LG = 2, NI = 4, NJ = 2, BK = 16;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP32, standard tile of eight waves: 128 x 256, each wave 64 x 64 (196
// VGPRs, one workgroup per CU); for real f32 products between the small and
// the big tile, the triangular inverse multiplies among them.
template <> struct mfma_cfg<float, kTileStd8> {
    static constexpr int WI = 2, WJ = 4;
    static constexpr int BLK = 32, LG = 2, NI = 2, NJ = 2, BK = 32;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP32, small: a wave owns one 32 x 32 block, a 64 x 64 workgroup tile: four
// times the workgroups of the standard tile for products that would leave
// CUs idle (the block-inverse merges, single problems in block rows, the
// products of mid-size solves).
template <> struct mfma_cfg<float, kTileSmall> {
    static constexpr int WI = 2, WJ = 2;
    static constexpr int BLK = 32, LG = 2, NI = 1, NJ = 1, BK = 32;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP64: v_mfma_f64_16x16x4f64, a wave owns 64 x 64 outputs as 4 x 4 blocks
// (a larger tile would double the 128-register accumulator).
template <> struct mfma_cfg<double, kTileStd> {
    static constexpr int WI = 2, WJ = 2;
    static constexpr int BLK = 16, LG = 4, NI = 4, NJ = 4, BK = 8;
    using acc_t = f64x4;
    static constexpr int NACC = 4;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP64, standard tile of eight waves: 128 x 256, each wave 64 x 64, for
// the triangular products of real f64 (the inverse multiplies of f64 and,
// in real form, of c128).
template <> struct mfma_cfg<double, kTileStd8> {
    static constexpr int WI = 2, WJ = 4;
    static constexpr int BLK = 16, LG = 4, NI = 4, NJ = 4, BK = 8;
    using acc_t = f64x4;
    static constexpr int NACC = 4;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};
// FP64, small: a wave owns 32 x 32 outputs as 2 x 2 blocks, a 64 x 64 tile.
template <> struct mfma_cfg<double, kTileSmall> {
    static constexpr int WI = 2, WJ = 2;
    static constexpr int BLK = 16, LG = 4, NI = 2, NJ = 2, BK = 8;
    using acc_t = f64x4;
    static constexpr int NACC = 4;
    static constexpr int BM = WI * NI * BLK, BN = WJ * NJ * BLK, NT = 64 * WI * WJ;
};

__device__ inline f32x16 mfma_op(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ inline f64x4 mfma_op(double a, double b, f64x4 c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
template <typename R> struct vec16;
template <> struct vec16<float> { using type = f32x4; static constexpr int N = 4; };
template <> struct vec16<double> { using type = f64x2; static constexpr int N = 2; };

constexpr int kMaxBM = 256;    // largest workgroup tile height over the element types
constexpr int64_t kSmallTileBelow = 512;  // standard-tile count under which the 64 x 64 tile runs
constexpr int kXcds = 8;        // XCDs of the GPU (round-robin workgroup placement)
constexpr int64_t kGroupRows = 8;  // row tiles per group in the XCD-local tile order

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
    R alpha, cscale;  // C = alpha * (cscale * C + A*B); cscale = beta / alpha, alpha != 0
    int a_lower;
    // Batch (grid z): product z = g * bin + k uses A + g*sAo + k*sAi (elements
    // of T) and B, C shifted likewise (real units).
    int64_t bin;
    int64_t sAi, sAo, sBi, sBo, sCi, sCo;
};

template <typename T, bool VEC, int TILE>
__global__ void __launch_bounds__((mfma_cfg<typename traits<T>::real, TILE>::NT), 2) gemm_kernel(GemmArgs<T> p)
{
    using R = typename traits<T>::real;
    using cfg = mfma_cfg<R, TILE>;
    using V16 = typename vec16<R>::type;
    constexpr int VN = vec16<R>::N;           // reals per 16 bytes
    constexpr bool CPX = traits<T>::is_complex;
    constexpr int BLK = cfg::BLK, LG = cfg::LG, NI = cfg::NI, NJ = cfg::NJ, BK = cfg::BK;
    constexpr int kBM = cfg::BM, kBN = cfg::BN;
    constexpr int KS = BK / LG / (BK / (LG * VN)) ;  // k per lane group per 16-byte read = VN
    static_assert(KS == VN, "one 16-byte B read per lane group");
    constexpr int LDA_S = kBM + 4 / (int)(sizeof(R) / 4);   // As[k][i] row stride (+16 bytes)
    constexpr int LDB_S = BK + VN;                           // Bs[j][k] row stride (+16 bytes)
    __shared__ __attribute__((aligned(16))) R As[2][BK * LDA_S];
    __shared__ __attribute__((aligned(16))) R Bs[2][kBN * LDB_S];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = (wave % cfg::WI) * (NI * BLK);  // wave's row offset inside the tile (i)
    const int wj = (wave / cfg::WI) * (NJ * BLK);  // wave's column offset (j)
    // Tile of this workgroup. Workgroups are dealt to the 8 XCDs round-robin
    // by linear id, and each XCD has its own L2; for a single product the
    // ids are renumbered so that every XCD gets a contiguous range, walked in
    // groups of kGroupRows row tiles, so the workgroups resident on one XCD
    // share a few A row panels and B column panels.
    int64_t bx = blockIdx.x, by = blockIdx.y;
    {
        const int64_t gx = gridDim.x, gy = gridDim.y, total = gx * gy;
        if (p.a_lower) {
            // Triangular A: row tile x carries x + 1 K blocks. The heaviest
            // row tiles are dispatched first (consecutive ids, dealt to the
            // XCDs in turn, take the column tiles of one row tile), so the
            // light ones fill in at the end.
            const int64_t id = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gx;
            bx = gx - 1 - id / gy;
            by = id % gy;
        } else if (gridDim.z == 1 && total % kXcds == 0) {
            const int64_t id = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gx;
            const int64_t t = (id % kXcds) * (total / kXcds) + id / kXcds;
            const int64_t first = t / (kGroupRows * gy) * kGroupRows;
            const int64_t gs = gx - first < kGroupRows ? gx - first : kGroupRows;
            const int64_t r = t % (kGroupRows * gy);
            bx = first + r % gs;
            by = r / gs;
        }
    }
    const int64_t i0 = bx * kBM;
    const int64_t j0 = by * kBN;
    {
        const int64_t z = blockIdx.z, g = z / p.bin, k = z % p.bin;
        p.A += g * p.sAo + k * p.sAi;
        p.B += g * p.sBo + k * p.sBi;
        p.C += g * p.sCo + k * p.sCi;
    }

    // ---- staging of one K step: A as 16-byte chunks along i, B along k ----
    // A tile: BK x kBM reals = (kBM/VN) chunks per k row; chunks per thread:
    constexpr int NT = cfg::NT;
    constexpr int A_CH = BK * kBM / VN / NT;
    constexpr int B_CH = BK * kBN / VN / NT;
    static_assert(A_CH * NT * VN == BK * kBM && B_CH * NT * VN == BK * kBN,
                  "the threads' 16-byte chunks cover a K step's tiles exactly");
    // PF K steps of staging registers: step s+PF is fetched while step s is
    // multiplied (with PF = 2, s+1 already sits in the other LDS buffer).
    // Measured on MI355X, PF = 2 gained nothing over PF = 1, which needs
    // fewer registers.
    constexpr int PF = 1;
    V16 ra[PF][A_CH], rb[PF][B_CH];

    // Interior tiles and steps (the common case) take branch-free 16-byte
    // loads; the bounds and triangle checks only run at the edges.
    int64_t kend = p.Kr;
    if (p.a_lower && i0 + kBM < kend) kend = i0 + kBM;  // A is zero right of the diagonal (block)
    const bool tile_interior = VEC && i0 + kBM <= p.Mr && j0 + kBN <= p.N;
    auto load_step = [&](int64_t k0, int slot) {
        // a_lower 2 (the real form of a complex lower triangle): entry (i, k)
        // is used when k <= i | 1, so a step is whole when it ends at i0 + 1
        const int blk2 = p.a_lower == 2;
        const bool fast = tile_interior && k0 + BK <= p.Kr && (!p.a_lower || k0 + BK <= i0 + 1 + blk2);
        {
            if (fast) {
#pragma unroll
                for (int e = 0; e < A_CH; ++e) {
                    const int idx = tid + NT * e;
                    const int ic = idx % (kBM / VN), kl = idx / (kBM / VN);
                    if constexpr (CPX) {
                        // 16 bytes = VN/2 complex entries of complex column (k0+kl)/2;
                        // real row 2kc holds (re, im), row 2kc+1 holds (-im, re)
                        const int64_t kc = (k0 + kl) >> 1;
                        const V16 raw = *(const V16 *)(p.A + (i0 / 2 + (int64_t)ic * (VN / 2)) + kc * p.lda);
                        V16 v = raw;
                        if (kl & 1) {
#pragma unroll
                            for (int t = 0; t < VN; t += 2) { v[t] = -raw[t + 1]; v[t + 1] = raw[t]; }
                        }
                        ra[slot][e] = v;
                    } else {
                        ra[slot][e] = *(const V16 *)(p.A + i0 + (int64_t)ic * VN + (k0 + kl) * p.lda);
                    }
                }
#pragma unroll
                for (int e = 0; e < B_CH; ++e) {
                    const int idx = tid + NT * e;
                    const int kc = idx % (BK / VN), jl = idx / (BK / VN);
                    rb[slot][e] = *(const V16 *)(p.B + k0 + kc * VN + (j0 + jl) * p.ldb);
                }
                return;
            }
        }
#pragma unroll
        for (int e = 0; e < A_CH; ++e) {
            const int idx = tid + NT * e;
            const int ic = idx % (kBM / VN), kl = idx / (kBM / VN);  // chunk column, k row
            const int64_t k = k0 + kl;
            V16 v;
            if constexpr (CPX) {
                // VN reals of one real row = VN/2 complex entries of A's complex row ...
                // real row index r = 2*ic_c + p  -> complex rows i0/2 + ic*VN/2 ...
                // Load the complex entries (kc = k/2 column, rows ic*VN/2 .. +VN/2); the
                // expansion to [[re, -im], [im, re]] happens when writing LDS.
                const int64_t kc = k >> 1;
                const int64_t ib = i0 / 2 + (int64_t)ic * (VN / 2);
                R tmp[VN];
#pragma unroll
                for (int t = 0; t < VN / 2; ++t) {
                    const int64_t irow = ib + t;
                    const bool ok = irow < p.Mr / 2 && kc < p.Kr / 2 && (!p.a_lower || kc <= irow);
                    T a = ok ? p.A[irow + kc * p.lda] : zero_of(T());
                    // row 2kc (k even): (re, im); row 2kc+1 (k odd): (-im, re)
                    if ((k & 1) == 0) { tmp[2 * t] = a.re; tmp[2 * t + 1] = a.im; }
                    else { tmp[2 * t] = -a.im; tmp[2 * t + 1] = a.re; }
                }
#pragma unroll
                for (int t = 0; t < VN; ++t) v[t] = tmp[t];
            } else {
                const int64_t ib = i0 + (int64_t)ic * VN;
                const bool full = VEC && ib + VN <= p.Mr && k < p.Kr && (!p.a_lower || k <= ib + blk2);
                if (full) {
                    v = *(const V16 *)(p.A + ib + k * p.lda);
                } else {
#pragma unroll
                    for (int t = 0; t < VN; ++t) {
                        const int64_t i = ib + t;
                        const bool ok = i < p.Mr && k < p.Kr && (!p.a_lower || k <= (i | blk2));
                        v[t] = ok ? p.A[i + k * p.lda] : R(0);
                    }
                }
            }
            ra[slot][e] = v;
        }
#pragma unroll
        for (int e = 0; e < B_CH; ++e) {
            const int idx = tid + NT * e;
            const int kc = idx % (BK / VN), jl = idx / (BK / VN);
            const int64_t kb = k0 + kc * VN, j = j0 + jl;
            V16 v;
            if (VEC && kb + VN <= p.Kr && j < p.N) {
                v = *(const V16 *)(p.B + kb + j * p.ldb);
            } else {
#pragma unroll
                for (int t = 0; t < VN; ++t) v[t] = (kb + t < p.Kr && j < p.N) ? p.B[kb + t + j * p.ldb] : R(0);
            }
            rb[slot][e] = v;
        }
    };
    auto store_step = [&](int buf, int slot) {
#pragma unroll
        for (int e = 0; e < A_CH; ++e) {
            const int idx = tid + NT * e;
            const int ic = idx % (kBM / VN), kl = idx / (kBM / VN);
            *(V16 *)&As[buf][kl * LDA_S + ic * VN] = ra[slot][e];
        }
#pragma unroll
        for (int e = 0; e < B_CH; ++e) {
            const int idx = tid + NT * e;
            const int kc = idx % (BK / VN), jl = idx / (BK / VN);
            *(V16 *)&Bs[buf][jl * LDB_S + kc * VN] = rb[slot][e];
        }
    };

    const int lrow = lane % BLK;  // MFMA operand row / output column inside a block
    const int lg = lane / BLK;    // lane group along k

    // Output-row index of accumulator register r (lane layouts of the two MFMA forms).
    auto jrow = [&](int r) -> int {
        if constexpr (BLK == 32) return 8 * (r / 4) + 4 * lg + (r % 4);
        else return lg + 4 * r;
    };

    typename cfg::acc_t acc[NJ][NI];
#pragma unroll
    for (int b = 0; b < NJ; ++b)
#pragma unroll
        for (int a = 0; a < NI; ++a)
#pragma unroll
            for (int r = 0; r < cfg::NACC; ++r) acc[b][a][r] = 0;

    const int nsteps = (int)((kend + BK - 1) / BK);
    if (nsteps > 0) {
        load_step(0, 0);
        if (PF == 2 && nsteps > 1) load_step(BK, PF - 1);
        store_step(0, 0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        // PF = 2: slot (st+1)&1 holds step st+1 and slot st&1 is free for st+2
        if (st + PF < nsteps) load_step((int64_t)(st + PF) * BK, PF == 2 ? (st & 1) : 0);
        const R *as = As[buf];
        const R *bs = Bs[buf];
        // BK = NQ groups of LG*VN k values. All fragments of the step are read
        // from LDS first; a scheduling barrier keeps the compiler from sinking
        // each read to just before its MFMAs (which exposes LDS latency with a
        // full wait per MFMA group). LDS returns in order, so the MFMAs start
        // as soon as their own fragments have arrived.
        constexpr int NQ = BK / (LG * VN);
        V16 bv[NQ][NJ];
        R av[NQ][VN][NI];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int kq = q * LG * VN + lg * VN;  // this lane group's first k in the group
#pragma unroll
            for (int b = 0; b < NJ; ++b)
                bv[q][b] = *(const V16 *)&bs[(wj + b * BLK + lrow) * LDB_S + kq];
#pragma unroll
            for (int s = 0; s < VN; ++s)
#pragma unroll
                for (int a = 0; a < NI; ++a) av[q][s][a] = as[(kq + s) * LDA_S + wi + a * BLK + lrow];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int s = 0; s < VN; ++s)
#pragma unroll
                for (int b = 0; b < NJ; ++b)
#pragma unroll
                    for (int a = 0; a < NI; ++a)
                        acc[b][a] = mfma_op(bv[q][b][s], av[q][s][a], acc[b][a]);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < nsteps) store_step(buf ^ 1, PF == 2 ? ((st + 1) & 1) : 0);
        __syncthreads();
    }

    // ---- epilogue: acc[b][a] holds D[j][i] for j in block b, i in block a ----
#pragma unroll
    for (int b = 0; b < NJ; ++b)
#pragma unroll
        for (int a = 0; a < NI; ++a)
#pragma unroll
            for (int r = 0; r < cfg::NACC; ++r) {
                const int64_t i = i0 + wi + a * BLK + lrow;
                const int64_t j = j0 + wj + b * BLK + jrow(r);
                if (i < p.Mr && j < p.N) {
                    R *cp = p.C + i + j * p.ldc;
                    R v = acc[b][a][r];
                    if (p.cscale != R(0)) v += p.cscale * *cp;
                    *cp = p.alpha * v;
                }
            }
}

// Batched product: batch = nout * bin products; product z = g*bin + k uses
// A + g*sAo + k*sAi, B + g*sBo + k*sBi, C + g*sCo + k*sCi (strides in elements).
template <typename T>
static hipError_t gemm_batched(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha,
                               const T *A, int64_t lda, int64_t sAi, int64_t sAo, const T *B,
                               int64_t ldb, int64_t sBi, int64_t sBo, typename traits<T>::real beta,
                               T *C, int64_t ldc, int64_t sCi, int64_t sCo, int64_t bin,
                               int64_t batch, int a_lower, hipStream_t s)
{
    using R = typename traits<T>::real;
    constexpr int f = traits<T>::is_complex ? 2 : 1;
    if (M == 0 || N == 0 || batch == 0) return hipSuccess;
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
    p.a_lower = a_lower;
    p.bin = bin > 0 ? bin : 1;
    p.sAi = sAi; p.sAo = sAo;
    p.sBi = sBi * f; p.sBo = sBo * f;
    p.sCi = sCi * f; p.sCo = sCo * f;
    if (alpha == R(0)) {
        // C = beta * C with beta in {0, 1}: nothing to multiply
        if (beta != R(0)) return hipSuccess;
        p.alpha = R(1);
        p.cscale = R(0);
        p.Kr = 0;
    } else {
        p.alpha = alpha;
        p.cscale = beta / alpha;
    }
    // the large f32 tiles for large full products: K of 2048 or more and at
    // least one big tile per CU for real f32 (a 256 x 256 tile, eight waves),
    // two wide tiles per CU for c64 (256 x 128, four waves); a triangular
    // product keeps the finer tiles, which balance its uneven rows better
    constexpr bool kBigF = std::is_same<T, float>::value;
    using CW = mfma_cfg<R, std::is_same<R, float>::value ? (kBigF ? kTileBig : kTileWide) : kTileStd>;
    using CS = mfma_cfg<R, kTileStd>;
    using CM = mfma_cfg<R, kTileSmall>;
    const bool wide = std::is_same<R, float>::value && !a_lower && p.Kr >= 2048 &&
                      ((p.Mr + CW::BM - 1) / CW::BM) * ((N + CW::BN - 1) / CW::BN) * batch >= (kBigF ? 256 : 512);
    // the 64 x 64 tile: for fewer than two standard tiles per CU (four times
    // the workgroups of the same product; measured on MI355X against a limit
    // of one per CU, 1.0-1.27x faster solves, and mixed, 0.96-1.16x, at
    // four), and for products whose rows or columns fit one small tile (a
    // standard tile would be at least half padding)
    const bool small = !wide && (((p.Mr + CS::BM - 1) / CS::BM) * ((N + CS::BN - 1) / CS::BN) * batch <
                                     kSmallTileBelow ||
                                 p.Mr <= CM::BM || N <= CM::BN);
    const int64_t kBM = wide ? CW::BM : small ? CM::BM : CS::BM;
    const int64_t kBN = wide ? CW::BN : small ? CM::BN : CS::BN;
    const int64_t gx = (p.Mr + kBM - 1) / kBM;
    const int64_t gy = (N + kBN - 1) / kBN;
    if (gx > 0x7fffffff || gy > 65535 || batch > 65535) return hipErrorInvalidConfiguration;
    // 16-byte loads need 16-byte aligned columns of A and B (every batch member).
    const int64_t sz = (int64_t)sizeof(T);
    const bool vec = (uintptr_t)A % 16 == 0 && (uintptr_t)B % 16 == 0 && (lda * sz) % 16 == 0 &&
                     (ldb * sz) % 16 == 0 && (sAi * sz) % 16 == 0 && (sAo * sz) % 16 == 0 &&
                     (sBi * sz) % 16 == 0 && (sBo * sz) % 16 == 0;
    const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)batch);
    if constexpr (std::is_same<R, float>::value) {
        if (wide) {
            constexpr int TW = kBigF ? kTileBig : kTileWide;
            if (vec) hipLaunchKernelGGL((gemm_kernel<T, true, TW>), grid, dim3(CW::NT), 0, s, p);
            else hipLaunchKernelGGL((gemm_kernel<T, false, TW>), grid, dim3(CW::NT), 0, s, p);
            return hipGetLastError();
        }
    }
    if (small) {
        if (vec) hipLaunchKernelGGL((gemm_kernel<T, true, kTileSmall>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<T, false, kTileSmall>), grid, dim3(256), 0, s, p);
        return hipGetLastError();
    }
    // real f32 products, and triangular real f64 ones, with at least one
    // 128 x 256 tile per CU take the eight-wave standard tile (MI355X: f32
    // m = n = 8192 solve 5.75 -> 5.50 ms, 4096 x 4096 x 1024 0.374 -> 0.357
    // ms, from 512 tiles up only 5.58 ms; f64 m = n = 8192 10.22 -> 10.08 ms,
    // c128 37.97 -> 37.62 ms; full f64 products lose with it); the per-wave
    // order of the products is that of the four-wave tile
    if constexpr (std::is_same<T, float>::value || std::is_same<T, double>::value) {
        using C8 = mfma_cfg<R, kTileStd8>;
        const int64_t gx8 = (p.Mr + C8::BM - 1) / C8::BM, gy8 = (N + C8::BN - 1) / C8::BN;
        if ((std::is_same<T, float>::value || a_lower) && gx8 * gy8 * batch >= 256 && gy8 <= 65535) {
            const dim3 grid8((unsigned)gx8, (unsigned)gy8, (unsigned)batch);
            if (vec) hipLaunchKernelGGL((gemm_kernel<T, true, kTileStd8>), grid8, dim3(C8::NT), 0, s, p);
            else hipLaunchKernelGGL((gemm_kernel<T, false, kTileStd8>), grid8, dim3(C8::NT), 0, s, p);
            return hipGetLastError();
        }
    }
    if (vec) hipLaunchKernelGGL((gemm_kernel<T, true, kTileStd>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_kernel<T, false, kTileStd>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t gemm_strided(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha,
                        const T *A, int64_t lda, int64_t strideA, const T *B, int64_t ldb,
                        int64_t strideB, typename traits<T>::real beta, T *C, int64_t ldc,
                        int64_t strideC, int64_t batch, hipStream_t s)
{
    const int64_t kMaxZ = 65535;  // grid z
    for (int64_t b0 = 0; b0 < batch; b0 += kMaxZ) {
        const int64_t nb = batch - b0 < kMaxZ ? batch - b0 : kMaxZ;
        hipError_t e = gemm_batched<T>(M, N, K, alpha, A + b0 * strideA, lda, strideA, 0,
                                       B + b0 * strideB, ldb, strideB, 0, beta, C + b0 * strideC,
                                       ldc, strideC, 0, nb, nb, false, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t gemm(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha, const T *A,
                int64_t lda, const T *B, int64_t ldb, typename traits<T>::real beta, T *C,
                int64_t ldc, int a_lower, hipStream_t s)
{
    return gemm_batched<T>(M, N, K, alpha, A, lda, 0, 0, B, ldb, 0, 0, beta, C, ldc, 0, 0, 1, 1,
                           a_lower, s);
}

// ---------------------------------------------------------------------------
// Split-K for products with few output tiles: with N <= 128 (few
// right-hand sides) a product has one column of 128 x 128 tiles, so a
// trailing update of M rows runs on M/128 workgroups for 256 CUs; the
// products of a solve with m <= 4096 have few tiles at any n (m = n = 1024
// with N_B = 256: 16 tiles). The K range is cut into S equal chunks of at
// least 64; a batched product writes the S partial products
// P_s = A[:, K_s] B[K_s, :] to workspace, and reduce_kernel forms
// C = beta C + alpha (P_0 + ... + P_{S-1}), summing in a fixed order so the
// result is the same on every run. Measured on MI355X against chunks of at
// least 256 and no split above n = 256: 1.2-2.8x for m <= 4096 in all four
// types, unchanged where every product already has 256 tiles or more.

template <typename R>
__global__ void __launch_bounds__(256) reduce_kernel(const R *__restrict__ P, int64_t rows,
                                                     int64_t cols, int64_t S, R alpha, R beta,
                                                     R *__restrict__ C, int64_t ldc)
{
    const int64_t total = rows * cols;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        R acc = P[e];
        for (int64_t k = 1; k < S; ++k) acc += P[k * total + e];
        const int64_t i = e % rows, j = e / rows;
        R *c = C + i + j * ldc;
        *c = beta == R(0) ? alpha * acc : beta * *c + alpha * acc;
    }
}

constexpr int kSplitTarget = 512;   // workgroups a split product aims for (2 per CU)
constexpr int kSplitMinChunk = 64;  // smallest K chunk
constexpr int64_t kSplitMaxPart = int64_t(8) << 20;  // partial-product elements above n = 256

// Chunks for an M x N x K product (elements of T), 1 = no split.
template <typename T>
int64_t splitk_chunks(int64_t M, int64_t N, int64_t K, int64_t part_elems)
{
    const int64_t f = traits<T>::is_complex ? 2 : 1;
    constexpr int64_t kBM = mfma_cfg<typename traits<T>::real>::BM;
    constexpr int64_t kBN = mfma_cfg<typename traits<T>::real>::BN;
    const int64_t tiles = ((M * f + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    if (tiles >= 256 || K < 2 * kSplitMinChunk || M * N <= 0) return 1;
    int64_t S = (kSplitTarget + tiles - 1) / tiles;
    if (S > K / kSplitMinChunk) S = K / kSplitMinChunk;
    if (S > part_elems / (M * N)) S = part_elems / (M * N);
    while (S > 1 && K % S != 0) --S;
    return S < 1 ? 1 : S;
}

int64_t splitk_part_elems(int64_t m, int64_t n)
{
    // partials of at most kSplitTarget tiles' worth of rows (plus one tile
    // of rounding) for n <= 256; above that, at most 16 partials of the
    // whole block row, capped at kSplitMaxPart elements (splitk_chunks
    // lowers S to what fits)
    if (n <= 256) {
        const int64_t rows = (int64_t)kSplitTarget * kMaxBM + 16 * (int64_t)kMaxBM;
        return (rows < 16 * m ? rows : 16 * m) * n;
    }
    const int64_t full = 16 * m * n;
    return full < kSplitMaxPart ? full : kSplitMaxPart;
}

template <typename T>
hipError_t gemm_splitk(int64_t M, int64_t N, int64_t K, typename traits<T>::real alpha, const T *A,
                       int64_t lda, const T *B, int64_t ldb, typename traits<T>::real beta, T *C,
                       int64_t ldc, bool a_lower, T *part, int64_t part_elems, hipStream_t s)
{
    using R = typename traits<T>::real;
    const int64_t S = part ? splitk_chunks<T>(M, N, K, part_elems) : 1;
    if (S <= 1) return gemm<T>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, a_lower, s);
    const int64_t Kc = K / S;
    // partial s: A[:, s*Kc ..] B[s*Kc .., :] into part + s*M*N (ld M); a
    // triangular A runs as a full one (its upper part holds exact zeros)
    hipError_t e = gemm_batched<T>(M, N, Kc, R(1), A, lda, Kc * lda, 0, B, ldb, Kc, 0, R(0), part, M,
                                   M * N, 0, S, S, false, s);
    if (e != hipSuccess) return e;
    constexpr int64_t f = traits<T>::is_complex ? 2 : 1;
    const int64_t total = M * f * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(reduce_kernel<R>, dim3((unsigned)blocks), dim3(256), 0, s, (const R *)part,
                       M * f, N, S, alpha, beta, (R *)C, ldc * f);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Diagonal-block inversion by the blocked-inverse formula
//
// The HSMA-TRSM paper's two-level blocking reuses the small-scale solver for
// the small diagonal sub-blocks and turns the inter-sub-block updates into
// matrix multiplies through the blocked matrix inversion formula:
//
//   [L11   0 ]^-1   [ L11^-1               0     ]
//   [L21  L22]    = [ -L22^-1 L21 L11^-1   L22^-1 ]
//
// Here: (1) every 64 x 64 diagonal sub-block is inverted by the small-regime
// lane-per-column kernel against an identity right-hand side, in place in
// invA; (2) sub-blocks are merged pairwise, 64 -> 128 -> ... -> N_B, each level
// two batched GEMMs over all pairs of all diagonal blocks:
//   T = L21 L11^-1,   (inverse)21 = -L22^-1 T   (L22^-1 lower: zero tiles skipped).
// Used when m is a multiple of N_B and N_B of 64; otherwise diag_inv_kernel.

template <typename T>
__global__ void __launch_bounds__(256) identity_kernel(T *out, int64_t total, int64_t nb)
{
    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t within = e % (nb * nb);
        out[e] = (within % nb == within / nb) ? one : zero_of(T());
    }
}

int64_t blocked_inverse_temp_elems(int64_t m, int nb)
{
    const int64_t nt = (m + nb - 1) / nb;
    return nt * (int64_t)nb * nb / 4 + 1;
}

template <typename T>
static bool blocked_inverse_applies(int64_t m, int nb)
{
    return m % nb == 0 && nb % 64 == 0 && nb >= 128;
}

// What HSMA_INV_AUTO takes: the blocked-inverse formula where it applies,
// except for blocks of 128 in f64 and c64 (of at most 256 in c128), where
// one column substitution launch measured as fast or faster on MI355X than
// the small solves plus log2(nb / 64) rounds of merge products.
template <typename T>
static bool auto_merges(int64_t m, int nb)
{
    if (!blocked_inverse_applies<T>(m, nb)) return false;
    if (std::is_same<T, float>::value) return true;
    return nb > (sizeof(T) == 16 ? 256 : 128);
}

template <typename T>
static hipError_t blocked_inverse(int64_t m, int nb, const T *A, int64_t lda, T *invA, T *temp,
                                  hipStream_t s)
{
    using R = typename traits<T>::real;
    const int64_t nt = m / nb;
    const int64_t total = nt * (int64_t)nb * nb;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(identity_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, invA, total,
                       (int64_t)nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    // (1) 64 x 64 diagonal sub-blocks: problem z = t * (nb/64) + k
    e = small_colane2<T>(64, one, A, lda, 64 * (lda + 1), nb * (lda + 1), invA, nb,
                         64 * ((int64_t)nb + 1), (int64_t)nb * nb, nb / 64, m / 64, s);
    if (e != hipSuccess) return e;
    // (2) merge pairs of s x s inverses
    for (int64_t sz = 64; sz < nb; sz *= 2) {
        const int64_t pairs = nb / (2 * sz), batch = nt * pairs;
        // T = L21 * inv11
        e = gemm_batched<T>(sz, sz, sz, R(1), A + sz, lda, 2 * sz * (lda + 1), (int64_t)nb * (lda + 1),
                            invA, nb, 2 * sz * ((int64_t)nb + 1), (int64_t)nb * nb, R(0), temp, sz,
                            sz * sz, pairs * sz * sz, pairs, batch, false, s);
        if (e != hipSuccess) return e;
        // inv21 = -inv22 * T. inv22 is lower triangular with exact zeros above
        // its diagonal; it is multiplied as a full matrix (the zero tiles add
        // exact zeros): at these sizes skipping them measured no faster for
        // f32 and f64.
        e = gemm_batched<T>(sz, sz, sz, R(-1), invA + sz * ((int64_t)nb + 1), nb,
                            2 * sz * ((int64_t)nb + 1), (int64_t)nb * nb, temp, sz, sz * sz,
                            pairs * sz * sz, R(0), invA + sz, nb, 2 * sz * ((int64_t)nb + 1),
                            (int64_t)nb * nb, pairs, batch, false, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Fused inversion of 2*I_B x 2*I_B diagonal blocks (the "traditional" fused
// kernel of the HSMA-TRSM paper's blocked section, kept as an A/B route):
// one workgroup holds a whole 2I_B x 2I_B diagonal block in LDS -- the
// paper's 4 I_B^2 elements, which caps I_B at 64 (32 for double complex) on
// gfx950's 160 KB -- inverts its two I_B x I_B diagonal blocks by
// substitution against identity columns (one lane per row, the columns in
// registers, rows broadcast with v_readlane), then forms
// the off-diagonal block of the inverse, -L22^{-1} L21 L11^{-1}, with two
// small products in LDS (T = L21 L11^{-1} kept in the otherwise unused upper
// right quarter). Larger blocks are then merged by the batched products of
// blocked_inverse.

template <typename T, int IB>
__global__ void __launch_bounds__(256) fused_inv_kernel(const T *__restrict__ A, int64_t lda,
                                                         int nb, T *__restrict__ invA)
{
    constexpr int S2 = 2 * IB;       // block order
    constexpr int LD = S2 + 1;       // LDS column stride (element (i, j) at j*LD + i)
    constexpr int RT = IB / 16;      // rows and columns of a thread's product sub-tile
    static_assert(IB % 16 == 0, "I_B must be a multiple of 16");
    extern __shared__ __attribute__((aligned(16))) char fused_lds[];
    T *S = (T *)fused_lds;
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * S2;           // first row of this block in A
    const T *D = A + r0 + r0 * lda;
    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;

    // (0) the lower triangle of the block into LDS (the diagonal blocks'
    // strictly upper parts are never read, the upper right quarter is T)
    for (int e = tid; e < S2 * S2; e += 256) {
        const int i = e % S2, j = e / S2;
        if (j <= i) S[j * LD + i] = D[i + (int64_t)j * lda];
    }
    __syncthreads();

    // (1) L11^{-1} and L22^{-1} by substitution against identity columns.
    // Wave w takes diagonal block q = w / 2 and half of its columns; lane i
    // holds row i of those columns in registers. Step j finishes row j
    // (scaled by 1/l_jj, exact zero left of the diagonal), broadcasts it with
    // v_readlane and the rows below subtract l_ij times it. Only the loop
    // over columns is unrolled, so no register array is indexed by j.
    {
        constexpr int NC = IB / 2;
        const int wave = tid >> 6, lane = tid & 63;
        const int o = (wave >> 1) * IB, cb = (wave & 1) * NC;
        T w[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) w[c] = pick(lane == cb + c, one, zero_of(T()));
        for (int j = 0; j < IB; ++j) {
            const T r = recip(S[(o + j) * LD + o + j]);
            T a = zero_of(T());
            if (lane < IB) a = S[(o + j) * LD + o + lane];   // l_ij of this block
            const bool below = lane > j, at = lane == j;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const T x = pick(j >= cb + c, mul(readlane(w[c], j), r), zero_of(T()));
                w[c] = pick(below, fms(w[c], a, x), pick(at, x, w[c]));
            }
        }
        __syncthreads();   // every coefficient read before the inverse overwrites them
        if (lane < IB) {
#pragma unroll
            for (int c = 0; c < NC; ++c) S[(o + cb + c) * LD + o + lane] = w[c];
        }
    }
    __syncthreads();

    // (2) -T = -L21 L11^{-1} into the upper right quarter: thread sub-tile
    // of RT x RT outputs, rows ti*RT.., columns tj*RT..
    const int ti = tid % 16, tj = tid / 16;
    {
        T acc[RT][RT];
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < RT; ++b) acc[a][b] = zero_of(T());
        for (int k = 0; k < IB; ++k) {
            T l[RT], v[RT];
#pragma unroll
            for (int a = 0; a < RT; ++a) l[a] = S[k * LD + IB + ti * RT + a];          // L21(i, k)
#pragma unroll
            for (int b = 0; b < RT; ++b) v[b] = S[(tj * RT + b) * LD + k];             // L11^{-1}(k, c)
#pragma unroll
            for (int a = 0; a < RT; ++a)
#pragma unroll
                for (int b = 0; b < RT; ++b) acc[a][b] = fms(acc[a][b], l[a], v[b]);    // -sum
        }
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < RT; ++b) S[(IB + tj * RT + b) * LD + ti * RT + a] = acc[a][b];
    }
    __syncthreads();

    // (3) the inverse's lower left block, L22^{-1} (-T), over L21
    {
        T acc[RT][RT];
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < RT; ++b) acc[a][b] = zero_of(T());
        for (int k = 0; k < IB; ++k) {
            T l[RT], v[RT];
#pragma unroll
            for (int a = 0; a < RT; ++a) l[a] = S[(IB + k) * LD + IB + ti * RT + a];   // L22^{-1}(i, k)
#pragma unroll
            for (int b = 0; b < RT; ++b) v[b] = S[(IB + tj * RT + b) * LD + k];        // -T(k, c)
#pragma unroll
            for (int a = 0; a < RT; ++a)
#pragma unroll
                for (int b = 0; b < RT; ++b) acc[a][b] = fms(acc[a][b], l[a], v[b]);
        }
        __syncthreads();   // every thread's reads done before L21 is overwritten
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < RT; ++b) {
                // acc = -(L22^{-1} (-T)): stored negated
                S[(tj * RT + b) * LD + IB + ti * RT + a] = fms(zero_of(T()), one, acc[a][b]);
            }
    }
    __syncthreads();

    // (4) the 2I_B x 2I_B inverse into invA (column-major, ld nb), zeros above
    // the diagonal
    const int64_t t = r0 / nb, off = r0 % nb;
    T *out = invA + t * (int64_t)nb * nb + off + off * nb;
    for (int e = tid; e < S2 * S2; e += 256) {
        const int i = e % S2, j = e / S2;
        out[i + (int64_t)j * nb] = (j <= i && !(i < IB && j >= IB)) ? S[j * LD + i] : zero_of(T());
    }
}

// Largest fused inner block for the element type (4 I_B^2 elements in LDS).
template <typename T>
constexpr int fused_max_ib() { return sizeof(T) == 16 ? 32 : 64; }

template <typename T>
static bool fused_inverse_applies(int64_t m, int nb, int ib)
{
    return (ib == 32 || ib == 64) && ib <= fused_max_ib<T>() && m % nb == 0 && nb % (2 * ib) == 0;
}

template <typename T>
static hipError_t fused_inverse(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA,
                                T *temp, hipStream_t s)
{
    using R = typename traits<T>::real;
    const int64_t nt = m / nb;
    const int64_t total = nt * (int64_t)nb * nb;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(identity_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, invA, total,
                       (int64_t)nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nblk = m / (2 * ib);
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)(2 * ib) * (2 * ib + 1) * sizeof(T);
    if (ib == 64) {
        if constexpr (fused_max_ib<T>() >= 64) {
            hipLaunchKernelGGL((fused_inv_kernel<T, 64>), dim3((unsigned)nblk), dim3(256), lds, s, A,
                               lda, nb, invA);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL((fused_inv_kernel<T, 32>), dim3((unsigned)nblk), dim3(256), lds, s, A,
                           lda, nb, invA);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // merge pairs of s x s inverses from 2 I_B up to N_B, as in blocked_inverse
    for (int64_t sz = 2 * ib; sz < nb; sz *= 2) {
        const int64_t pairs = nb / (2 * sz), batch = nt * pairs;
        e = gemm_batched<T>(sz, sz, sz, R(1), A + sz, lda, 2 * sz * (lda + 1), (int64_t)nb * (lda + 1),
                            invA, nb, 2 * sz * ((int64_t)nb + 1), (int64_t)nb * nb, R(0), temp, sz,
                            sz * sz, pairs * sz * sz, pairs, batch, false, s);
        if (e != hipSuccess) return e;
        e = gemm_batched<T>(sz, sz, sz, R(-1), invA + sz * ((int64_t)nb + 1), nb,
                            2 * sz * ((int64_t)nb + 1), (int64_t)nb * nb, temp, sz, sz * sz,
                            pairs * sz * sz, R(0), invA + sz, nb, 2 * sz * ((int64_t)nb + 1),
                            (int64_t)nb * nb, pairs, batch, false, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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

// Elements of T for a complex trailing panel or inverted diagonal block in
// real form, 2 x 2 reals per complex entry: at most max(m - nb, nb) x nb
// entries (0 for real types).
template <typename T>
static int64_t expand_elems(int64_t m, int nb)
{
    if (!traits<T>::is_complex) return 0;
    const int64_t rows = m - nb > nb ? m - nb : nb;  // a trailing panel or a diagonal block
    return 2 * rows * (int64_t)nb;
}

template <typename T>
int64_t blocked_workspace_elems(int64_t m, int64_t n, int nb)
{
    const int64_t nt = (m + nb - 1) / nb;
    int64_t w = (int64_t)nb * n;
    const int64_t t = blocked_inverse_temp_elems(m, nb);
    if (t > w) w = t;  // the merge temporaries live in W before W is used
    w = (w + 63) / 64 * 64;   // the split-K partials start 256-byte aligned
    const int64_t ex = expand_elems<T>(m, nb);
    const int64_t part = (splitk_part_elems(m, n) + 63) / 64 * 64;
    return nt * nb * nb + w + part + ex;
}

template <typename T>
bool invert_route_applies(int64_t m, int nb, int ib, int route)
{
    switch (route) {
    case HSMA_INV_AUTO: return true;
    case HSMA_INV_BLOCKED: return blocked_inverse_applies<T>(m, nb);
    case HSMA_INV_FUSED: return fused_inverse_applies<T>(m, nb, ib);
    case HSMA_INV_COLUMN: return nb <= 1024;
    default: return false;
    }
}

template <typename T>
hipError_t blocked_invert(int64_t m, int nb, int ib, const T *A, int64_t lda, T *invA, T *temp,
                          hipStream_t s, int route)
{
    if (!invert_route_applies<T>(m, nb, ib, route)) return hipErrorInvalidValue;
    if (route == HSMA_INV_FUSED) return fused_inverse<T>(m, nb, ib, A, lda, invA, temp, s);
    if (route == HSMA_INV_COLUMN) return diag_invert<T>(m, nb, ib, A, lda, invA, s);
    if (route == HSMA_INV_BLOCKED || (route == HSMA_INV_AUTO && auto_merges<T>(m, nb)))
        return blocked_inverse<T>(m, nb, A, lda, invA, temp, s);
    return diag_invert<T>(m, nb, ib, A, lda, invA, s);
}

// The complex panel P (M x K, column-major, ld lda) in real form E (2M x 2K,
// column-major, ld 2M): entry (i, k) becomes the 2 x 2 block [[re, -im],
// [im, re]] at rows 2i, 2i+1 and columns 2k, 2k+1, so E's column 2k is P's
// column k read as reals and column 2k+1 is (-im, re) pairs. The real
// product E * W (W read as real, 2K x n) is the complex product P * W with
// every real multiply-add of the complex kernel, which builds the same
// blocks on its way into LDS; expanding once per block row instead of per
// tile fetch halves the loads of A's panel and lets the product run as a
// real one.
template <typename R>
__global__ void __launch_bounds__(256) expand_kernel(const cplx<R> *__restrict__ P, int64_t lda, int64_t M,
                                                     R *__restrict__ E)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t k = blockIdx.y;
    if (i >= M) return;
    const cplx<R> a = P[i + k * lda];
    R *e0 = E + 2 * k * (2 * M) + 2 * i;
    R *e1 = e0 + 2 * M;
    e0[0] = a.re;
    e0[1] = a.im;
    e1[0] = -a.im;
    e1[1] = a.re;
}

template <typename T>
hipError_t blocked_apply(int64_t m, int64_t n, int nb, const T *A, int64_t lda, const T *invA,
                         T *B, int64_t ldb, T *W, hipStream_t s, PhaseRec *rec, T *part,
                         int64_t part_elems, const CopyOverlap *ov, T *expand)
{
    using R = typename traits<T>::real;
    const int64_t nt = (m + nb - 1) / nb;
    auto mark = [&](int ph) { return rec ? rec->mark(ph, s) : hipSuccess; };
    hipError_t e = hipSuccess;
    for (int64_t t = 0; t < nt && e == hipSuccess; ++t) {
        const int64_t r0 = t * nb;
        const int64_t rb = m - r0 < nb ? m - r0 : nb;
        // X_t = D_t^{-1} B_t (D_t^{-1} is lower triangular: upper tiles skipped)
        e = mark(HSMA_PHASE_INV_GEMM);
        bool inv_done = false;
        if constexpr (traits<T>::is_complex) {
            // products that would not be split along K: the inverted block in
            // real form (lower triangular in 2 x 2 blocks), then the real product
            const int64_t S = part ? splitk_chunks<T>(rb, n, rb, part_elems) : 1;
            if (e == hipSuccess && expand && S == 1) {
                hipLaunchKernelGGL(expand_kernel<R>, dim3((unsigned)((rb + 255) / 256), (unsigned)rb), dim3(256), 0,
                                   s, invA + t * nb * nb, (int64_t)nb, rb, (R *)expand);
                e = hipGetLastError();
                if (e == hipSuccess)
                    e = gemm<R>(2 * rb, n, 2 * rb, R(1), (const R *)expand, 2 * rb, (const R *)(B + r0),
                                2 * ldb, R(0), (R *)W, 2 * (int64_t)nb, 2, s);
                inv_done = true;
            }
        }
        if (e == hipSuccess && !inv_done)
            e = gemm_splitk<T>(rb, n, rb, R(1), invA + t * nb * nb, nb, B + r0, ldb, R(0), W, nb, true,
                               part, part_elems, s);
        if (e == hipSuccess) e = mark(HSMA_PHASE_COPY);
        if (e != hipSuccess) break;
        // X_t into B_t: on the second stream when given, after W is ready
        hipStream_t cs = s;
        if (ov) {
            e = hipEventRecord(ov->ready, s);
            if (e == hipSuccess) e = hipStreamWaitEvent(ov->aux, ov->ready, 0);
            if (e != hipSuccess) break;
            cs = ov->aux;
        }
        for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += 65535) {
            const int64_t nc = n - c0 < 65535 ? n - c0 : 65535;
            hipLaunchKernelGGL(copy_kernel<T>, dim3((unsigned)((rb + 255) / 256), (unsigned)nc),
                               dim3(256), 0, cs, W + c0 * nb, (int64_t)nb, rb, B + r0 + c0 * ldb, ldb);
            e = hipGetLastError();
        }
        bool copy_pending = false;
        if (ov) {
            const hipError_t ew = hipEventRecord(ov->copied, ov->aux);
            if (ew == hipSuccess) copy_pending = true;
            else (void)hipStreamSynchronize(ov->aux);
            if (e == hipSuccess) e = ew;
        }
        // B[below] -= A[below, t] X_t: reads W and writes only the rows below
        // B_t, so it runs beside the copy
        if (e == hipSuccess && r0 + rb < m) {
            e = mark(HSMA_PHASE_TRAILING);
            const int64_t mt = m - r0 - rb;
            bool done = false;
            if constexpr (traits<T>::is_complex) {
                // complex products that would not be split along K: the panel
                // in real form once, then the real product
                const int64_t S = part ? splitk_chunks<T>(mt, n, rb, part_elems) : 1;
                if (e == hipSuccess && expand && S == 1 && mt <= 0x7fffffffLL * 256 && rb <= 65535) {
                    hipLaunchKernelGGL(expand_kernel<R>, dim3((unsigned)((mt + 255) / 256), (unsigned)rb),
                                       dim3(256), 0, s, A + (r0 + rb) + r0 * lda, lda, mt, (R *)expand);
                    e = hipGetLastError();
                    if (e == hipSuccess)
                        e = gemm<R>(2 * mt, n, 2 * rb, R(-1), (const R *)expand, 2 * mt, (const R *)W,
                                    2 * (int64_t)nb, R(1), (R *)(B + r0 + rb), 2 * ldb, false, s);
                    done = true;
                }
            }
            if (e == hipSuccess && !done)
                e = gemm_splitk<T>(mt, n, rb, R(-1), A + (r0 + rb) + r0 * lda, lda, W, nb,
                                   R(1), B + r0 + rb, ldb, false, part, part_elems, s);
        }
        // s does not go on to overwrite W (next block row) or finish before
        // the copy has read it, also after a failure
        if (copy_pending) {
            const hipError_t ew = hipStreamWaitEvent(s, ov->copied, 0);
            if (ew != hipSuccess) (void)hipStreamSynchronize(ov->aux);
            if (e == hipSuccess) e = ew;
        }
        if (e != hipSuccess) break;
    }
    if (e == hipSuccess) e = mark(HSMA_PHASE_END);
    return e;
}

// Block rows of at least this many elements copy W -> B_t on the second
// stream: on MI355X the copy of an m = n = 8192 solve (N_B = 2048) is 2 % of
// it; below this size the event round trip costs about what it hides.
constexpr int64_t kOverlapMinElems = int64_t(1) << 22;

template <typename T>
hipError_t blocked_solve(int64_t m, int64_t n, int nb, int ib, const T *A, int64_t lda, T *B,
                         int64_t ldb, T *work, hipStream_t s, PhaseRec *rec, int route)
{
    const int64_t nt = (m + nb - 1) / nb;
    T *invA = work;
    T *W = work + nt * nb * nb;   // also the inversion's temporary, before W is used
    int64_t wlen = (int64_t)nb * n;
    const int64_t tl = blocked_inverse_temp_elems(m, nb);
    if (tl > wlen) wlen = tl;
    wlen = (wlen + 63) / 64 * 64;
    T *part = W + wlen;           // split-K partial products (few right-hand sides)
    const int64_t part_elems = splitk_part_elems(m, n);
    // complex: the trailing panel in real form (after the partials, 256-byte aligned)
    T *expand = expand_elems<T>(m, nb) > 0 ? part + (part_elems + 63) / 64 * 64 : nullptr;
    hipError_t e = rec ? rec->mark(HSMA_PHASE_DIAG_INV, s) : hipSuccess;
    if (e == hipSuccess) e = blocked_invert<T>(m, nb, ib, A, lda, invA, W, s, route);
    if (e != hipSuccess) return e;
    // Large block rows: the W -> B_t copies run on a second stream beside the
    // trailing products (not when the caller times the phases on s)
    CopyOverlap ov{};
    const bool overlap = !rec && nt > 1 && (int64_t)nb * n >= kOverlapMinElems &&
                         aux_stream(&ov.aux) == hipSuccess &&
                         hipEventCreateWithFlags(&ov.ready, hipEventDisableTiming) == hipSuccess;
    const bool overlap2 = overlap &&
                          hipEventCreateWithFlags(&ov.copied, hipEventDisableTiming) == hipSuccess;
    e = blocked_apply<T>(m, n, nb, A, lda, invA, B, ldb, W, s, rec, part_elems ? part : nullptr,
                         part_elems, overlap2 ? &ov : nullptr, expand);
    // (events still pending are released by the runtime once they complete)
    if (overlap) (void)hipEventDestroy(ov.ready);
    if (overlap2) (void)hipEventDestroy(ov.copied);
    return e;
}

#define HSMA_INST(T)                                                                              \
    template hipError_t diag_invert<T>(int64_t, int, int, const T *, int64_t, T *, hipStream_t);  \
    template hipError_t diag_invert_any<T>(int64_t, int, int, const T *, int64_t, T *, hipStream_t, \
                                           int);                                                  \
    template bool invert_route_applies<T>(int64_t, int, int, int);                                \
    template hipError_t gemm<T>(int64_t, int64_t, int64_t, typename traits<T>::real, const T *,    \
                                int64_t, const T *, int64_t, typename traits<T>::real, T *,       \
                                int64_t, int, hipStream_t);                                       \
    template hipError_t gemm_strided<T>(int64_t, int64_t, int64_t, typename traits<T>::real,       \
                                        const T *, int64_t, int64_t, const T *, int64_t, int64_t, \
                                        typename traits<T>::real, T *, int64_t, int64_t, int64_t, \
                                        hipStream_t);                                             \
    template hipError_t blocked_solve<T>(int64_t, int64_t, int, int, const T *, int64_t, T *,     \
                                         int64_t, T *, hipStream_t, PhaseRec *, int);             \
    template hipError_t blocked_invert<T>(int64_t, int, int, const T *, int64_t, T *, T *,        \
                                          hipStream_t, int);                                      \
    template hipError_t blocked_apply<T>(int64_t, int64_t, int, const T *, int64_t, const T *, T *, \
                                         int64_t, T *, hipStream_t, PhaseRec *, T *, int64_t,   \
                                         const CopyOverlap *, T *);                              \
    template int64_t blocked_workspace_elems<T>(int64_t, int64_t, int);
HSMA_INST(float)
HSMA_INST(double)
HSMA_INST(c32)
HSMA_INST(c64)
#undef HSMA_INST

}  // namespace hsma
