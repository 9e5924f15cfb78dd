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

    const int64_t b = blockIdx.x;
    const int64_t i2 = b % p.ne02, i3 = b / p.ne02;
    const T *Ab = p.A + i2 * p.sa2 + i3 * p.sa3;
    const T *Bb = p.B + i2 * p.sb2 + i3 * p.sb3;
    T *Xb = p.X + i2 * p.sx2 + i3 * p.sx3;
    const int m = p.m;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;

    T one = zero_of(T());
    if constexpr (traits<T>::is_complex) one.re = 1; else one = 1;
    // Lane i owns row i: its own 1/a_ii, no exchange needed.
    const T inv = recip(lane < m ? Ab[lane * (p.sai + p.saj)] : one);

    // Stage tril(A) scaled by its row's inverse diagonal, strictly lower part
    // only (diagonal and above are zero), transposed: AT[j][i] = a_ij / a_ii.
    // Wave w takes columns j = w, w + nw, ...; the loop is unrolled so the
    // loads of a group are all in flight together.
    const int per = (64 + nw - 1) / nw;
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        const int j = wave * per + t;
        if (t < per && j < 64) {
            T v = zero_of(T());
            if (lane < m && j < lane) v = mul(Ab[lane * p.sai + j * p.saj], inv);
            AT[j * kLdsStride + lane] = v;
        }
    }

    // This wave's right-hand-side columns, one row per lane, pre-scaled the
    // same way: w_i = alpha * b_i / a_ii.
    const int c0 = (blockIdx.y * nw + wave) * KW;
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
    auto step = [&](int j) {
        const T a = AT[j * kLdsStride + lane];
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const T x = readlane(w[q], j);
            w[q] = fms(w[q], a, x);
        }
    };
    if (m == 64) {
#pragma unroll
        for (int j = 0; j < 64; ++j) step(j);
    } else {
        for (int j = 0; j < m; ++j) step(j);
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
template <typename T>
using gptr = __attribute__((address_space(1))) T *;

// p, made to look modified once dep is available (no instruction emitted),
// returned as a global-address-space pointer so loads through it stay
// global_load (a generic pointer would turn them into flat loads, which also
// count against the scalar-load counter).
template <typename T, typename D>
__device__ __forceinline__ gptr<T> global_after(T *p, const D &dep)
{
    uint64_t a = (uint64_t)p;
    if constexpr (traits<D>::is_complex) asm volatile("" : "+v"(a) : "v"(dep.re));
    else asm volatile("" : "+v"(a) : "v"(dep));
    return (gptr<T>)a;
}

// Same for a wave-uniform pointer (kept in SGPRs).
template <typename T, typename D>
__device__ __forceinline__ T *uniform_after(T *p, const D &dep)
{
    uint64_t a = (uint64_t)p;
    if constexpr (traits<D>::is_complex) asm volatile("" : "+s"(a) : "v"(dep.re));
    else asm volatile("" : "+s"(a) : "v"(dep));
    return (T *)a;
}

template <typename T>
__device__ __forceinline__ T ld_global(gptr<T> p, int idx)
{
    if constexpr (traits<T>::is_complex) {
        using R = typename traits<T>::real;
        const gptr<R> q = (gptr<R>)p;
        return T{q[2 * idx], q[2 * idx + 1]};
    } else {
        return p[idx];
    }
}

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

// Empty asm that makes v look modified after `dep` is available: values
// derived from v cannot be computed before dep. Emits no instruction.
template <typename V, typename T>
__device__ __forceinline__ void order_after(V &v, const T &dep)
{
    if constexpr (traits<T>::is_complex) asm volatile("" : "+s"(v) : "v"(dep.re));
    else asm volatile("" : "+s"(v) : "v"(dep));
}

// Compile-time plan of the coefficient stream of one row panel [R0, R0+P)
// of the lane-per-column solve. The stream is a list of column segments:
// first the R0 earlier columns (rows R0..R0+P-1 each, applied with the
// finished x_k read back), then the panel's own columns j (rows below j).
// Segments are cut into pieces and the pieces packed into batches of at
// most G coefficients. A batch is fetched with scalar loads and consumed
// after a single wait: scalar loads can return out of order, so every wait
// is a full wait, and fewer, larger batches mean fewer exposed latencies.
template <int P, int R0, int G>
struct PanelPlan {
    struct Piece {
        int col, lo, hi;  // column of A, panel-local rows [lo, hi)
        int first;        // first piece of its segment: x is formed here
        int reload;       // segment of an earlier panel: x is read back
    };
    static constexpr int count()
    {
        int n = 0;
        for (int k = 0; k < R0; ++k) n += (P + G - 1) / G;
        for (int j = 0; j < P; ++j) n += (P - 1 - j) == 0 ? 1 : (P - 1 - j + G - 1) / G;
        return n;
    }
    static constexpr int NP = count();
    struct Table {
        Piece pc[NP];
        int off[NP];       // offset of the piece inside its batch buffer
        int bfirst[NP + 1];
        int nbatch;
    };
    static constexpr Table build()
    {
        Table t{};
        int n = 0;
        for (int k = 0; k < R0; ++k)
            for (int lo = 0; lo < P; lo += G)
                t.pc[n++] = Piece{k, lo, lo + G < P ? lo + G : P, lo == 0, 1};
        for (int j = 0; j < P; ++j) {
            if (j + 1 == P) { t.pc[n++] = Piece{R0 + j, P, P, 1, 0}; continue; }
            for (int lo = j + 1; lo < P; lo += G)
                t.pc[n++] = Piece{R0 + j, lo, lo + G < P ? lo + G : P, lo == j + 1, 0};
        }
        int b = 0, used = 0;
        t.bfirst[0] = 0;
        for (int i = 0; i < NP; ++i) {
            const int L = t.pc[i].hi - t.pc[i].lo;
            if (used + L > G && used > 0) { ++b; used = 0; t.bfirst[b] = i; }
            t.off[i] = used;
            used += L;
        }
        t.nbatch = b + 1;
        t.bfirst[t.nbatch] = NP;
        return t;
    }
    static constexpr Table T = build();
};

// Coefficients per batch: 64 dwords of SGPRs.
template <typename T>
constexpr int kBatch = (int)(256 / sizeof(T));

// Per-panel state shared by the batch recursion below.
template <typename T, int P>
struct PanelState {
    T w[P];       // this lane's rows of the panel
    T x;          // multiplier of the current column segment
    cptr<T> a4;   // A of this problem (scalar loads)
    int64_t lda;
    T *Bc;        // this lane's column of B (read back finished rows)
    T myinv;      // 1/a_ll of this lane's row index l
    T alpha_inv;
};

// Scalar loads of the pieces [Q, Q1) of a batch into cb.
template <typename T, int P, int R0, int G, int Q, int Q1>
__device__ __forceinline__ void batch_load(T (&cb)[G], cptr<T> ap, int64_t lda)
{
    if constexpr (Q < Q1) {
        using Plan = PanelPlan<P, R0, G>;
        constexpr auto pc = Plan::T.pc[Q];
        constexpr int off = Plan::T.off[Q];
        const cptr<T> colp = ap + (R0 + (int64_t)pc.col * lda);
#pragma unroll
        for (int r = pc.lo; r < pc.hi; ++r) cb[off + r - pc.lo] = ld_uniform<T>(colp, r);
        batch_load<T, P, R0, G, Q + 1, Q1>(cb, ap, lda);
    }
}

// The updates of pieces [Q, Q1) of a batch.
template <typename T, int P, int R0, int G, int Q, int Q1>
__device__ __forceinline__ void batch_compute(PanelState<T, P> &st, const T (&cb)[G])
{
    if constexpr (Q < Q1) {
        using Plan = PanelPlan<P, R0, G>;
        constexpr auto pc = Plan::T.pc[Q];
        constexpr int off = Plan::T.off[Q];
        if constexpr (pc.first) {
            if constexpr (pc.reload) {
                // finished x_k of an earlier panel, read back from B
                const gptr<T> bk = global_after(st.Bc + pc.col, st.x);
                st.x = mul(ld_global<T>(bk, 0), st.alpha_inv);
            } else {
                constexpr int j = pc.col - R0;
                // Tie the broadcast of 1/a_jj to w[j] so the compiler cannot
                // hoist all broadcasts to the top (that would exhaust SGPRs).
                T inv = st.myinv;
                if constexpr (traits<T>::is_complex) {
                    asm volatile("" : "+v"(inv.re), "+v"(inv.im) : "v"(st.w[j].re), "v"(st.w[j].im));
                } else {
                    asm volatile("" : "+v"(inv) : "v"(st.w[j]));
                }
                st.x = mul(st.w[j], readlane(inv, pc.col));
                st.w[j] = st.x;
            }
        }
#pragma unroll
        for (int r = pc.lo; r < pc.hi; ++r) st.w[r] = fms(st.w[r], cb[off + r - pc.lo], st.x);
        batch_compute<T, P, R0, G, Q + 1, Q1>(st, cb);
    }
}

// Batches [Bi, nbatch) of the panel at rows R0: fetch, one wait, update.
template <typename T, int P, int R0, int G, int Bi>
__device__ __forceinline__ void run_batches(PanelState<T, P> &st)
{
    using Plan = PanelPlan<P, R0, G>;
    if constexpr (Bi < Plan::T.nbatch) {
        constexpr int p0 = Plan::T.bfirst[Bi], p1 = Plan::T.bfirst[Bi + 1];
        // fetch this batch once the previous one has been consumed
        cptr<T> ap = st.a4;
        order_after(ap, st.x);
        T cb[G];
        batch_load<T, P, R0, G, p0, p1>(cb, ap, st.lda);
        batch_compute<T, P, R0, G, p0, p1>(st, cb);
        __builtin_amdgcn_sched_barrier(0);
        run_batches<T, P, R0, G, Bi + 1>(st);
    }
}

template <typename T, int P, int NPANEL, int PI>
__device__ __forceinline__ void run_panels(PanelState<T, P> &st, bool live, T alpha,
                                           typename traits<T>::real wlast)
{
    if constexpr (PI < NPANEL) {
        constexpr int r0 = PI * P;
        // a later panel's rows are loaded only after the earlier panel is done
        const gptr<T> bp = global_after(st.Bc, wlast);
#pragma unroll
        for (int r = 0; r < P; ++r) st.w[r] = ld_global<T>(bp, r0 + r);
        st.x = zero_of(T());
        run_batches<T, P, r0, kBatch<T>, 0>(st);
        // The solve ran on B itself; alpha is applied to X on the way out
        // (A (alpha^{-1} X) = B has the same substitution with alpha factored out).
        if (live) {
#pragma unroll
            for (int r = 0; r < P; ++r) st.Bc[r0 + r] = mul(alpha, st.w[r]);
        }
        typename traits<T>::real wl;
        if constexpr (traits<T>::is_complex) wl = st.w[P - 1].re; else wl = st.w[P - 1];
        run_panels<T, P, NPANEL, PI + 1>(st, live, alpha, wl);
    }
}

template <typename T, int NPANEL>
__global__ void __launch_bounds__(256, sizeof(T) == 4 ? 4 : 2) colane_kernel(const T *__restrict__ A, int64_t lda,
                                                         int64_t strideA, T *__restrict__ B,
                                                         int64_t ldb, int64_t strideB, int64_t n,
                                                         int64_t nchunks, int64_t items, T alpha,
                                                         T alpha_inv, int64_t per, int64_t strideA2,
                                                         int64_t strideB2)
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

    // problem prob = g * per + k lives at A + g*strideA2 + k*strideA (B alike)
    const int64_t pg = prob / per, pk = prob % per;
    const T *Ap = A + pg * strideA2 + pk * strideA;
    // Lanes past n work on a copy of the wave's first column (always valid)
    // and never store, so loads need no guard.
    T *Bc0 = B + pg * strideB2 + pk * strideB + cfirst * ldb;

    PanelState<T, P> st;
    st.a4 = (cptr<T>)Ap;
    st.lda = lda;
    st.Bc = Bc0 + (live ? lane : 0) * ldb;
    st.alpha_inv = alpha_inv;

    // Warm L2 with this problem's triangle: lane l touches every cache line
    // of column l from the diagonal down, one dword per line, so the scalar
    // loads below find the coefficients in L2 instead of HBM.
    constexpr int kLine = 128 / (int)sizeof(T);  // elements per 128-byte line
    constexpr int kTouch = 64 / kLine + 2;
    uint32_t touch[kTouch];
    {
        const uint32_t *colp = (const uint32_t *)(Ap + lane * lda);
#pragma unroll
        for (int q = 0; q < kTouch; ++q) {
            int row = lane + q * kLine;
            row = row < 63 ? row : 63;
            touch[q] = colp[row * (int)(sizeof(T) / 4)];
        }
    }
    st.myinv = recip(Ap[lane + lane * lda]);
    run_panels<T, P, NPANEL, 0>(st, live, alpha, typename traits<T>::real(0));
#pragma unroll
    for (int q = 0; q < kTouch; ++q) asm volatile("" ::"v"(touch[q]));
}

// Compute units of the current device (cached per device).
static int num_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

template <typename T>
hipError_t small_colane(int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA, T *B,
                        int64_t ldb, int64_t strideB, int64_t batch, hipStream_t s)
{
    return small_colane2<T>(n, alpha, A, lda, strideA, 0, B, ldb, strideB, 0, batch, batch, s);
}

template <typename T>
hipError_t small_colane2(int64_t n, T alpha, const T *A, int64_t lda, int64_t strideA,
                         int64_t strideA2, T *B, int64_t ldb, int64_t strideB, int64_t strideB2,
                         int64_t per, int64_t batch, hipStream_t s)
{
    if (per <= 0) per = 1;
    const int64_t nchunks = (n + 63) / 64;
    const int64_t items = nchunks * batch;
    const int64_t blocks = (items + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // Whole 64-row columns in registers for f32, f64 and c64 (no re-reads of
    // finished rows); two row panels for c128, whose full column would take
    // all 256 VGPRs. Measured on MI355X against 2/2/4 panels at 4 waves per
    // SIMD: f64 139 -> 114 us, c64 149 -> 136 us, c128 422 -> 291 us per
    // 4096 problems (re-read rows had been evicted from L2 and came back
    // from HBM).
    constexpr int NP = sizeof(T) == 16 ? 2 : 1;
    // Earlier panels' rows are read back from B already scaled by alpha.
    const T alpha_inv = host_recip(alpha);
    // Spread the workgroups evenly over the CUs: left alone, the dispatcher
    // may pack up to the occupancy limit onto fewer CUs. Reserving LDS (the
    // kernel uses none) caps the workgroups per CU at the even share.
    const int64_t per_cu = (blocks + num_cus() - 1) / num_cus();
    size_t lds = 0;
    if (per_cu >= 3 && per_cu < 8) lds = ((size_t)(160 * 1024) / (size_t)per_cu) & ~(size_t)1023;
    hipLaunchKernelGGL((colane_kernel<T, NP>), dim3((unsigned)blocks), dim3(256), lds, s, A, lda,
                       strideA, B, ldb, strideB, n, nchunks, items, alpha, alpha_inv, per, strideA2,
                       strideB2);
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
    template hipError_t small_colane2<T>(int64_t, T, const T *, int64_t, int64_t, int64_t, T *,    \
                                         int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);\
    template hipError_t scale_matrix<T>(T *, int64_t, int64_t, int64_t, int64_t, int64_t, T, bool, \
                                        hipStream_t);
HSMA_INST(float)
HSMA_INST(double)
HSMA_INST(c32)
HSMA_INST(c64)
#undef HSMA_INST

}  // namespace hsma
