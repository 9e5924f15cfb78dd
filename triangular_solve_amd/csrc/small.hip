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
#include <type_traits>

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
    int unit;  // unit diagonal: a_ii = 1, the stored diagonal is not read
};

// One, as the first element of a float or double array, for the unit
// diagonal: its address stands in for the diagonal with stride 0.
__device__ const float kOneF[2] = {1.0f, 0.0f};
__device__ const double kOneD[2] = {1.0, 0.0};
template <typename T>
__device__ __forceinline__ const T *unit_one()
{
    if constexpr (std::is_same<typename traits<T>::real, float>::value) return (const T *)kOneF;
    else return (const T *)kOneD;
}

constexpr int kLdsStride = 65;  // padded LDS column stride of the staged triangle

// RR: lane i keeps row i of A in registers, loaded with 16-byte loads (real
// types, m = 64, rows contiguous and 16-byte aligned: the ggml row-major
// layout). Then nothing is staged in LDS and no barrier is needed; step j
// reads its coefficient a_ij from register j.
template <typename T, int KW, bool RR>
__global__ void __launch_bounds__(256) rowlane_kernel(RowlaneArgs<T> p)
{
    __shared__ T AT[RR ? 1 : 64 * kLdsStride];

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
    // Lane i owns row i: its own 1/a_ii, no exchange needed. A unit
    // diagonal reads the constant one instead (stride 0).
    const T *dg = p.unit ? unit_one<T>() : Ab;
    const int64_t sdg = p.unit ? 0 : p.sai + p.saj;
    T d = one;
    if (lane < m) d = dg[lane * sdg];
    const T inv = recip(d);

    if constexpr (RR) {
        static_assert(!traits<T>::is_complex, "row registers for real types only");
        constexpr int V = 16 / (int)sizeof(T);
        typedef T vec_t __attribute__((ext_vector_type(V)));
        // a[j] = a_ij / a_ii below the diagonal, 0 on and above it
        T a[64];
        const T *Ar = Ab + lane * p.sai;
#pragma unroll
        for (int k = 0; k < 64 / V; ++k) {
            const vec_t v = *(const vec_t *)(Ar + k * V);
#pragma unroll
            for (int e = 0; e < V; ++e) a[k * V + e] = v[e];
        }
        const int c0 = (blockIdx.y * nw + wave) * KW;
        T w[KW];
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const int c = c0 + q;
            w[q] = c < p.n ? mul(mul(p.alpha, Bb[lane * p.sbi + c * p.sbj]), inv) : zero_of(T());
        }
#pragma unroll
        for (int j = 0; j < 64; ++j) a[j] = j < lane ? mul(a[j], inv) : zero_of(T());
        // Step j updates only the rows below j: a finished row keeps its
        // value even when a later x_j is inf or NaN (0 * inf would be NaN).
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const bool below = j < lane;
#pragma unroll
            for (int q = 0; q < KW; ++q) {
                const T u = fms(w[q], a[j], readlane(w[q], j));
                w[q] = pick(below, u, w[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const int c = c0 + q;
            if (c < p.n) Xb[lane * p.sxi + c * p.sxj] = w[q];
        }
        return;
    }

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
    // j keep their value (also when x_j is inf or NaN).
    auto step = [&](int j) {
        const T a = AT[j * kLdsStride + lane];
        const bool below = j < lane;
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            const T x = readlane(w[q], j);
            const T u = fms(w[q], a, x);
            w[q] = pick(below, u, w[q]);
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
    const dim3 grid((unsigned)nprob, (unsigned)ychunks);
    // Rows in registers: m = 64, contiguous 16-byte aligned rows of A (all
    // problems), real types with few columns per wave.
    const int64_t sz = (int64_t)sizeof(T);
    const bool rr = !traits<T>::is_complex && KW <= 4 && p.m == 64 && p.saj == 1 &&
                    (uintptr_t)p.A % 16 == 0 && (p.sai * sz) % 16 == 0 &&
                    (p.sa2 * sz) % 16 == 0 && (p.sa3 * sz) % 16 == 0;
    if constexpr (!traits<T>::is_complex && KW <= 4) {
        if (rr) {
            hipLaunchKernelGGL((rowlane_kernel<T, KW, true>), grid, dim3(64 * nwaves), 0, s, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((rowlane_kernel<T, KW, false>), grid, dim3(64 * nwaves), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t small_rowlane(const T *A, int64_t sai, int64_t saj, int64_t sa2, int64_t sa3,
                         const T *B, int64_t sbi, int64_t sbj, int64_t sb2, int64_t sb3,
                         T *X, int64_t sxi, int64_t sxj, int64_t sx2, int64_t sx3,
                         int64_t m, int64_t n, int64_t ne02, int64_t ne03, T alpha, hipStream_t s,
                         bool unit)
{
    RowlaneArgs<T> p;
    p.unit = unit ? 1 : 0;
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

// 16 bytes as four dwords: the unit of B's tile traffic.
typedef int v4i __attribute__((ext_vector_type(4)));
using lptr = __attribute__((address_space(3))) char *;
using lptr_v4i = __attribute__((address_space(3))) v4i *;

// Orders this wave's LDS accesses before and after the call: lanes exchange
// data through the wave's own tile, and the fences keep the compiler from
// moving an access across the exchange (one wave's LDS operations complete
// in issue order, so no wait is needed in hardware).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// B and X stream through the vector path with the non-temporal hint: each
// line is used once, and marking it for early eviction leaves L2 to the
// triangle lines that the coefficient prefetch brings in ahead of the scalar
// loads (4096 problems of 64 x 64, MI355X: f32 51.6 -> 38.8 us, f64
// 97.8 -> 83.6 us, c64 127 -> 114 us per launch).
template <typename T>
__device__ __forceinline__ v4i ld_b(gptr<T> p)
{
    return __builtin_nontemporal_load((const gptr<v4i>)p);
}
template <bool NT = true, typename T>
__device__ __forceinline__ void st_x(gptr<T> p, v4i v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, (gptr<v4i>)p);
    else *(gptr<v4i>)p = v;
}

// Per-wave LDS tile of 64 columns x one 128-byte line; the 16-byte pad of
// the column stride keeps both the line-wise and the column-wise 16-byte
// accesses free of bank conflicts.
constexpr int kTileCol = 144;
constexpr int kTileBytes = 64 * kTileCol;

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
// DIAG: an own column's segment starts at its diagonal entry, so the batch
// also brings a_jj and x_j = w_j / a_jj is formed from it.
template <int P, int R0, int G, bool DIAG>
struct PanelPlan {
    struct Piece {
        int col, lo, hi;  // column of A, panel-local rows [lo, hi)
        int first;        // first piece of its segment: x is formed here
        int reload;       // segment of an earlier panel: x is read back
        int diag;         // row lo is the diagonal entry a_jj
    };
    static constexpr int count()
    {
        int n = 0;
        for (int k = 0; k < R0; ++k) n += (P + G - 1) / G;
        for (int j = 0; j < P; ++j)
            n += DIAG ? (P - j + G - 1) / G : (P - 1 - j) == 0 ? 1 : (P - 1 - j + G - 1) / G;
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
                t.pc[n++] = Piece{k, lo, lo + G < P ? lo + G : P, lo == 0, 1, 0};
        for (int j = 0; j < P; ++j) {
            if (DIAG) {
                for (int lo = j; lo < P; lo += G)
                    t.pc[n++] = Piece{R0 + j, lo, lo + G < P ? lo + G : P, lo == j, 0, lo == j};
                continue;
            }
            if (j + 1 == P) { t.pc[n++] = Piece{R0 + j, P, P, 1, 0, 0}; continue; }
            for (int lo = j + 1; lo < P; lo += G)
                t.pc[n++] = Piece{R0 + j, lo, lo + G < P ? lo + G : P, lo == j + 1, 0, 0};
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

// The diagonal travels with the coefficient stream for the real types: f32
// takes one v_rcp_f32 of the scalar value (within an ulp), f64 v_rcp_f64
// refined by two Newton steps. For the complex types a reciprocal per column
// would cost more instructions, so every lane computes 1/a_ll of its row
// once at the start.
template <typename T>
constexpr bool kDiagInStream = std::is_same<T, float>::value || std::is_same<T, double>::value;

// Coefficients per batch: 64 dwords of SGPRs.
template <typename T>
constexpr int kBatch = (int)(256 / sizeof(T));

// Prefetch distance of A's coefficients, in stream coefficients. Measured
// on MI355X (4096 problems of 64 x 64) from 32 to 768 coefficients: 96 is
// best for f32, f64 and c64, 48 for c128; further ahead loses (the lines
// compete for L2 with the other resident waves' lines).
template <typename T>
constexpr int kAhead = sizeof(T) == 16 ? 48 : 96;

// L2 prefetch schedule of a panel's coefficient stream. Every non-empty
// column segment s (one column of A, rows [lo, hi) of the panel) has its
// cache lines fetched by a vector load at batch tb(s), the batch in which
// the stream reaches AH coefficients before the segment, and the load's
// result is retired at batch cb(s), the batch that reads the segment with
// scalar loads. The scalar loads then find the lines in L2 instead of
// waiting on HBM with a full wait each. Both tb and cb grow with s, so each
// batch handles a contiguous range of segments.
template <int P, int R0, int G, int AH, bool DIAG>
struct TouchPlan {
    using Plan = PanelPlan<P, R0, G, DIAG>;
    static constexpr int NS = R0 + P - (DIAG ? 0 : 1);
    struct Seg {
        int col, lo, hi;
    };
    struct Table {
        Seg sg[NS > 0 ? NS : 1];
        int tfirst[Plan::NP + 1];  // segments touched at batch b: [tfirst[b], tfirst[b+1])
        int cfirst[Plan::NP + 1];  // segments retired at batch b: [cfirst[b], cfirst[b+1])
    };
    static constexpr Table build()
    {
        Table t{};
        constexpr auto &pt = Plan::T;
        int bpos[Plan::NP + 1] = {};
        int tb[NS > 0 ? NS : 1] = {}, cb[NS > 0 ? NS : 1] = {};
        int pos = 0, ns = 0;
        for (int b = 0; b < pt.nbatch; ++b) {
            bpos[b] = pos;
            for (int i = pt.bfirst[b]; i < pt.bfirst[b + 1]; ++i) {
                const auto &pc = pt.pc[i];
                if (pc.first && pc.hi > pc.lo) {
                    // a segment runs over consecutive pieces of one column
                    int hi = pc.hi;
                    for (int k = i + 1; k < Plan::NP && !pt.pc[k].first; ++k) hi = pt.pc[k].hi;
                    t.sg[ns] = Seg{pc.col, pc.lo, hi};
                    cb[ns] = b;
                    int at = 0;
                    while (at + 1 < pt.nbatch && pos - AH >= bpos[at + 1] && at + 1 <= b) ++at;
                    tb[ns] = at;
                    ++ns;
                }
                pos += pc.hi - pc.lo;
            }
        }
        bpos[pt.nbatch] = pos;
        for (int b = 0; b <= pt.nbatch; ++b) {
            int f = 0, c = 0;
            while (f < ns && tb[f] < b) ++f;
            while (c < ns && cb[c] < b) ++c;
            t.tfirst[b] = f;
            t.cfirst[b] = c;
        }
        return t;
    }
    static constexpr Table T = build();
};

// Kept-column panels (f64, c64 in launches of many problems): the whole
// 64-row column stays in registers and is solved in row panels of one
// 128-byte line; a panel applies the finished rows of the earlier panels
// straight from registers (no row is read back from memory, and each element
// sees its updates in the same order as in one panel), while the next panel's
// lines of B are on their way. f32, and f64 and c64 in smaller launches,
// solve the kept column in one panel (P = 64); double complex keeps only its
// current panel (a whole column would take all 256 VGPRs) and reads the
// earlier rows back from X.
template <typename T, int P>
constexpr bool kKeep = sizeof(T) == 8 && P < 64;

// Rows per kept-column panel (one 128-byte line).
template <typename T>
constexpr int kKeepRows = 128 / (int)sizeof(T);

// Where the coefficient prefetch loads land. Their results are never used;
// a load into registers has to be waited for before the registers are
// reused (and the wait, in issue order, also waits for every load issued
// before it, such as the next panel's B lines), so the kept-column panels
// direct them into a few LDS bytes that nothing reads.
// For the single-panel f32 solve the waits are harmless and the LDS form
// measured slower (38.4 -> 47.5 us per 4096 problems).
template <typename T, int P>
constexpr bool kTouchLds = kKeep<T, P>;

// Registers of a lane's column, and the register of panel row 0 of the panel
// at rows R0.
template <typename T, int P>
constexpr int kRegs = kKeep<T, P> ? 64 : P;
template <typename T, int P, int R0>
constexpr int kRegOff = kKeep<T, P> ? R0 : 0;

// Per-panel state shared by the batch recursion below.
template <typename T, int P>
struct PanelState {
    T w[kRegs<T, P>];  // this lane's rows (all of them, or the current panel's)
    T x;          // multiplier of the current column segment
    cptr<T> a4;   // A of this problem (scalar loads)
    int64_t lda;
    T *Bw;        // first of the wave's 64 columns of B
    int64_t ldb;
    int ncol;     // columns of the wave that exist (<= 64)
    lptr tile;    // this wave's LDS tile
    int lane128;  // lane * 128: this lane's line of a prefetched segment
    int tv[64];   // results of the segments' prefetch loads, retired later
    lptr sink;    // LDS bytes the prefetch loads write to (never read)
    T myinv;      // 1/a_ll of this lane's row index l
};

// alpha * rows [r0, r0 + P) of the wave's columns into st.w, lane = column.
// Each 128-byte line of a column is fetched by 8 lanes with 16-byte loads (a
// lane-per-column load would touch 64 lines per instruction), written to
// the tile and read back one column per lane. The next tile's loads are in
// flight while the current one is transposed.
template <typename T, int P>
__device__ __forceinline__ void load_panel(PanelState<T, P> &st, gptr<T> bw, int r0, T alpha,
                                           bool scale)
{
    constexpr int V = 16 / (int)sizeof(T);
    constexpr int L = 128 / (int)sizeof(T);
    constexpr int NCH = P / L;
    static_assert(P % L == 0, "panel rows must be whole lines");
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
    int64_t goff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        int col = q * 8 + (lane >> 3);
        col = col < st.ncol ? col : st.ncol - 1;  // duplicates of a valid column
        goff[q] = col * st.ldb + r0 + sub * V;
    }
    v4i cur[8], nxt[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) cur[q] = ld_b(bw + goff[q]);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch + 1 < NCH) {
#pragma unroll
            for (int q = 0; q < 8; ++q) nxt[q] = ld_b(bw + goff[q] + (ch + 1) * L);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            *(lptr_v4i)(st.tile + (q * 8 + (lane >> 3)) * kTileCol + sub * 16) = cur[q];
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const v4i v = *(const lptr_v4i)(st.tile + lane * kTileCol + k * 16);
            T t[V];
            __builtin_memcpy(t, &v, 16);
#pragma unroll
            for (int e = 0; e < V; ++e) st.w[ch * L + k * V + e] = t[e];
        }
        wave_lds_sync();
        if (ch + 1 < NCH) {
#pragma unroll
            for (int q = 0; q < 8; ++q) cur[q] = nxt[q];
        }
    }
    // alpha applied on the way in, so the solve and every stored row of X
    // are in the units of X (a later panel reads finished rows back as they
    // are)
    if (scale) {
#pragma unroll
        for (int e = 0; e < P; ++e) st.w[e] = mul(alpha, st.w[e]);
    }
}

// st.w into rows [r0, r0 + P) of the wave's columns, the reverse of
// load_panel (columns past ncol are not written).
template <typename T, int P, bool NT = true>
__device__ __forceinline__ void store_panel(PanelState<T, P> &st, gptr<T> bw, int r0)
{
    constexpr int V = 16 / (int)sizeof(T);
    constexpr int L = 128 / (int)sizeof(T);
    constexpr int NCH = P / L;
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            T t[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = st.w[ch * L + k * V + e];
            v4i v;
            __builtin_memcpy(&v, t, 16);
            *(lptr_v4i)(st.tile + lane * kTileCol + k * 16) = v;
        }
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int col = q * 8 + (lane >> 3);
            const v4i v = *(const lptr_v4i)(st.tile + col * kTileCol + sub * 16);
            if (col < st.ncol) st_x<NT>(bw + col * st.ldb + r0 + ch * L + sub * V, v);
        }
        wave_lds_sync();
    }
}

// Rows [k0, k0 + 8) of the wave's columns of B (one 128-byte line per
// column, double complex: the only type with a second row panel) into the
// tile: the finished x of the first panel, read back by the reload
// segments. The lines go straight from memory into LDS (no registers):
// instruction q fetches the lines of columns 8q..8q+7 and lane 8a+b lands at
// byte 16(8a+b) of the instruction's 1 KB; the lane fetches row (a+b) mod 8
// of column 8q+b, so that reload_x's eight lanes of a group of columns
// read eight different 16-byte bank groups.
template <typename T, int P>
__device__ __forceinline__ void reload_fill(PanelState<T, P> &st, int k0)
{
    static_assert(sizeof(T) == 16, "one element per 16 bytes");
    const int lane = threadIdx.x & 63;
    const int a = lane >> 3, b = lane & 7;
    const int r = (a + b) & 7;
    const gptr<T> bw = global_after(st.Bw, st.x);
    // every earlier read of the tile has returned before the loads below
    // overwrite it
    wave_lds_sync();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        int col = q * 8 + b;
        col = col < st.ncol ? col : st.ncol - 1;  // duplicates of a valid column
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(bw + (col * st.ldb + k0 + r)),
                                         (__attribute__((address_space(3))) void *)(st.tile + q * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile has landed
    wave_lds_sync();
}

// x of row k0 + k (k < 8) of this lane's column from the tile reload_fill wrote.
template <typename T, int P>
__device__ __forceinline__ T reload_x(const PanelState<T, P> &st, int k)
{
    const int c = threadIdx.x & 63;
    const int q = c >> 3, b = c & 7;
    using R = typename traits<T>::real;
    const __attribute__((address_space(3))) R *e =
        (const __attribute__((address_space(3))) R *)(st.tile + q * 1024 + (8 * ((k - b) & 7) + b) * 16);
    return T{e[0], e[1]};
}

// Scalar loads of the pieces [Q, Q1) of a batch into cb.
template <typename T, int P, int R0, int G, int Q, int Q1>
__device__ __forceinline__ void batch_load(T (&cb)[G], cptr<T> ap, int64_t lda)
{
    if constexpr (Q < Q1) {
        using Plan = PanelPlan<P, R0, G, kDiagInStream<T>>;
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
        using Plan = PanelPlan<P, R0, G, kDiagInStream<T>>;
        constexpr auto pc = Plan::T.pc[Q];
        constexpr int off = Plan::T.off[Q];
        constexpr int wo = kRegOff<T, P, R0>;
        if constexpr (pc.first) {
            if constexpr (pc.reload && kKeep<T, P>) {
                // finished x_k of an earlier panel, still in its register
                st.x = st.w[pc.col];
            } else if constexpr (pc.reload) {
                // finished x_k of an earlier panel, read back from B through
                // the tile: one line of rows per refill for all the wave's
                // columns, then one LDS read per segment
                if constexpr (pc.col % 8 == 0) reload_fill<T, P>(st, pc.col);
                st.x = reload_x<T, P>(st, pc.col % 8);
            } else if constexpr (pc.diag) {
                constexpr int j = wo + pc.col - R0;
                if constexpr (std::is_same<T, float>::value) {
                    float r = __builtin_amdgcn_rcpf(cb[off]);
                    asm volatile("" : "+v"(r) : "v"(st.w[j]));
                    st.x = st.w[j] * r;
                } else if constexpr (std::is_same<T, double>::value) {
                    const double dv = cb[off];
                    double r = __builtin_amdgcn_rcp(dv);
                    asm volatile("" : "+v"(r) : "v"(st.w[j]));
                    double e = __builtin_fma(-dv, r, 1.0);
                    r = __builtin_fma(r, e, r);
                    e = __builtin_fma(-dv, r, 1.0);
                    r = __builtin_fma(r, e, r);
                    // IEEE special cases of 1/dv (zero, infinite or NaN pivot,
                    // overflowing reciprocal), which the Newton steps turn
                    // into NaN
                    r = __builtin_amdgcn_div_fixup(r, dv, 1.0);
                    st.x = st.w[j] * r;
                }
                st.w[j] = st.x;
            } else {
                constexpr int j = wo + pc.col - R0;
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
        for (int r = pc.lo + pc.diag; r < pc.hi; ++r)
            st.w[wo + r] = fms(st.w[wo + r], cb[off + r - pc.lo], st.x);
        batch_compute<T, P, R0, G, Q + 1, Q1>(st, cb);
    }
}

// L2 prefetch of segments [S, S1): lane l loads one dword of the l-th
// 128-byte line from the line holding the segment's first coefficient on;
// the buffer's range check (the records end at the segment's last byte)
// turns the lanes past the segment into no-ops.
template <typename T, int P, int R0, int G, int AH, int S, int S1>
__device__ __forceinline__ void batch_touch(PanelState<T, P> &st, cptr<T> ap)
{
    if constexpr (S < S1) {
        constexpr auto sg = TouchPlan<P, R0, G, AH, kDiagInStream<T>>::T.sg[S];
        const uint64_t first = (uint64_t)(ap + (R0 + sg.lo + (int64_t)sg.col * st.lda));
        const uint64_t line = first & ~(uint64_t)127;
        const int bytes = (int)(first - line) + (sg.hi - sg.lo) * (int)sizeof(T);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)line, (short)0, bytes, 0x00020000);
        if constexpr (kTouchLds<T, P>)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)st.sink, 4,
                                                     st.lane128, 0, 0, 0);
        else
            st.tv[S] = __builtin_amdgcn_raw_buffer_load_b32(rs, st.lane128, 0, 0);
        batch_touch<T, P, R0, G, AH, S + 1, S1>(st, ap);
    }
}

// Retire the prefetch loads of segments [S, S1) (waits for them if needed).
template <typename T, int P, int S, int S1>
__device__ __forceinline__ void batch_retire(PanelState<T, P> &st)
{
    if constexpr (S < S1) {
        asm volatile("" ::"v"(st.tv[S]));
        batch_retire<T, P, S + 1, S1>(st);
    }
}

// Batches [Bi, nbatch) of the panel at rows R0: prefetch ahead, fetch, one
// wait, update.
template <typename T, int P, int R0, int G, int AH, int Bi>
__device__ __forceinline__ void run_batches(PanelState<T, P> &st)
{
    using Plan = PanelPlan<P, R0, G, kDiagInStream<T>>;
    using TP = TouchPlan<P, R0, G, AH, kDiagInStream<T>>;
    if constexpr (Bi < Plan::T.nbatch) {
        constexpr int p0 = Plan::T.bfirst[Bi], p1 = Plan::T.bfirst[Bi + 1];
        // fetch this batch once the previous one has been consumed
        cptr<T> ap = st.a4;
        order_after(ap, st.x);
        batch_touch<T, P, R0, G, AH, TP::T.tfirst[Bi], TP::T.tfirst[Bi + 1]>(st, ap);
        T cb[G];
        batch_load<T, P, R0, G, p0, p1>(cb, ap, st.lda);
        if constexpr (!kTouchLds<T, P>) batch_retire<T, P, TP::T.cfirst[Bi], TP::T.cfirst[Bi + 1]>(st);
        batch_compute<T, P, R0, G, p0, p1>(st, cb);
        __builtin_amdgcn_sched_barrier(0);
        run_batches<T, P, R0, G, AH, Bi + 1>(st);
    }
}

template <typename T, int P, int NPANEL, int PI>
__device__ __forceinline__ void run_panels(PanelState<T, P> &st, T alpha, bool scale,
                                           typename traits<T>::real wlast)
{
    if constexpr (PI < NPANEL) {
        constexpr int r0 = PI * P;
        // a later panel's rows are loaded only after the earlier panel is done
        const gptr<T> bw = global_after(st.Bw, wlast);
        load_panel<T, P>(st, bw, r0, alpha, scale);
        st.x = zero_of(T());
        run_batches<T, P, r0, kBatch<T>, kAhead<T>, 0>(st);
        // the rows of an earlier panel are read back moments later: those
        // stores go through L2 normally (c128, 4096 problems: 205 -> 195 us)
        store_panel<T, P, (PI + 1 == NPANEL)>(st, bw, r0);
        typename traits<T>::real wl;
        if constexpr (traits<T>::is_complex) wl = st.w[P - 1].re; else wl = st.w[P - 1];
        run_panels<T, P, NPANEL, PI + 1>(st, alpha, scale, wl);
    }
}

// Kept-column panels: the loads of the rows [r0, r0 + P) of the wave's
// columns (one 128-byte line per column), 8 lanes per line.
template <typename T, int P>
__device__ __forceinline__ void panel_issue(const PanelState<T, P> &st, gptr<T> bw, int r0, v4i (&nb)[8])
{
    constexpr int V = 16 / (int)sizeof(T);
    static_assert(P * (int)sizeof(T) == 128, "a kept-column panel is one line per column");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        int col = q * 8 + (lane >> 3);
        col = col < st.ncol ? col : st.ncol - 1;  // duplicates of a valid column
        nb[q] = ld_b(bw + (col * st.ldb + r0 + (lane & 7) * V));
    }
}

// alpha * the loaded rows into registers [R0, R0 + P) of the column, lane =
// column, through the wave's tile.
template <typename T, int P, int R0>
__device__ __forceinline__ void panel_finish(PanelState<T, P> &st, const v4i (&nb)[8], T alpha, bool scale)
{
    constexpr int V = 16 / (int)sizeof(T);
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        *(lptr_v4i)(st.tile + (q * 8 + (lane >> 3)) * kTileCol + sub * 16) = nb[q];
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const v4i v = *(const lptr_v4i)(st.tile + lane * kTileCol + k * 16);
        T t[V];
        __builtin_memcpy(t, &v, 16);
#pragma unroll
        for (int e = 0; e < V; ++e) st.w[R0 + k * V + e] = t[e];
    }
    wave_lds_sync();
    if (scale) {
#pragma unroll
        for (int e = 0; e < P; ++e) st.w[R0 + e] = mul(alpha, st.w[R0 + e]);
    }
}

// Registers [R0, R0 + P) into rows [R0, R0 + P) of the wave's columns.
template <typename T, int P, int R0>
__device__ __forceinline__ void panel_store(PanelState<T, P> &st, gptr<T> bw)
{
    constexpr int V = 16 / (int)sizeof(T);
    const int lane = threadIdx.x & 63;
    const int sub = lane & 7;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        T t[V];
#pragma unroll
        for (int e = 0; e < V; ++e) t[e] = st.w[R0 + k * V + e];
        v4i v;
        __builtin_memcpy(&v, t, 16);
        *(lptr_v4i)(st.tile + lane * kTileCol + k * 16) = v;
    }
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int col = q * 8 + (lane >> 3);
        const v4i v = *(const lptr_v4i)(st.tile + col * kTileCol + sub * 16);
        if (col < st.ncol) st_x(bw + col * st.ldb + R0 + sub * V, v);
    }
    wave_lds_sync();
}

// Panel PI of a kept column: its B lines (nb) were requested during the
// previous panel; request the next panel's, solve this one, store its rows of
// X (the stores drain while the next panel is solved). The coefficient
// prefetch runs ahead of the stream as in the single-panel solve, into the
// LDS sink, so that nothing waits for it.
template <typename T, int P, int NPANEL, int PI>
__device__ __forceinline__ void run_panels_keep(PanelState<T, P> &st, const T *Ap, gptr<T> bw, T alpha,
                                                bool scale, v4i (&nb)[8])
{
    if constexpr (PI < NPANEL) {
        constexpr int r0 = PI * P;
        if constexpr (!kDiagInStream<T>) {
            // 1/a_ll for the panel's rows l (lane l mod P holds row l)
            const int l = r0 + ((threadIdx.x & 63) & (P - 1));
            st.myinv = recip(ld_global<T>((gptr<T>)(uint64_t)(Ap + (l + l * st.lda)), 0));
        }
        panel_finish<T, P, r0>(st, nb, alpha, scale);
        if constexpr (PI + 1 < NPANEL) panel_issue<T, P>(st, bw, r0 + P, nb);
        __builtin_amdgcn_sched_barrier(0);
        st.x = zero_of(T());
        run_batches<T, P, r0, kBatch<T>, kAhead<T>, 0>(st);
        // no prefetch may still be writing the LDS sink when the wave ends
        if constexpr (PI + 1 == NPANEL) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        panel_store<T, P, r0>(st, bw);
        run_panels_keep<T, P, NPANEL, PI + 1>(st, Ap, bw, alpha, scale, nb);
    }
}

template <typename T, int NPANEL>
__global__ void __launch_bounds__(256, sizeof(T) == 4 ? 4 : 2) colane_kernel(const T *__restrict__ A, int64_t lda,
                                                         int64_t strideA, T *__restrict__ B,
                                                         int64_t ldb, int64_t strideB, int64_t n,
                                                         int64_t nchunks, int64_t items, T alpha,
                                                         int scale, int64_t per, int64_t strideA2,
                                                         int64_t strideB2)
{
    extern __shared__ __attribute__((aligned(16))) char colane_lds[];
    __shared__ int colane_sink[64];
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

    // problem prob = g * per + k lives at A + g*strideA2 + k*strideA (B alike)
    const int64_t pg = prob / per, pk = prob % per;
    const T *Ap = A + pg * strideA2 + pk * strideA;
    // Lanes past n work on a copy of a valid column and never store, so
    // loads need no guard.
    T *Bc0 = B + pg * strideB2 + pk * strideB + cfirst * ldb;

    PanelState<T, P> st;
    st.a4 = (cptr<T>)Ap;
    st.lda = lda;
    st.Bw = Bc0;
    st.ldb = ldb;
    st.ncol = (int)(n - cfirst < 64 ? n - cfirst : 64);
    st.tile = (lptr)colane_lds + wave * kTileBytes;
    st.sink = (lptr)colane_sink;

    st.lane128 = lane * 128;
    if constexpr (kKeep<T, P>) {
        const gptr<T> bw = (gptr<T>)(uint64_t)Bc0;
        v4i nb[8];
        panel_issue<T, P>(st, bw, 0, nb);
        __builtin_amdgcn_sched_barrier(0);
        run_panels_keep<T, P, NPANEL, 0>(st, Ap, bw, alpha, scale != 0, nb);
    } else {
        if constexpr (!kDiagInStream<T>) st.myinv = recip(Ap[lane + lane * lda]);
        run_panels<T, P, NPANEL, 0>(st, alpha, scale != 0, typename traits<T>::real(0));
    }
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
    // all 256 VGPRs. Measured against re-reading the finished rows of 2/2/4
    // panels: f64 139 -> 114 us, c64 149 -> 136 us, c128 422 -> 291 us per
    // 4096 problems (re-read rows had been evicted from L2 and came back from
    // HBM). f64 and c64 solve the kept column in four one-line panels when a
    // launch has many problems per CU, so the next panel's B lines load while
    // a panel is solved, and in one panel otherwise; f32 loses with panels
    // (38.8 -> 43.8 us per 4096 problems). Per launch on MI355X, one panel
    // against four: f64 1024 problems 31.1 / 32.2 us, 2048: 41.0 / 42.8,
    // 2560: 63.2 / 61.8, 3072: 71.0 / 67.7, 4096: 85.8 / 82.6; c64 1024:
    // 44.7 / 46.7, 2048: 60.3 / 62.0, 3072: 91.2 / 93.4, 4096: 111.7 / 108.9.
    constexpr int NP = sizeof(T) == 16 ? 2 : 1;
    constexpr int64_t kPanelsFromPerCu = traits<T>::is_complex ? 16 : 10;
    const bool panels = sizeof(T) == 8 && items >= kPanelsFromPerCu * num_cus();
    // The 16-byte tile accesses need 16-byte aligned columns.
    if (((uintptr_t)B & 15) != 0 || ((ldb * (int64_t)sizeof(T)) & 15) != 0 ||
        ((strideB * (int64_t)sizeof(T)) & 15) != 0 || ((strideB2 * (int64_t)sizeof(T)) & 15) != 0)
        return hipErrorInvalidValue;
    // One tile per wave. Spread the workgroups evenly over the CUs: left
    // alone, the dispatcher may pack up to the occupancy limit onto fewer
    // CUs; reserving more LDS than the tiles need caps the workgroups per CU
    // at the even share.
    const int64_t per_cu = (blocks + num_cus() - 1) / num_cus();
    size_t lds = 4 * kTileBytes;
    if (per_cu >= 3 && per_cu < 8) {
        const size_t share = ((size_t)(160 * 1024) / (size_t)per_cu) & ~(size_t)1023;
        if (share > lds) lds = share;
    }
    if constexpr (sizeof(T) == 8) {
        if (panels) {
            hipLaunchKernelGGL((colane_kernel<T, 64 / kKeepRows<T>>), dim3((unsigned)blocks), dim3(256), lds, s,
                               A, lda, strideA, B, ldb, strideB, n, nchunks, items, alpha, is_one(alpha) ? 0 : 1,
                               per, strideA2, strideB2);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((colane_kernel<T, NP>), dim3((unsigned)blocks), dim3(256), lds, s, A, lda,
                       strideA, B, ldb, strideB, n, nchunks, items, alpha, is_one(alpha) ? 0 : 1, per, strideA2,
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
                                         hipStream_t, bool);                                       \
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
