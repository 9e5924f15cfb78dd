// common.hpp - element types and arithmetic shared by the library's kernels.
//
// Four element types: float, double and the two complex types, each complex
// value stored as an interleaved (re, im) pair exactly like
// hsma_float_complex / hsma_double_complex in the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hsma {

template <typename R>
struct cplx {
    R re, im;
};

using c32 = cplx<float>;
using c64 = cplx<double>;

template <typename T> struct traits;
template <> struct traits<float> {
    using real = float;
    static constexpr bool is_complex = false;
    static constexpr int dtype = 0;
};
template <> struct traits<double> {
    using real = double;
    static constexpr bool is_complex = false;
    static constexpr int dtype = 1;
};
template <> struct traits<c32> {
    using real = float;
    static constexpr bool is_complex = true;
    static constexpr int dtype = 2;
};
template <> struct traits<c64> {
    using real = double;
    static constexpr bool is_complex = true;
    static constexpr int dtype = 3;
};

// ---- scalar arithmetic, written once for real and complex ------------------

__host__ __device__ inline float zero_of(float) { return 0.f; }
__host__ __device__ inline double zero_of(double) { return 0.0; }
__host__ __device__ inline c32 zero_of(c32) { return {0.f, 0.f}; }
__host__ __device__ inline c64 zero_of(c64) { return {0.0, 0.0}; }

__host__ __device__ inline bool is_zero(float a) { return a == 0.f; }
__host__ __device__ inline bool is_zero(double a) { return a == 0.0; }
__host__ __device__ inline bool is_zero(c32 a) { return a.re == 0.f && a.im == 0.f; }
__host__ __device__ inline bool is_zero(c64 a) { return a.re == 0.0 && a.im == 0.0; }

__host__ __device__ inline bool is_one(float a) { return a == 1.f; }
__host__ __device__ inline bool is_one(double a) { return a == 1.0; }
__host__ __device__ inline bool is_one(c32 a) { return a.re == 1.f && a.im == 0.f; }
__host__ __device__ inline bool is_one(c64 a) { return a.re == 1.0 && a.im == 0.0; }

__device__ inline float fmaR(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ inline double fmaR(double a, double b, double c) { return __builtin_fma(a, b, c); }

__device__ inline float mul(float a, float b) { return a * b; }
__device__ inline double mul(double a, double b) { return a * b; }
template <typename R>
__device__ inline cplx<R> mul(cplx<R> a, cplx<R> b)
{
    return {fmaR(a.re, b.re, -a.im * b.im), fmaR(a.re, b.im, a.im * b.re)};
}

// w - a*x, as fused multiply-adds.
__device__ inline float fms(float w, float a, float x) { return __builtin_fmaf(-a, x, w); }
__device__ inline double fms(double w, double a, double x) { return __builtin_fma(-a, x, w); }
template <typename R>
__device__ inline cplx<R> fms(cplx<R> w, cplx<R> a, cplx<R> x)
{
    cplx<R> r;
    r.re = fmaR(-a.re, x.re, w.re);
    r.re = fmaR(a.im, x.im, r.re);
    r.im = fmaR(-a.re, x.im, w.im);
    r.im = fmaR(-a.im, x.re, r.im);
    return r;
}

// 1/d with IEEE division. Complex d by Smith's method: with p the part of
// larger magnitude and q the other, r = q/p and t = 1/(p + q r); then
// 1/d = (t, -r t) when p = re, (r t, -t) when p = im. Nothing is squared,
// so no intermediate over- or underflows where 1/d is representable (the
// plain conj(d)/|d|^2 loses half of the exponent range). d = 0 gives NaN.
__device__ inline float recip(float d) { return 1.0f / d; }
__device__ inline double recip(double d) { return 1.0 / d; }
template <typename R>
__device__ inline cplx<R> recip(cplx<R> d)
{
    const bool sw = __builtin_fabs(d.im) > __builtin_fabs(d.re);
    const R p = sw ? d.im : d.re, q = sw ? d.re : d.im;
    const R r = q / p;
    const R t = R(1) / fmaR(q, r, p);
    const R u = r * t;
    return {sw ? u : t, sw ? -t : -u};
}

// c ? a : b on values, component by component for complex types. A
// conditional expression whose operands are complex lvalues selects between
// their addresses, which can keep a register array in scratch memory.
__device__ inline float pick(bool c, float a, float b) { return c ? a : b; }
__device__ inline double pick(bool c, double a, double b) { return c ? a : b; }
template <typename R>
__device__ inline cplx<R> pick(bool c, cplx<R> a, cplx<R> b)
{
    return {c ? a.re : b.re, c ? a.im : b.im};
}

// ---- cross-lane broadcast of a wave-uniform lane index (v_readlane) --------

__device__ inline float readlane(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ inline double readlane(double v, int lane)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffff), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
template <typename R>
__device__ inline cplx<R> readlane(cplx<R> v, int lane)
{
    return {readlane(v.re, lane), readlane(v.im, lane)};
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E), so
// that register-array indices inside f are constants after inlining.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace hsma
