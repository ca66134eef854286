// dual2.h -- second-order forward-mode dual numbers held in registers.
//
// A Dual2<T, N> carries a scalar u together with its gradient du/dz (N
// entries) and its Hessian d2u/dz2 (N(N+1)/2 packed upper-triangle entries)
// with respect to N seeded variables z.  Every operation propagates all three
// by the chain rule, so evaluating a local energy on seeded inputs yields its
// value, dense local gradient and dense local Hessian in one forward pass,
// with no tape and no memory traffic.  Source: page "Locality-Aware Automatic
// Differentiation on the GPU for Mesh-Based Computations", key design 1
// (element-level forward mode; primal, directional derivatives and local
// Hessians stay in registers or shared memory).
//
// Everything is fully unrolled at compile time; N is small (3 for two-vertex
// radial terms, 6 for faces, 9 for a face seeded in world coordinates).
#pragma once

#include <hip/hip_runtime.h>

namespace lad {

template <int N>
struct Tri {
    static constexpr int size = N * (N + 1) / 2;
    // packed index of (i, j), i <= j, row-major upper triangle
    __host__ __device__ static constexpr int idx(int i, int j)
    {
        return i * N - (i * (i - 1)) / 2 + (j - i);
    }
};

// Fused multiply-add; the rules below are written as chains of them, one
// rounding per product term.
__device__ __forceinline__ float lad_fma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double lad_fma(double a, double b, double c) { return __builtin_fma(a, b, c); }

template <typename T, int N>
struct Dual2 {
    static constexpr int NH = Tri<N>::size;
    T v;
    T g[N];
    T h[NH];

    __device__ __forceinline__ static Dual2 constant(T c)
    {
        Dual2 r;
        r.v = c;
#pragma unroll
        for (int i = 0; i < N; ++i) r.g[i] = T(0);
#pragma unroll
        for (int i = 0; i < NH; ++i) r.h[i] = T(0);
        return r;
    }
    // the k-th seeded variable with value c
    __device__ __forceinline__ static Dual2 var(T c, int k)
    {
        Dual2 r = constant(c);
#pragma unroll
        for (int i = 0; i < N; ++i) r.g[i] = (i == k) ? T(1) : T(0);
        return r;
    }
    __device__ __forceinline__ T hess(int i, int j) const
    {
        return i <= j ? h[Tri<N>::idx(i, j)] : h[Tri<N>::idx(j, i)];
    }
};

// ---- linear operations --------------------------------------------------
template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator+(const Dual2<T, N> &a, const Dual2<T, N> &b)
{
    Dual2<T, N> r;
    r.v = a.v + b.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = a.g[i] + b.g[i];
#pragma unroll
    for (int i = 0; i < Dual2<T, N>::NH; ++i) r.h[i] = a.h[i] + b.h[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator-(const Dual2<T, N> &a, const Dual2<T, N> &b)
{
    Dual2<T, N> r;
    r.v = a.v - b.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = a.g[i] - b.g[i];
#pragma unroll
    for (int i = 0; i < Dual2<T, N>::NH; ++i) r.h[i] = a.h[i] - b.h[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator-(const Dual2<T, N> &a)
{
    Dual2<T, N> r;
    r.v = -a.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = -a.g[i];
#pragma unroll
    for (int i = 0; i < Dual2<T, N>::NH; ++i) r.h[i] = -a.h[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator*(T s, const Dual2<T, N> &a)
{
    Dual2<T, N> r;
    r.v = s * a.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = s * a.g[i];
#pragma unroll
    for (int i = 0; i < Dual2<T, N>::NH; ++i) r.h[i] = s * a.h[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator+(const Dual2<T, N> &a, T s)
{
    Dual2<T, N> r = a;
    r.v = a.v + s;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator-(const Dual2<T, N> &a, T s)
{
    Dual2<T, N> r = a;
    r.v = a.v - s;
    return r;
}

// ---- product rule ---------------------------------------------------------
// (ab)'  = a'b + ab'
// (ab)'' = a''b + ab'' + a' b'^T + b' a'^T
template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator*(const Dual2<T, N> &a, const Dual2<T, N> &b)
{
    Dual2<T, N> r;
    r.v = a.v * b.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = lad_fma(a.v, b.g[i], b.v * a.g[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = i; j < N; ++j) {
            const int k = Tri<N>::idx(i, j);
            r.h[k] = lad_fma(a.g[i], b.g[j],
                             lad_fma(a.g[j], b.g[i], lad_fma(a.v, b.h[k], b.v * a.h[k])));
        }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> sqr(const Dual2<T, N> &a)
{
    Dual2<T, N> r;
    r.v = a.v * a.v;
    const T two_v = T(2) * a.v;
    T two_g[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = two_v * a.g[i];
        two_g[i] = T(2) * a.g[i];
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = i; j < N; ++j) {
            const int k = Tri<N>::idx(i, j);
            r.h[k] = lad_fma(two_g[i], a.g[j], two_v * a.h[k]);
        }
    return r;
}

// ---- scalar functions: f(a)' = f1 a',  f(a)'' = f1 a'' + f2 a' a'^T ------
template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> chain(const Dual2<T, N> &a, T f0, T f1, T f2)
{
    Dual2<T, N> r;
    r.v = f0;
    T f2g[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = f1 * a.g[i];
        f2g[i] = f2 * a.g[i];
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = i; j < N; ++j) {
            const int k = Tri<N>::idx(i, j);
            r.h[k] = lad_fma(f2g[i], a.g[j], f1 * a.h[k]);
        }
    return r;
}

// Reciprocal, and square root with its reciprocal, of a positive normal
// value.  fp32 takes the hardware reciprocal and reciprocal square root
// (v_rcp_f32, v_rsq_f32: each within 1 ulp), two instructions where a
// correctly rounded square root and division take about thirty; the fp32
// outputs are held to 2e-5 relative error against the fp64 definition,
// some hundred ulp.  fp64 keeps correctly rounded operations.
__device__ __forceinline__ float lad_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ double lad_rcp(double x) { return 1.0 / x; }
__device__ __forceinline__ void lad_sqrt_rcp(float x, float &s, float &inv)
{
    inv = __builtin_amdgcn_rsqf(x);
    s = x * inv;
}
__device__ __forceinline__ void lad_sqrt_rcp(double x, double &s, double &inv)
{
    s = __builtin_sqrt(x);
    inv = 1.0 / s;
}
__device__ __forceinline__ float lad_log(float x) { return ::logf(x); }
__device__ __forceinline__ double lad_log(double x) { return ::log(x); }

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> sqrt(const Dual2<T, N> &a)
{
    T s, inv;
    lad_sqrt_rcp(a.v, s, inv);
    return chain(a, s, T(0.5) * inv, T(-0.25) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> log(const Dual2<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, lad_log(a.v), inv, -inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> reciprocal(const Dual2<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, inv, -inv * inv, T(2) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ Dual2<T, N> operator/(const Dual2<T, N> &a, const Dual2<T, N> &b)
{
    return a * reciprocal(b);
}

// ---------------------------------------------------------------------------
// Directional second-order duals for Hessian-vector products.
//
// A DualHv<T, N> carries u, its gradient du/dz (N entries), its derivative
// along one fixed direction p (t = du/dz . p) and the derivative of the
// gradient along p (gt = d2u/dz2 p, N entries).  Seeding the variables with
// z_k = var(value, k, p_k) and evaluating a local energy once gives its
// gradient and the product of its Hessian with p, without forming the
// Hessian: 2 + 2N numbers per intermediate instead of the 1 + N + N(N+1)/2
// of Dual2 (14 instead of 28 for a face seeded in its 6 deformation-gradient
// entries).  The product and chain rules below are those of Dual2 contracted
// with p.
// ---------------------------------------------------------------------------
template <typename T, int N>
struct DualHv {
    T v, t;
    T g[N];
    T gt[N];

    __device__ __forceinline__ static DualHv constant(T c)
    {
        DualHv r;
        r.v = c;
        r.t = T(0);
#pragma unroll
        for (int i = 0; i < N; ++i) r.g[i] = r.gt[i] = T(0);
        return r;
    }
    // the k-th seeded variable with value c and direction component pk
    __device__ __forceinline__ static DualHv var(T c, int k, T pk)
    {
        DualHv r = constant(c);
        r.t = pk;
#pragma unroll
        for (int i = 0; i < N; ++i) r.g[i] = (i == k) ? T(1) : T(0);
        return r;
    }
};

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator+(const DualHv<T, N> &a, const DualHv<T, N> &b)
{
    DualHv<T, N> r;
    r.v = a.v + b.v;
    r.t = a.t + b.t;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = a.g[i] + b.g[i];
        r.gt[i] = a.gt[i] + b.gt[i];
    }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator-(const DualHv<T, N> &a, const DualHv<T, N> &b)
{
    DualHv<T, N> r;
    r.v = a.v - b.v;
    r.t = a.t - b.t;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = a.g[i] - b.g[i];
        r.gt[i] = a.gt[i] - b.gt[i];
    }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator*(T s, const DualHv<T, N> &a)
{
    DualHv<T, N> r;
    r.v = s * a.v;
    r.t = s * a.t;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = s * a.g[i];
        r.gt[i] = s * a.gt[i];
    }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator+(const DualHv<T, N> &a, T s)
{
    DualHv<T, N> r = a;
    r.v = a.v + s;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator-(const DualHv<T, N> &a, T s)
{
    DualHv<T, N> r = a;
    r.v = a.v - s;
    return r;
}

// (ab)' = a'b + ab';  (ab)'' p = a'' p b + a b'' p + a' (b' . p) + b' (a' . p)
template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator*(const DualHv<T, N> &a, const DualHv<T, N> &b)
{
    DualHv<T, N> r;
    r.v = a.v * b.v;
    r.t = lad_fma(a.v, b.t, b.v * a.t);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = lad_fma(a.v, b.g[i], b.v * a.g[i]);
        r.gt[i] = lad_fma(a.g[i], b.t,
                          lad_fma(b.g[i], a.t, lad_fma(a.v, b.gt[i], b.v * a.gt[i])));
    }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> sqr(const DualHv<T, N> &a)
{
    DualHv<T, N> r;
    const T two_v = T(2) * a.v;
    r.v = a.v * a.v;
    r.t = two_v * a.t;
    const T two_t = T(2) * a.t;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = two_v * a.g[i];
        r.gt[i] = lad_fma(two_t, a.g[i], two_v * a.gt[i]);
    }
    return r;
}

// f(a)' = f1 a';  f(a)'' p = f1 a'' p + f2 a' (a' . p)
template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> chain(const DualHv<T, N> &a, T f0, T f1, T f2)
{
    DualHv<T, N> r;
    r.v = f0;
    r.t = f1 * a.t;
    const T f2t = f2 * a.t;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.g[i] = f1 * a.g[i];
        r.gt[i] = lad_fma(f2t, a.g[i], f1 * a.gt[i]);
    }
    return r;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> sqrt(const DualHv<T, N> &a)
{
    T s, inv;
    lad_sqrt_rcp(a.v, s, inv);
    return chain(a, s, T(0.5) * inv, T(-0.25) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> log(const DualHv<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, lad_log(a.v), inv, -inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> reciprocal(const DualHv<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, inv, -inv * inv, T(2) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator/(const DualHv<T, N> &a, const DualHv<T, N> &b)
{
    return a * reciprocal(b);
}

// Mixed and unary forms, for generic term code written once for every
// number type.
template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator-(const DualHv<T, N> &a)
{
    return T(-1) * a;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator*(const DualHv<T, N> &a, T s)
{
    return s * a;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator+(T s, const DualHv<T, N> &a)
{
    return a + s;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator-(T s, const DualHv<T, N> &a)
{
    return (T(-1) * a) + s;
}

template <typename T, int N>
__device__ __forceinline__ DualHv<T, N> operator/(const DualHv<T, N> &a, T s)
{
    return lad_rcp(s) * a;
}

}  // namespace lad
