// strip_dual.h -- second-order forward-mode numbers that carry only the
// Hessian rows of one vertex.
//
// A StripDual<T, N> holds u, its gradient du/dz (N entries) and the three
// rows d2u / dz_r dz_k for r = 0, 1, 2 and every k: the row vertex's
// variables are seeded as z_0 .. z_2, the element's other vertices after
// them.  Evaluating a local term on such numbers gives, for the row that
// owns vertex z_0..z_2, its gradient part and its 3 x N strip of the local
// Hessian -- the row's blocks -- at 1 + 4N numbers per value instead of a
// full second-order number's 1 + N + N(N+1)/2 (37 against 55 for a
// three-vertex element).  Source: page "Locality-Aware Automatic
// Differentiation on the GPU for Mesh-Based Computations", section "Method"
// (element-level forward mode, local Hessians assembled through S_j) and key
// design 1 (every intermediate stays in registers).
//
// Rules, with a_r = da/dz_r (r < 3):
//   (a b)''[r][k] = a b''[r][k] + b a''[r][k] + a_r b_k + b_r a_k
//   f(a)''[r][k]  = f'(a) a''[r][k] + f''(a) a_r a_k
#pragma once

#include <hip/hip_runtime.h>

#include "dual2.h"  // lad_sqrt_rcp, lad_rcp, lad_log

namespace lad {

template <typename T, int N>
struct StripDual {
    static_assert(N >= 3, "the strip's vertex has three variables");
    T v;
    T g[N];
    T h[3][N];

    __device__ __forceinline__ static StripDual constant(T c)
    {
        StripDual r;
        r.v = c;
#pragma unroll
        for (int k = 0; k < N; ++k) r.g[k] = T(0);
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
            for (int k = 0; k < N; ++k) r.h[s][k] = T(0);
        return r;
    }
    // variable number `idx` (a runtime value) with value c
    __device__ __forceinline__ static StripDual var(T c, int idx)
    {
        StripDual r = constant(c);
#pragma unroll
        for (int k = 0; k < N; ++k) r.g[k] = k == idx ? T(1) : T(0);
        return r;
    }
};

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator+(const StripDual<T, N> &a,
                                                     const StripDual<T, N> &b)
{
    StripDual<T, N> r;
    r.v = a.v + b.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = a.g[k] + b.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = a.h[s][k] + b.h[s][k];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator-(const StripDual<T, N> &a,
                                                     const StripDual<T, N> &b)
{
    StripDual<T, N> r;
    r.v = a.v - b.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = a.g[k] - b.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = a.h[s][k] - b.h[s][k];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator-(const StripDual<T, N> &a)
{
    StripDual<T, N> r;
    r.v = -a.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = -a.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = -a.h[s][k];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator*(T c, const StripDual<T, N> &a)
{
    StripDual<T, N> r;
    r.v = c * a.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = c * a.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = c * a.h[s][k];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator*(const StripDual<T, N> &a, T c)
{
    return c * a;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator+(const StripDual<T, N> &a, T c)
{
    StripDual<T, N> r = a;
    r.v = a.v + c;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator+(T c, const StripDual<T, N> &a)
{
    return a + c;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator-(const StripDual<T, N> &a, T c)
{
    StripDual<T, N> r = a;
    r.v = a.v - c;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator-(T c, const StripDual<T, N> &a)
{
    StripDual<T, N> r = -a;
    r.v = c - a.v;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator*(const StripDual<T, N> &a,
                                                     const StripDual<T, N> &b)
{
    StripDual<T, N> r;
    r.v = a.v * b.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = a.v * b.g[k] + b.v * a.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k)
            r.h[s][k] = a.v * b.h[s][k] + b.v * a.h[s][k] + (a.g[s] * b.g[k] + b.g[s] * a.g[k]);
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> sqr(const StripDual<T, N> &a)
{
    StripDual<T, N> r;
    r.v = a.v * a.v;
    const T two_v = T(2) * a.v;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = two_v * a.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = two_v * a.h[s][k] + T(2) * (a.g[s] * a.g[k]);
    return r;
}

// f(a) from f(a.v), f'(a.v), f''(a.v)
template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> chain(const StripDual<T, N> &a, T f0, T f1, T f2)
{
    StripDual<T, N> r;
    r.v = f0;
#pragma unroll
    for (int k = 0; k < N; ++k) r.g[k] = f1 * a.g[k];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < N; ++k) r.h[s][k] = f1 * a.h[s][k] + f2 * (a.g[s] * a.g[k]);
    return r;
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> sqrt(const StripDual<T, N> &a)
{
    T s, inv;
    lad_sqrt_rcp(a.v, s, inv);
    return chain(a, s, T(0.5) * inv, T(-0.25) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> log(const StripDual<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, lad_log(a.v), inv, -inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> reciprocal(const StripDual<T, N> &a)
{
    const T inv = lad_rcp(a.v);
    return chain(a, inv, -inv * inv, T(2) * inv * inv * inv);
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator/(const StripDual<T, N> &a,
                                                     const StripDual<T, N> &b)
{
    return a * reciprocal(b);
}

template <typename T, int N>
__device__ __forceinline__ StripDual<T, N> operator/(const StripDual<T, N> &a, T c)
{
    return lad_rcp(c) * a;
}

}  // namespace lad
