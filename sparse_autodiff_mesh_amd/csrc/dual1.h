// dual1.h -- first-order forward-mode dual numbers held in registers.
//
// A Dual1<T, N> carries a scalar u and its gradient du/dz with respect to N
// seeded variables.  Evaluating a local residual on seeded inputs yields its
// value and its dense local Jacobian row in one forward pass.  Source: page
// "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", section "Method" (vector objectives: local Jacobians J_j)
// and key design 1 (element-level forward mode in registers).
#pragma once

#include <hip/hip_runtime.h>

#include "dual2.h"  // lad_sqrt_rcp

namespace lad {

template <typename T, int N>
struct Dual1 {
    T v;
    T g[N];

    __device__ __forceinline__ static Dual1 constant(T c)
    {
        Dual1 r;
        r.v = c;
#pragma unroll
        for (int i = 0; i < N; ++i) r.g[i] = T(0);
        return r;
    }
    // the k-th seeded variable with value c
    __device__ __forceinline__ static Dual1 var(T c, int k)
    {
        Dual1 r = constant(c);
        r.g[k] = T(1);
        return r;
    }
};

template <typename T, int N>
__device__ __forceinline__ Dual1<T, N> operator+(const Dual1<T, N> &a, const Dual1<T, N> &b)
{
    Dual1<T, N> r;
    r.v = a.v + b.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = a.g[i] + b.g[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual1<T, N> operator-(const Dual1<T, N> &a, T s)
{
    Dual1<T, N> r = a;
    r.v = a.v - s;
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual1<T, N> operator*(T s, const Dual1<T, N> &a)
{
    Dual1<T, N> r;
    r.v = s * a.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = s * a.g[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual1<T, N> sqr(const Dual1<T, N> &a)
{
    Dual1<T, N> r;
    r.v = a.v * a.v;
    const T t = T(2) * a.v;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = t * a.g[i];
    return r;
}

template <typename T, int N>
__device__ __forceinline__ Dual1<T, N> sqrt(const Dual1<T, N> &a)
{
    Dual1<T, N> r;
    T inv;
    lad_sqrt_rcp(a.v, r.v, inv);
    const T d = T(0.5) * inv;
#pragma unroll
    for (int i = 0; i < N; ++i) r.g[i] = d * a.g[i];
    return r;
}

}  // namespace lad
