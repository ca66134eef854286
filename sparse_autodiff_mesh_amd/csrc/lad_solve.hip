// lad_solve.hip -- truncated Newton-CG direction on the matrix-free HVP.
//
// Conjugate gradients on H p = -g from p = 0, stopped when |r| < eps or at
// the first direction of non-positive curvature (line-search Newton-CG,
// Nocedal and Wright, Numerical Optimization, 2nd ed., Algorithm 7.1), with
// an iteration cap.  The page "Locality-Aware Automatic Differentiation on
// the GPU for Mesh-Based Computations" motivates it (fast Hessian-vector
// products are what make Newton-type methods practical on large meshes) but
// fixes no solver.
//
// Every scalar of the iteration lives in a device-side CgState written by
// single-workgroup kernels, so a whole solve is enqueued without the host
// reading anything: vector kernels read alpha / beta from the state and
// return at once after the solve has ended.  Dot products are accumulated
// in fp64 per workgroup, and the partial sums are added in index order by
// one workgroup, so every run takes the same decisions and gives the same
// bits.  Vector updates are computed in fp64 and rounded to the working
// precision.
#include "lad.h"
#include "lad_device.h"
#include "lad_solve.h"

namespace lad {

namespace {

constexpr int NT = kCgThreads;
constexpr int NS = 1024;            // threads of the single-workgroup kernels
constexpr int kSumLoads = 4;        // partial sums each of their threads loads at once

// This workgroup's contiguous span [i0, i1) of n elements.
__device__ __forceinline__ void span(int64_t n, int64_t &i0, int64_t &i1)
{
    i0 = n * blockIdx.x / gridDim.x;
    i1 = n * (blockIdx.x + 1) / gridDim.x;
}

// Sum of parts[0 .. n) in a fixed order, by one workgroup of NS threads:
// thread t adds parts[t], parts[t + NS], ... in that order, then the
// workgroup reduction adds the threads' sums; valid in thread 0.  The
// partial sums were just written by other XCDs, so every load misses this
// XCD's L2: each thread issues kSumLoads of them before adding any, which
// pays that latency once per group instead of once per value.
__device__ __forceinline__ double sum_parts(const double *__restrict__ parts, int n, double *red)
{
    double s = 0.0;
    for (int i0 = 0; i0 < n; i0 += NS * kSumLoads) {
        double v[kSumLoads];
#pragma unroll
        for (int k = 0; k < kSumLoads; ++k) {
            const int i = i0 + k * NS + int(threadIdx.x);
            v[k] = i < n ? parts[i] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kSumLoads; ++k) s += v[k];
    }
    return block_sum<NS>(s, red);
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_init(const T *__restrict__ g, T *__restrict__ p, T *__restrict__ r, T *__restrict__ d,
          int64_t n, double *__restrict__ parts)
{
    __shared__ double red[NT / 64];
    int64_t i0, i1;
    span(n, i0, i1);
    double acc = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) {
        const T gi = g[i];
        r[i] = gi;
        d[i] = -gi;
        p[i] = T(0);
        acc += double(gi) * double(gi);
    }
    const double s = block_sum<NT>(acc, red);
    if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

__global__ void __launch_bounds__(NS)
k_cg_start(const double *__restrict__ parts, int nparts, CgState *st, double eta,
           int32_t max_iters)
{
    __shared__ double red[NS / 64];
    const double gg = sum_parts(parts, nparts, red);
    if (threadIdx.x != 0) return;
    const double gn = sqrt(gg);
    const double eps = eta > 0.0 ? eta * gn : fmin(0.5, sqrt(gn)) * gn;
    CgState s{};
    s.rr = gg;
    s.eps2 = eps * eps;
    s.gnorm = gn;
    s.iter = 0;
    if (gg <= s.eps2) {
        s.stop = 1;
        s.reason = LAD_CG_CONVERGED;
    } else if (max_iters <= 0) {
        s.stop = 1;
        s.reason = LAD_CG_MAX_ITERS;
    }
    *st = s;
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_dot(const T *__restrict__ a, const T *__restrict__ b, int64_t n, double *__restrict__ parts,
         const CgState *st)
{
    __shared__ double red[NT / 64];
    if (st->stop) return;
    int64_t i0, i1;
    span(n, i0, i1);
    double acc = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) acc += double(a[i]) * double(b[i]);
    const double s = block_sum<NT>(acc, red);
    if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

__global__ void __launch_bounds__(NS) k_cg_alpha(const double *__restrict__ parts, int nparts,
                                                 CgState *st)
{
    __shared__ double red[NS / 64];
    // the stop flag is loaded alongside the partial sums, not before them
    const int32_t stop = st->stop;
    const double dBd = sum_parts(parts, nparts, red);
    if (stop || threadIdx.x != 0) return;
    if (!(dBd > 0.0)) {
        st->stop = 1;
        st->reason = LAD_CG_NEG_CURVATURE;
    } else {
        st->alpha = st->rr / dBd;
    }
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_update(T *__restrict__ p, T *__restrict__ r, const T *__restrict__ d,
            const T *__restrict__ y, int64_t n, double *__restrict__ parts, const CgState *st)
{
    __shared__ double red[NT / 64];
    if (st->stop) return;
    const double al = st->alpha;
    int64_t i0, i1;
    span(n, i0, i1);
    double acc = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) {
        p[i] = T(double(p[i]) + al * double(d[i]));
        const T ri = T(double(r[i]) + al * double(y[i]));
        r[i] = ri;
        acc += double(ri) * double(ri);
    }
    const double s = block_sum<NT>(acc, red);
    if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

__global__ void __launch_bounds__(NS) k_cg_beta(const double *__restrict__ parts, int nparts,
                                                CgState *st, int32_t max_iters)
{
    __shared__ double red[NS / 64];
    const int32_t stop = st->stop;
    const double rr = sum_parts(parts, nparts, red);
    if (stop || threadIdx.x != 0) return;
    const int32_t it = st->iter + 1;
    st->iter = it;
    if (rr < st->eps2) {
        st->stop = 1;
        st->reason = LAD_CG_CONVERGED;
    } else if (it >= max_iters) {
        st->stop = 1;
        st->reason = LAD_CG_MAX_ITERS;
    } else {
        st->beta = rr / st->rr;
    }
    st->rr = rr;
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_dir(const T *__restrict__ r, T *__restrict__ d, int64_t n, const CgState *st)
{
    if (st->stop) return;
    const double be = st->beta;
    int64_t i0, i1;
    span(n, i0, i1);
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) d[i] = T(-double(r[i]) + be * double(d[i]));
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_final(const T *__restrict__ g, T *__restrict__ p, int64_t n, const CgState *st)
{
    if (!(st->reason == LAD_CG_NEG_CURVATURE && st->iter == 0)) return;
    int64_t i0, i1;
    span(n, i0, i1);
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) p[i] = -g[i];
}

}  // namespace

int cg_vec_grid(int64_t n)
{
    const int64_t g = (n + 4 * NT - 1) / (4 * NT);  // at least 4 elements per thread
    return int(g < 1 ? 1 : (g > kCgMaxGrid ? kCgMaxGrid : g));
}

template <typename T>
hipError_t launch_cg_init(const T *g, T *p, T *r, T *d, int64_t n, double *parts, int grid,
                          hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_init<T>, dim3(grid), dim3(NT), 0, s, g, p, r, d, n, parts);
    return hipGetLastError();
}

hipError_t launch_cg_start(const double *parts, int nparts, CgState *st, double eta,
                           int32_t max_iters, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_start, dim3(1), dim3(NS), 0, s, parts, nparts, st, eta, max_iters);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_dot(const T *a, const T *b, int64_t n, double *parts, int grid,
                         const CgState *st, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_dot<T>, dim3(grid), dim3(NT), 0, s, a, b, n, parts, st);
    return hipGetLastError();
}

hipError_t launch_cg_alpha(const double *parts, int nparts, CgState *st, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_alpha, dim3(1), dim3(NS), 0, s, parts, nparts, st);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_update(T *p, T *r, const T *d, const T *y, int64_t n, double *parts,
                            int grid, const CgState *st, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_update<T>, dim3(grid), dim3(NT), 0, s, p, r, d, y, n, parts, st);
    return hipGetLastError();
}

hipError_t launch_cg_beta(const double *parts, int nparts, CgState *st, int32_t max_iters,
                          hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_beta, dim3(1), dim3(NS), 0, s, parts, nparts, st, max_iters);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_dir(const T *r, T *d, int64_t n, int grid, const CgState *st,
                         hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_dir<T>, dim3(grid), dim3(NT), 0, s, r, d, n, st);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_final(const T *g, T *p, int64_t n, int grid, const CgState *st,
                           hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_final<T>, dim3(grid), dim3(NT), 0, s, g, p, n, st);
    return hipGetLastError();
}

#define LAD_SOLVE_INST(T)                                                                         \
    template hipError_t launch_cg_init<T>(const T *, T *, T *, T *, int64_t, double *, int,       \
                                          hipStream_t);                                           \
    template hipError_t launch_cg_dot<T>(const T *, const T *, int64_t, double *, int,            \
                                         const CgState *, hipStream_t);                           \
    template hipError_t launch_cg_update<T>(T *, T *, const T *, const T *, int64_t, double *,    \
                                            int, const CgState *, hipStream_t);                   \
    template hipError_t launch_cg_dir<T>(const T *, T *, int64_t, int, const CgState *,           \
                                         hipStream_t);                                            \
    template hipError_t launch_cg_final<T>(const T *, T *, int64_t, int, const CgState *,         \
                                           hipStream_t);
LAD_SOLVE_INST(float)
LAD_SOLVE_INST(double)

}  // namespace lad
