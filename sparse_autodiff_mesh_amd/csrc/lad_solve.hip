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
// The scalars of the iteration live in a device-side CgState, so a whole
// solve is enqueued without the host reading anything.  Each scalar step is
// taken by every workgroup of the kernel that needs its result (the update
// takes the step giving alpha, the next direction's kernel the step giving
// beta), from the partial sums of the previous kernel in one fixed order:
// all workgroups take the same decision and no launch sits between the
// vector kernels.  Dot products are accumulated in fp64 per workgroup, so
// every run takes the same decisions and gives the same bits.  Vector
// updates are computed in fp64 and rounded to the working precision.
#include "cg_device.h"
#include "lad.h"
#include "lad_device.h"
#include "lad_solve.h"

namespace lad {

namespace {

constexpr int NT = kCgThreads;
constexpr int NS = 1024;            // threads of the single-workgroup kernels
// This workgroup's contiguous span [i0, i1) of n elements.
__device__ __forceinline__ void span(int64_t n, int64_t &i0, int64_t &i1)
{
    i0 = n * blockIdx.x / gridDim.x;
    i1 = n * (blockIdx.x + 1) / gridDim.x;
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
    __shared__ double dbc;
    const double gg = cg_sum<NS>(parts, nparts, red, &dbc);
    if (threadIdx.x != 0) return;
    const double gn = sqrt(gg);
    const double eps = eta > 0.0 ? eta * gn : fmin(0.5, sqrt(gn)) * gn;
    CgState s{};
    s.rrv[0] = gg;
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
    __shared__ int32_t sbc;
    if (cg_stop<NT>(st, &sbc)) return;
    int64_t i0, i1;
    span(n, i0, i1);
    double acc = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) acc += double(a[i]) * double(b[i]);
    const double s = block_sum<NT>(acc, red);
    if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

// Update `iter`: d.Bd from its partial sums (every workgroup, same order);
// non-positive curvature ends the solve (workgroup 0 records it), else
// alpha = r.r / d.Bd and the vectors move.
template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_update(T *__restrict__ p, T *__restrict__ r, const T *__restrict__ d,
            const T *__restrict__ y, int64_t n, const double *__restrict__ dy_parts, int n_dy,
            double *__restrict__ rr_parts, CgState *st, int32_t iter)
{
    __shared__ double red[NT / 64];
    __shared__ double dbc;
    __shared__ int32_t sbc;
    int64_t i0, i1;
    span(n, i0, i1);
    // the first element's operands are loaded before the step below, so
    // that their latency overlaps its sum
    const int64_t ib = i0 + threadIdx.x;
    T p0 = T(0), d0 = T(0), r0 = T(0), y0 = T(0);
    if (ib < i1) {
        p0 = p[ib];
        d0 = d[ib];
        r0 = r[ib];
        y0 = y[ib];
    }
    if (cg_stop<NT>(st, &sbc)) return;
    const double dBd = cg_sum<NT>(dy_parts, n_dy, red, &dbc);
    const bool writer = blockIdx.x == 0 && threadIdx.x == 0;
    if (!(dBd > 0.0)) {
        if (writer) {
            st->reason = LAD_CG_NEG_CURVATURE;
            st->stop = 1;
        }
        return;
    }
    const double al = st->rrv[iter & 1] / dBd;
    if (writer) st->alpha = al;
    double acc = 0.0;
    if (ib < i1) {
        p[ib] = T(double(p0) + al * double(d0));
        const T ri = T(double(r0) + al * double(y0));
        r[ib] = ri;
        acc += double(ri) * double(ri);
    }
    for (int64_t i = ib + NT; i < i1; i += NT) {
        p[i] = T(double(p[i]) + al * double(d[i]));
        const T ri = T(double(r[i]) + al * double(y[i]));
        r[i] = ri;
        acc += double(ri) * double(ri);
    }
    const double s = block_sum<NT>(acc, red);
    if (threadIdx.x == 0) rr_parts[blockIdx.x] = s;
}

// Direction `iter` >= 1 (patch path): the step closing update iter - 1,
// then d = -r + beta d.
template <typename T>
__global__ void __launch_bounds__(NT)
k_cg_dir(const T *__restrict__ r, T *__restrict__ d, int64_t n, const double *__restrict__ rr_parts,
         int n_rr, CgState *st, int32_t iter)
{
    __shared__ double red[NT / 64];
    __shared__ double dbc;
    __shared__ int32_t sbc;
    if (cg_stop<NT>(st, &sbc)) return;
    int32_t stop = 0;
    const double be = cg_beta_step<NT>(st, rr_parts, n_rr, iter, blockIdx.x == 0, stop, red, &dbc);
    if (stop) return;
    int64_t i0, i1;
    span(n, i0, i1);
    for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) d[i] = T(-double(r[i]) + be * double(d[i]));
}

// After the last update: the step closing it.  Convergence, else the cap.
__global__ void __launch_bounds__(NS) k_cg_close(const double *__restrict__ rr_parts, int n_rr,
                                                 CgState *st, int32_t iters)
{
    __shared__ double red[NS / 64];
    __shared__ double dbc;
    __shared__ int32_t sbc;
    if (cg_stop<NS>(st, &sbc)) return;
    const double rr = cg_sum<NS>(rr_parts, n_rr, red, &dbc);
    if (threadIdx.x != 0) return;
    st->rrv[iters & 1] = rr;
    st->iter = iters;
    st->reason = rr < st->eps2 ? LAD_CG_CONVERGED : LAD_CG_MAX_ITERS;
    st->stop = 1;
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

template <typename T>
hipError_t launch_cg_update(T *p, T *r, const T *d, const T *y, int64_t n, const double *dy_parts,
                            int n_dy, double *rr_parts, int grid, CgState *st, int32_t iter,
                            hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_update<T>, dim3(grid), dim3(NT), 0, s, p, r, d, y, n, dy_parts, n_dy,
                       rr_parts, st, iter);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_dir(const T *r, T *d, int64_t n, int grid, const double *rr_parts,
                         int n_rr, CgState *st, int32_t iter, hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_dir<T>, dim3(grid), dim3(NT), 0, s, r, d, n, rr_parts, n_rr, st, iter);
    return hipGetLastError();
}

hipError_t launch_cg_close(const double *rr_parts, int n_rr, CgState *st, int32_t iters,
                           hipStream_t s)
{
    hipLaunchKernelGGL(k_cg_close, dim3(1), dim3(NS), 0, s, rr_parts, n_rr, st, iters);
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
    template hipError_t launch_cg_update<T>(T *, T *, const T *, const T *, int64_t,              \
                                            const double *, int, double *, int, CgState *,        \
                                            int32_t, hipStream_t);                                \
    template hipError_t launch_cg_dir<T>(const T *, T *, int64_t, int, const double *, int,       \
                                         CgState *, int32_t, hipStream_t);                        \
    template hipError_t launch_cg_final<T>(const T *, T *, int64_t, int, const CgState *,         \
                                           hipStream_t);
LAD_SOLVE_INST(float)
LAD_SOLVE_INST(double)

}  // namespace lad
