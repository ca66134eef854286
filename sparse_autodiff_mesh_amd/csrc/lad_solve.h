// lad_solve.h -- truncated Newton-CG on the matrix-free Hessian-vector
// product: device state and launchers (defined in lad_solve.hip).  Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lad {

// Scalars of one Newton-CG solve, kept on the device so that no iteration
// needs the host: written only by the single-workgroup kernels
// (launch_cg_start / _alpha / _beta), read by the rest.
struct CgState {
    double rr;       // r.r of the current residual
    double eps2;     // stop when r.r < eps2
    double alpha;    // step of the current iteration
    double beta;     // direction update of the current iteration
    double gnorm;    // |g|
    int32_t iter;    // completed CG updates
    int32_t stop;    // nonzero once the solve has ended
    int32_t reason;  // LAD_CG_* code, valid once stop != 0
    int32_t pad;
};

constexpr int kCgThreads = 256;   // threads of every solver kernel
constexpr int kCgMaxGrid = 1024;  // workgroups (and partial sums) of the vector kernels

// Workgroups of the vector kernels for n elements (1..kCgMaxGrid).
int cg_vec_grid(int64_t n);

// r = g, d = -g, p = 0; partial sums of g.g into parts[0 .. grid).
template <typename T>
hipError_t launch_cg_init(const T *g, T *p, T *r, T *d, int64_t n, double *parts, int grid,
                          hipStream_t s);
// |g|, the threshold and the initial state from the partial sums of g.g.
hipError_t launch_cg_start(const double *parts, int nparts, CgState *st, double eta,
                           int32_t max_iters, hipStream_t s);
// Partial sums of a.b (skipped once the solve has ended).
template <typename T>
hipError_t launch_cg_dot(const T *a, const T *b, int64_t n, double *parts, int grid,
                         const CgState *st, hipStream_t s);
// d.Bd from its partial sums: negative-curvature exit or the step alpha.
hipError_t launch_cg_alpha(const double *parts, int nparts, CgState *st, hipStream_t s);
// p += alpha d, r += alpha y; partial sums of the new r.r.
template <typename T>
hipError_t launch_cg_update(T *p, T *r, const T *d, const T *y, int64_t n, double *parts,
                            int grid, const CgState *st, hipStream_t s);
// New r.r from its partial sums: convergence, the iteration cap, or beta.
hipError_t launch_cg_beta(const double *parts, int nparts, CgState *st, int32_t max_iters,
                          hipStream_t s);
// d = -r + beta d.
template <typename T>
hipError_t launch_cg_dir(const T *r, T *d, int64_t n, int grid, const CgState *st,
                         hipStream_t s);
// p = -g when the first direction already had non-positive curvature.
template <typename T>
hipError_t launch_cg_final(const T *g, T *p, int64_t n, int grid, const CgState *st,
                           hipStream_t s);

}  // namespace lad
