// lad_solve.h -- truncated Newton-CG on the matrix-free Hessian-vector
// product: device state and launchers (defined in lad_solve.hip).  Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lad {

// Scalars of one Newton-CG solve, kept on the device so that no iteration
// needs the host.  Each scalar step of an iteration is computed by every
// workgroup of the kernel that needs it, from the same partial sums in the
// same order, so all take the same decision; workgroup 0 records it here.
// r.r after k updates sits in rrv[k & 1]: a kernel that records the new
// value reads the previous one from the other slot, so no workgroup reads a
// field that workgroup 0 of the same kernel writes.
struct CgState {
    double rrv[2];   // r.r after an even / odd number of updates
    double eps2;     // stop when r.r < eps2
    double alpha;    // step of the latest update
    double beta;     // direction update of the latest direction
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
// Update `iter` (0-based): its step from the partial sums of d.Bd
// (dy_parts[0 .. n_dy)) -- the negative-curvature exit or alpha -- then
// p += alpha d, r += alpha y, and the partial sums of the new r.r into
// rr_parts[0 .. grid).
template <typename T>
hipError_t launch_cg_update(T *p, T *r, const T *d, const T *y, int64_t n, const double *dy_parts,
                            int n_dy, double *rr_parts, int grid, CgState *st, int32_t iter,
                            hipStream_t s);
// Direction `iter` (>= 1) on the patch path: the step closing update
// iter - 1 from the partial sums of r.r (convergence, or beta), then
// d = -r + beta d.
template <typename T>
hipError_t launch_cg_dir(const T *r, T *d, int64_t n, int grid, const double *rr_parts,
                         int n_rr, CgState *st, int32_t iter, hipStream_t s);
// After the last update (`iters` in all): the step closing it, convergence
// or the iteration cap.  One workgroup; nothing once the solve has ended.
hipError_t launch_cg_close(const double *rr_parts, int n_rr, CgState *st, int32_t iters,
                           hipStream_t s);
// p = -g when the first direction already had non-positive curvature.
template <typename T>
hipError_t launch_cg_final(const T *g, T *p, int64_t n, int grid, const CgState *st,
                           hipStream_t s);

}  // namespace lad
