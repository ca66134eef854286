// lad_jacobian.h -- vector objective (spring and inertia residuals): sparse
// Jacobian pattern and values, and the matrix-free Gauss-Newton product.
// Launchers defined in lad_jacobian.hip and lad_rows.hip.  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lad_internal.h"

namespace lad {

// Jacobian rows: ns spring rows, then (inertia on) 3 nv inertia rows.
// Spring row s holds 6 entries at 6s (the DOFs of its two vertices,
// ascending); inertia row ns + i holds one entry at 6 ns + i (DOF i).
hipError_t launch_jacobian_pattern(int32_t ns, const int32_t *springs, int64_t inertia_rows,
                                   int32_t *row_ptr, int32_t *col_idx, hipStream_t s);

// R and the Jacobian values in the pattern's order.
template <typename T>
hipError_t launch_residual_jacobian(int32_t ns, const int32_t *springs, const T *rest, T sqrt_k,
                                    int64_t inertia_rows, const T *x, const T *x_tilde, T sqrt_c,
                                    T *r, T *jvals, hipStream_t s);

// y = J^T (J v), row owner on the topology pattern (row path only).
template <typename T>
hipError_t launch_gauss_newton_rows(const RowArgs<T> &a, T sqrt_k, T sqrt_c, const T *x,
                                    const T *v, T *y, int grid, hipStream_t s);

}  // namespace lad
