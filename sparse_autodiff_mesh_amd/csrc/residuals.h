// residuals.h -- local residuals of the vector objective, templated on the
// number type (Dual1 in the kernels).
//
// The vector objective is the least-squares form of the spring and inertia
// terms: 0.5 |R|^2 equals their energy, with
//   spring s = (a, b):  R_s = sqrt(k) (|x_a - x_b| - L_s)
//   vertex v, coord c:  R   = sqrt(c) (x_v - xt_v)_c
// Its Jacobian J = sum_j P_j^T J_j S_j follows the page "Locality-Aware
// Automatic Differentiation on the GPU for Mesh-Based Computations",
// section "Method" (vector objectives).
#pragma once

#include "dual1.h"

namespace lad {

// Spring residual in the difference z = x_a - x_b of its endpoints: with z
// seeded, g holds d R / d x_a; d R / d x_b is its negative.
template <typename D, typename T>
__device__ __forceinline__ D spring_residual(const D z[3], T rest, T sqrt_k)
{
    return sqrt_k * (sqrt(sqr(z[0]) + sqr(z[1]) + sqr(z[2])) - rest);
}

}  // namespace lad
