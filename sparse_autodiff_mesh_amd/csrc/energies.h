// energies.h -- the local energy terms f_j, written once over a generic
// scalar type so that evaluating them on Dual2 inputs yields value, gradient
// and Hessian by forward-mode AD (page "Locality-Aware Automatic
// Differentiation on the GPU for Mesh-Based Computations", section "Method":
// the user writes only local energy terms; the framework differentiates
// them).
//
// Each term is expressed in its natural local coordinates z, which are a
// constant linear image of the element's vertex positions:
//   two-vertex radial terms:  z = x_a - x_b                 (3 numbers)
//   inertia:                  z = x_v - xt_v                (3 numbers)
//   symmetric Dirichlet face: z = F = [x1-x0, x2-x0] Dm^-1  (6 numbers)
// The kernels seed z, evaluate the term once, and map the z-space gradient
// and Hessian to the element's 6x6 or 9x9 vertex-space blocks through that
// constant linear map (H_j = B^T H_z B).
#pragma once

#include "dual2.h"

namespace lad {

// 0.5 k (|d| - L)^2
template <typename D, typename T>
__device__ __forceinline__ D spring_energy(const D d[3], T rest, T k)
{
    D l = sqrt(sqr(d[0]) + sqr(d[1]) + sqr(d[2]));
    return (T(0.5) * k) * sqr(l - rest);
}

// -kappa (|d| - dhat)^2 ln(|d| / dhat); the caller guarantees |d| < dhat.
template <typename D, typename T>
__device__ __forceinline__ D barrier_energy(const D d[3], T kappa, T dhat)
{
    D l = sqrt(sqr(d[0]) + sqr(d[1]) + sqr(d[2]));
    D t = l - dhat;
    return (-kappa) * (sqr(t) * log((T(1) / dhat) * l));
}

// 0.5 c |z|^2 with z = x - x_tilde
template <typename D, typename T>
__device__ __forceinline__ D inertia_energy(const D z[3], T c)
{
    return (T(0.5) * c) * (sqr(z[0]) + sqr(z[1]) + sqr(z[2]));
}

// A (tr C + tr C / det C), C = F^T F, F stored row-major F[2r + c]
// (r = space axis 0..2, c = material axis 0..1).
template <typename D, typename T>
__device__ __forceinline__ D face_energy(const D F[6], T area)
{
    D c00 = sqr(F[0]) + sqr(F[2]) + sqr(F[4]);
    D c01 = F[0] * F[1] + F[2] * F[3] + F[4] * F[5];
    D c11 = sqr(F[1]) + sqr(F[3]) + sqr(F[5]);
    D tr = c00 + c11;
    D det = c00 * c11 - sqr(c01);
    // A (tr + tr / det) = tr q with q = A (1 + 1 / det), a function of det
    // alone: one chain-rule step and one product, where the quotient, the
    // sum and the scaling by A would take three passes over the Hessian
    const T inv = lad_rcp(det.v);
    const T ai = area * inv;
    const D q = chain(det, area + ai, -ai * inv, T(2) * ai * inv * inv);
    return tr * q;
}

}  // namespace lad
