// user_terms.h -- local energy terms written against the term front end
// (terms_engine.h).  Each is what a user of the front end writes: a struct
// that states its stencil at compile time and gives its energy once, as a
// template over the number type.
//
//   struct Term {
//       static constexpr int kVerts;   // vertices per element (1 .. 4)
//       static constexpr int kConsts;  // per-element constants (numbers)
//       static constexpr bool kTranslationInvariant;  // depends on position
//                                      // differences only (moving every
//                                      // vertex by the same vector keeps it)
//       template <class D, class T>
//       __device__ static D energy(const D (&x)[kVerts][3], const T *c);
//   };
//
// The engine evaluates `energy` on second-order numbers for the explicit
// gradient and Hessian (StripDual) and on Hessian-vector numbers for the
// matrix-free product (DualHv); the pattern comes from the elements'
// vertex lists.  A term may use + - * /, sqr, sqrt and log between its
// numbers and with plain constants of type T, and any control flow that
// does not depend on derivatives.  Source: page "Locality-Aware Automatic
// Differentiation on the GPU for Mesh-Based Computations", section "Method"
// (the user writes only local energy terms over vertices, edges, faces or
// their neighbourhoods; the system analyses their stencil, evaluates,
// differentiates and assembles).
#pragma once

#include <hip/hip_runtime.h>

namespace lad {
namespace terms {

// 0.5 k (|x0 - x1| - L)^2;  c = {L, k}
struct Spring {
    static constexpr int kVerts = 2;
    static constexpr int kConsts = 2;
    static constexpr bool kTranslationInvariant = true;
    template <class D, class T>
    __device__ __forceinline__ static D energy(const D (&x)[2][3], const T *c)
    {
        const D l = sqrt(sqr(x[0][0] - x[1][0]) + sqr(x[0][1] - x[1][1]) +
                         sqr(x[0][2] - x[1][2]));
        return (T(0.5) * c[1]) * sqr(l - c[0]);
    }
};

// 0.5 c |x - xt|^2 at one vertex;  c = {xt_x, xt_y, xt_z, c}
struct Inertia {
    static constexpr int kVerts = 1;
    static constexpr int kConsts = 4;
    static constexpr bool kTranslationInvariant = false;
    template <class D, class T>
    __device__ __forceinline__ static D energy(const D (&x)[1][3], const T *c)
    {
        return (T(0.5) * c[3]) * (sqr(x[0][0] - c[0]) + sqr(x[0][1] - c[1]) +
                                  sqr(x[0][2] - c[2]));
    }
};

// Deformation gradient F = [x1 - x0, x2 - x0] Dm^-1 (3 x 2) and
// C = F^T F of a triangle, with c = {Dm^-1 row-major (4), rest area}.
template <class D, class T>
__device__ __forceinline__ void face_C(const D (&x)[3][3], const T *c, D &c00, D &c01, D &c11)
{
    D F[3][2];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const D d0 = x[1][r] - x[0][r], d1 = x[2][r] - x[0][r];
        F[r][0] = c[0] * d0 + c[2] * d1;
        F[r][1] = c[1] * d0 + c[3] * d1;
    }
    c00 = sqr(F[0][0]) + sqr(F[1][0]) + sqr(F[2][0]);
    c01 = F[0][0] * F[0][1] + F[1][0] * F[1][1] + F[2][0] * F[2][1];
    c11 = sqr(F[0][1]) + sqr(F[1][1]) + sqr(F[2][1]);
}

// As-rigid-as-possible: A sum_i (sigma_i - 1)^2 over F's two singular
// values, through sigma_1 + sigma_2 = sqrt(tr C + 2 sqrt(det C)):
//   A (tr C - 2 sqrt(tr C + 2 sqrt(det C)) + 2)
struct ArapFace {
    static constexpr int kVerts = 3;
    static constexpr int kConsts = 5;
    static constexpr bool kTranslationInvariant = true;
    template <class D, class T>
    __device__ __forceinline__ static D energy(const D (&x)[3][3], const T *c)
    {
        D c00, c01, c11;
        face_C(x, c, c00, c01, c11);
        const D tr = c00 + c11;
        const D det = c00 * c11 - sqr(c01);
        const D ssum = sqrt(tr + T(2) * sqrt(det));
        return c[4] * ((tr - T(2) * ssum) + T(2));
    }
};

// Symmetric Dirichlet: A (tr C + tr C / det C), the face term of the
// fixed-function kernels written as a user term.
struct SymDirichletFace {
    static constexpr int kVerts = 3;
    static constexpr int kConsts = 5;
    static constexpr bool kTranslationInvariant = true;
    template <class D, class T>
    __device__ __forceinline__ static D energy(const D (&x)[3][3], const T *c)
    {
        D c00, c01, c11;
        face_C(x, c, c00, c01, c11);
        const D tr = c00 + c11;
        const D det = c00 * c11 - sqr(c01);
        return c[4] * (tr + tr / det);
    }
};

// Quad planarity: 0.5 k det[x1 - x0, x2 - x0, x3 - x0]^2, the squared
// (six-fold) volume of the tetrahedron on a quad's four vertices, zero
// exactly when they are coplanar;  c = {k}
struct QuadPlanarity {
    static constexpr int kVerts = 4;
    static constexpr int kConsts = 1;
    static constexpr bool kTranslationInvariant = true;
    template <class D, class T>
    __device__ __forceinline__ static D energy(const D (&x)[4][3], const T *c)
    {
        D a[3], b[3], e[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            a[r] = x[1][r] - x[0][r];
            b[r] = x[2][r] - x[0][r];
            e[r] = x[3][r] - x[0][r];
        }
        const D det = a[0] * (b[1] * e[2] - b[2] * e[1]) + a[1] * (b[2] * e[0] - b[0] * e[2]) +
                      a[2] * (b[0] * e[1] - b[1] * e[0]);
        return (T(0.5) * c[0]) * sqr(det);
    }
};

}  // namespace terms
}  // namespace lad
