// lad_jacobian.hip -- residuals and explicit sparse Jacobian of the vector
// objective (least-squares form of the spring and inertia terms).
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", section "Method": a vector-valued objective yields small
// dense local Jacobians J_j assembled into J = sum_j P_j^T J_j S_j.  Every
// residual row belongs to exactly one local term (the P_j are disjoint), so
// assembly needs no accumulation: each term writes its own rows, one thread
// per spring and one per inertia DOF, values in the fixed pattern order.
// The spring's local Jacobian comes from a first-order dual evaluation in
// the endpoint difference z = x_a - x_b (d R / d x_a = dR/dz, d R / d x_b =
// -dR/dz).
#include "lad_jacobian.h"
#include "residuals.h"

namespace lad {

namespace {

constexpr int NT = 256;

__global__ void __launch_bounds__(NT)
k_jac_pattern(int32_t ns, const int32_t *__restrict__ springs, int64_t inertia_rows,
              int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx)
{
    const int64_t t = int64_t(blockIdx.x) * NT + threadIdx.x;
    const int64_t m = int64_t(ns) + inertia_rows;
    if (t < ns) {
        int32_t a = springs[2 * t], b = springs[2 * t + 1];
        if (a > b) {
            const int32_t q = a;
            a = b;
            b = q;
        }
        row_ptr[t] = int32_t(6 * t);
        int32_t *c = col_idx + 6 * t;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            c[k] = 3 * a + k;
            c[3 + k] = 3 * b + k;
        }
    } else if (t < m) {
        const int64_t i = t - ns;
        row_ptr[t] = int32_t(6 * int64_t(ns) + i);
        col_idx[6 * int64_t(ns) + i] = int32_t(i);
    }
    if (t == (m > 0 ? m - 1 : 0)) row_ptr[m] = int32_t(6 * int64_t(ns) + inertia_rows);
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_res_jac(int32_t ns, const int32_t *__restrict__ springs, const T *__restrict__ rest, T sqrt_k,
          int64_t inertia_rows, const T *__restrict__ x, const T *__restrict__ xt, T sqrt_c,
          T *__restrict__ r, T *__restrict__ jv)
{
    const int64_t t = int64_t(blockIdx.x) * NT + threadIdx.x;
    if (t < ns) {
        const int32_t a = springs[2 * t], b = springs[2 * t + 1];
        Dual1<T, 3> z[3];
#pragma unroll
        for (int c = 0; c < 3; ++c) z[c] = Dual1<T, 3>::var(x[3 * int64_t(a) + c] - x[3 * int64_t(b) + c], c);
        const Dual1<T, 3> e = spring_residual(z, rest[t], sqrt_k);
        r[t] = e.v;
        // columns ascending: the lower-numbered vertex's three DOFs first
        T *j = jv + 6 * t;
        const T sa = a < b ? T(1) : T(-1);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            j[k] = sa * e.g[k];
            j[3 + k] = -sa * e.g[k];
        }
    } else if (t < int64_t(ns) + inertia_rows) {
        // R = sqrt(c) (x_i - xt_i): value and its one derivative, sqrt(c)
        const int64_t i = t - ns;
        r[t] = sqrt_c * (x[i] - xt[i]);
        jv[6 * int64_t(ns) + i] = sqrt_c;
    }
}

inline unsigned blocks_for(int64_t n) { return unsigned((n + NT - 1) / NT); }

}  // namespace

hipError_t launch_jacobian_pattern(int32_t ns, const int32_t *springs, int64_t inertia_rows,
                                   int32_t *row_ptr, int32_t *col_idx, hipStream_t s)
{
    const int64_t m = int64_t(ns) + inertia_rows;
    hipLaunchKernelGGL(k_jac_pattern, dim3(blocks_for(m > 0 ? m : 1)), dim3(NT), 0, s, ns, springs,
                       inertia_rows, row_ptr, col_idx);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_residual_jacobian(int32_t ns, const int32_t *springs, const T *rest, T sqrt_k,
                                    int64_t inertia_rows, const T *x, const T *x_tilde, T sqrt_c,
                                    T *r, T *jvals, hipStream_t s)
{
    const int64_t m = int64_t(ns) + inertia_rows;
    if (m == 0) return hipSuccess;
    hipLaunchKernelGGL(k_res_jac<T>, dim3(blocks_for(m)), dim3(NT), 0, s, ns, springs, rest,
                       sqrt_k, inertia_rows, x, x_tilde, sqrt_c, r, jvals);
    return hipGetLastError();
}

template hipError_t launch_residual_jacobian<float>(int32_t, const int32_t *, const float *, float,
                                                    int64_t, const float *, const float *, float,
                                                    float *, float *, hipStream_t);
template hipError_t launch_residual_jacobian<double>(int32_t, const int32_t *, const double *,
                                                     double, int64_t, const double *,
                                                     const double *, double, double *, double *,
                                                     hipStream_t);

}  // namespace lad
