// contact_vf.h -- vertex-face contact term, templated on the number type
// (Dual2 for the explicit Hessian, DualHv for the Hessian-vector product).
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", key design 4 names vertex-face interactions beside
// vertex-vertex ones.  The term is the pair barrier
//   b(d) = -kappa (d - dhat)^2 ln(d / dhat)   (d < dhat)
// applied to the distance d from the contact vertex p to the triangle
// (t0, t1, t2).  The region of the triangle's closest point is decided at
// the current positions and d is then that region's smooth formula:
//   region 0, 1, 2   vertex t_i:            |p - t_i|
//   region 3, 4, 5   interior of edge (t0,t1), (t1,t2), (t2,t0) = (t_i, t_j):
//                    |(p - t_i) x (t_j - t_i)| / |t_j - t_i|
//   region 6         face interior:         |(p - t0) . n| / |n|,
//                    n = (t1 - t0) x (t2 - t0)
// The term is seeded in z_i = t_i - p (nine numbers; the distance depends
// only on them), so its z-space derivatives map to the four vertices as
//   d/dt_i = d/dz_i,   d/dp = -sum_i d/dz_i.
#pragma once

#include "dual2.h"

namespace lad {

// Region of the closest point of triangle (t0, t1, t2) to p: the Voronoi
// regions of the vertices, then of the edges, else the face, tested through
// the projections of p - t_k on the two edge directions from t0.
template <typename T>
__device__ __forceinline__ int vf_region(const T p[3], const T t0[3], const T t1[3],
                                         const T t2[3])
{
    T u[3], w[3], q0[3], q1[3], q2[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        u[c] = t1[c] - t0[c];
        w[c] = t2[c] - t0[c];
        q0[c] = p[c] - t0[c];
        q1[c] = p[c] - t1[c];
        q2[c] = p[c] - t2[c];
    }
    auto dot = [](const T a[3], const T b[3]) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2]; };
    const T a1 = dot(u, q0), a2 = dot(w, q0);
    const T b1 = dot(u, q1), b2 = dot(w, q1);
    const T c1 = dot(u, q2), c2 = dot(w, q2);
    if (a1 <= T(0) && a2 <= T(0)) return 0;
    if (b1 >= T(0) && b2 <= b1) return 1;
    if (c2 >= T(0) && c1 <= c2) return 2;
    if (a1 * b2 - b1 * a2 <= T(0) && a1 >= T(0) && b1 <= T(0)) return 3;
    if (b1 * c2 - c1 * b2 <= T(0) && b2 - b1 >= T(0) && c1 - c2 >= T(0)) return 4;
    if (c1 * a2 - a1 * c2 <= T(0) && a2 >= T(0) && c2 <= T(0)) return 5;
    return 6;
}

template <typename D>
__device__ __forceinline__ void cross3(const D a[3], const D b[3], D c[3])
{
    c[0] = a[1] * b[2] - a[2] * b[1];
    c[1] = a[2] * b[0] - a[0] * b[2];
    c[2] = a[0] * b[1] - a[1] * b[0];
}

template <typename D>
__device__ __forceinline__ D dot3(const D a[3], const D b[3])
{
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2];
}

// Distance of each region as a function of z_i = t_i - p (z[3i + c]).  The
// region's vertex indices are template arguments, so every access into z
// has a constant index and the seeds' structural zeros stay visible to the
// compiler (a runtime index would put z in scratch memory).
template <int I, typename D>
__device__ __forceinline__ D vf_vertex_distance(const D z[9])
{
    return sqrt(dot3(z + 3 * I, z + 3 * I));
}

// |(p - t_i) x e| / |e| = |z_i x e| / |e|,  e = t_j - t_i = z_j - z_i
template <int I, int J, typename D>
__device__ __forceinline__ D vf_edge_distance(const D z[9])
{
    D e[3], c[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) e[k] = z[3 * J + k] - z[3 * I + k];
    cross3(z + 3 * I, e, c);
    return sqrt(dot3(c, c) / dot3(e, e));
}

// |(t0 - p) . n| / |n|,  n = (t1 - t0) x (t2 - t0)
template <typename D>
__device__ __forceinline__ D vf_face_distance(const D z[9])
{
    D e1[3], e2[3], n[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        e1[k] = z[3 + k] - z[k];
        e2[k] = z[6 + k] - z[k];
    }
    cross3(e1, e2, n);
    const D s = dot3(z, n);
    return sqrt(sqr(s) / dot3(n, n));
}

template <typename D>
__device__ __forceinline__ D vf_distance(const D z[9], int region)
{
    switch (region) {
    case 0: return vf_vertex_distance<0>(z);
    case 1: return vf_vertex_distance<1>(z);
    case 2: return vf_vertex_distance<2>(z);
    case 3: return vf_edge_distance<0, 1>(z);
    case 4: return vf_edge_distance<1, 2>(z);
    case 5: return vf_edge_distance<2, 0>(z);
    default: return vf_face_distance(z);
    }
}

// -kappa (d - dhat)^2 ln(d / dhat); the caller guarantees d < dhat.
template <typename D, typename T>
__device__ __forceinline__ D barrier_of_distance(const D &d, T kappa, T dhat)
{
    const D t = d - dhat;
    return (-kappa) * (sqr(t) * log((T(1) / dhat) * d));
}

}  // namespace lad
