/*
 * oracle.h -- plain, slow, fp64 CPU oracle for per-element mesh
 * differentiation and sparse assembly.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this code.  It shares no source, header,
 * table or helper with the GPU library, and the GPU library never loads it.
 *
 * What it computes follows the page "Locality-Aware Automatic Differentiation
 * on the GPU for Mesh-Based Computations" (Mahmoud, Goel, Ragan-Kelley,
 * Solomon), section "Method": a partially separable scalar objective
 * F(x) = sum_j f_j(x_j), each term giving a dense local gradient g_j and
 * Hessian H_j, assembled as g = sum_j S_j^T g_j and H = sum_j S_j^T H_j S_j.
 * Key design 3 (CSR preallocated from topology) and key design 4 (runtime
 * vertex-vertex pairs add off-diagonal blocks) fix the sparsity pattern.
 *
 * Conventions (readings of what the page leaves open):
 *  - DOF 3*v + c is coordinate c of vertex v.
 *  - H is block CSR with 3x3 blocks, full symmetric storage, diagonal block
 *    always present, columns ascending within a row; block k holds
 *    d2F / dx_{row,r} dx_{col_idx[k],c} at vals[9k + 3r + c].
 *  - the pattern row of vertex a is {a} U {b : a, b share a face or a
 *    spring} U {pair partners of a} U {the face vertices of a's vertex-face
 *    contacts} U {the vertices in contact with a face of a} U {the other
 *    vertices of a's planarity quads}.
 *  - the Hessian is exact (no projection or clamping).
 *
 * Every function returns 0 on success and a negative value on bad input.
 */
#ifndef LAD_ORACLE_H
#define LAD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t nv;                  /* vertices */
    int32_t nf;                  /* triangles; faces[3*f + i] */
    const int32_t *faces;
    int32_t ns;                  /* springs; springs[2*s + i], 0 = none */
    const int32_t *springs;
    const double *rest_len;      /* [ns] */
    double k;                    /* spring stiffness */
    int32_t inertia;             /* 1 = add 0.5*c*|x_v - x_tilde_v|^2 per vertex */
    double c;
    const double *x_tilde;       /* [nv*3] */
    int32_t face_energy;         /* per face: 0 = none, 1 = symmetric Dirichlet,
                                    2 = as-rigid-as-possible */
    const double *dm_inv;        /* [nf*4] row-major inverse rest edge matrix */
    const double *area;          /* [nf] rest area */
    int32_t np;                  /* vertex-vertex pairs; pairs[2*p + i] */
    const int32_t *pairs;
    double kappa, dhat;          /* barrier stiffness and support */
    int32_t nvf;                 /* vertex-face contacts; vf[2*e] = vertex,
                                    vf[2*e + 1] = face id (not one of its own) */
    const int32_t *vf;
    int32_t nq;                  /* four-vertex planarity elements; quads[4*q + i] */
    const int32_t *quads;
    double kq;                   /* their stiffness */
} oracle_problem;

/* Pattern: number of blocks, then the arrays (row_ptr[nv+1], col_idx[nnzb]). */
int64_t oracle_pattern_nnzb(const oracle_problem *p);
int oracle_pattern(const oracle_problem *p, int32_t *row_ptr, int32_t *col_idx);

/* Energy, gradient g[3*nv] and block values hvals[9*nnzb] on the given
 * pattern (which must contain every block the terms touch). */
int oracle_eval(const oracle_problem *p, const int32_t *row_ptr,
                const int32_t *col_idx, const double *x, double *energy,
                double *g, double *hvals);

/* y = H v with H the oracle's own assembled Hessian (block-CSR SpMV). */
int oracle_hvp(const oracle_problem *p, const int32_t *row_ptr,
               const int32_t *col_idx, const double *x, const double *v,
               double *y);

/* Block-CSR SpMV y = H v, exported for the tests. */
int oracle_bsr_spmv(int32_t nv, const int32_t *row_ptr, const int32_t *col_idx,
                    const double *hvals, const double *v, double *y);

/* Element-level routines, exported so the tests can pin them alone.
 * Local DOF order: vertex-major (vertex 0 xyz, vertex 1 xyz, ...). */
void oracle_spring_local(const double *xa, const double *xb, double rest,
                         double k, double *E, double *g6, double *H36);
void oracle_barrier_local(const double *xa, const double *xb, double kappa,
                          double dhat, double *E, double *g6, double *H36);
void oracle_barrier_scalar(double d, double kappa, double dhat, double *b,
                           double *db, double *ddb);
void oracle_inertia_local(const double *xv, const double *xt, double c,
                          double *E, double *g3, double *H9);
void oracle_face_local(const double *x0, const double *x1, const double *x2,
                       const double *dm_inv, double area, double *E,
                       double *g9, double *H81);
/* As-rigid-as-possible face term A sum_i (sigma_i - 1)^2, sigma_i the
 * singular values of F = [x1 - x0, x2 - x0] Dm^{-1}; value and exact
 * derivatives from hyper-dual numbers. */
void oracle_arap_local(const double *x0, const double *x1, const double *x2,
                       const double *dm_inv, double area, double *E,
                       double *g9, double *H81);
/* Quad planarity 0.5 kq det[x1 - x0, x2 - x0, x3 - x0]^2 (six times the
 * signed volume of the tetrahedron on the four points, squared); value and
 * exact derivatives from hyper-dual numbers, local DOF order x0..x3. */
void oracle_quad_local(const double *x0, const double *x1, const double *x2,
                       const double *x3, double kq, double *E, double *g12, double *H144);
/* Vertex-face contact: the barrier b(d) of the distance d from point p to
 * the triangle (t0, t1, t2).  The closest point's region is decided at the
 * given positions (type 0-2: vertex t_i; 3, 4, 5: the interior of edge
 * (t0,t1), (t1,t2), (t2,t0); 6: the face interior) and d is that region's
 * smooth formula; E, g12 and H144 (local DOF order p, t0, t1, t2) are its
 * value and exact derivatives. */
int oracle_vf_distance_type(const double *p, const double *t0, const double *t1,
                            const double *t2);
void oracle_vf_local(const double *p, const double *t0, const double *t1,
                     const double *t2, double kappa, double dhat, double *E,
                     double *g12, double *H144);
/* Face gradient taken from the hyper-dual evaluator instead of the closed
 * form (for cross-checking the two). */
void oracle_face_grad_hyperdual(const double *x0, const double *x1,
                                const double *x2, const double *dm_inv,
                                double area, double *g9);

#ifdef __cplusplus
}
#endif
#endif
