/*
 * oracle.c -- plain fp64 CPU oracle (test infrastructure only; see oracle.h).
 *
 * Single-threaded, no blocking, no fusion.  Each element's derivatives come
 * from textbook closed forms (springs, inertia, barrier, face gradient) or
 * from a hyper-dual evaluator (face Hessian), never from the second-order
 * dual numbers the GPU library uses.  Assembly looks every block up by
 * binary search in the row and adds into it, element after element.
 *
 * Source: page "Locality-Aware Automatic Differentiation on the GPU for
 * Mesh-Based Computations", section "Method" (objective F(x) = sum_j f_j(x_j)
 * and assembly through selection matrices S_j), key designs 3 and 4 (pattern
 * from topology plus runtime vertex-vertex and vertex-face interactions).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Pattern: sort-unique of all directed vertex pairs that share an element  */
/* ------------------------------------------------------------------------ */

typedef struct { int32_t r, c; } rc_pair;

static int cmp_rc(const void *a, const void *b)
{
    const rc_pair *x = (const rc_pair *)a, *y = (const rc_pair *)b;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->c != y->c) return x->c < y->c ? -1 : 1;
    return 0;
}

static int check_problem(const oracle_problem *p)
{
    if (!p || p->nv < 0 || p->nf < 0 || p->ns < 0 || p->np < 0 || p->nvf < 0 || p->nq < 0)
        return -1;
    if (p->nq > 0 && !p->quads) return -1;
    for (int32_t q = 0; q < p->nq; ++q)
        for (int i = 0; i < 4; ++i) {
            int32_t v = p->quads[4 * (int64_t)q + i];
            if (v < 0 || v >= p->nv) return -1;
            for (int j = 0; j < i; ++j)
                if (p->quads[4 * (int64_t)q + j] == v) return -1;
        }
    if (p->nvf > 0 && !p->vf) return -1;
    if (p->nf > 0 && !p->faces) return -1;
    if (p->ns > 0 && (!p->springs || !p->rest_len)) return -1;
    if (p->np > 0 && !p->pairs) return -1;
    if (p->inertia && p->nv > 0 && !p->x_tilde) return -1;
    if (p->face_energy && p->nf > 0 && (!p->dm_inv || !p->area)) return -1;
    for (int64_t i = 0; i < 3 * (int64_t)p->nf; ++i)
        if (p->faces[i] < 0 || p->faces[i] >= p->nv) return -1;
    for (int64_t i = 0; i < 2 * (int64_t)p->ns; ++i)
        if (p->springs[i] < 0 || p->springs[i] >= p->nv) return -1;
    for (int64_t i = 0; i < 2 * (int64_t)p->np; ++i)
        if (p->pairs[i] < 0 || p->pairs[i] >= p->nv) return -1;
    /* a spring and a vertex-vertex pair join two distinct vertices (a pair
     * of one vertex would sit at distance zero, where the barrier is
     * infinite) */
    for (int32_t s = 0; s < p->ns; ++s)
        if (p->springs[2 * (int64_t)s] == p->springs[2 * (int64_t)s + 1]) return -1;
    for (int32_t q = 0; q < p->np; ++q)
        if (p->pairs[2 * (int64_t)q] == p->pairs[2 * (int64_t)q + 1]) return -1;
    for (int32_t e = 0; e < p->nvf; ++e) {
        int32_t v = p->vf[2 * (int64_t)e], f = p->vf[2 * (int64_t)e + 1];
        if (v < 0 || v >= p->nv || f < 0 || f >= p->nf) return -1;
        for (int i = 0; i < 3; ++i)
            if (p->faces[3 * (int64_t)f + i] == v) return -1;
    }
    return 0;
}

/* All directed (row, col) pairs: self, both directions of every face edge,
 * every spring, every pair.  Sorted, duplicates kept. */
static rc_pair *directed_pairs(const oracle_problem *p, int64_t *count)
{
    int64_t n = (int64_t)p->nv + 6 * (int64_t)p->nf + 2 * (int64_t)p->ns +
                2 * (int64_t)p->np + 6 * (int64_t)p->nvf + 12 * (int64_t)p->nq;
    rc_pair *e = (rc_pair *)malloc((size_t)(n > 0 ? n : 1) * sizeof(rc_pair));
    if (!e) return NULL;
    int64_t m = 0;
    for (int32_t v = 0; v < p->nv; ++v) { e[m].r = v; e[m].c = v; ++m; }
    for (int32_t f = 0; f < p->nf; ++f) {
        const int32_t *t = p->faces + 3 * (int64_t)f;
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                if (i != j) { e[m].r = t[i]; e[m].c = t[j]; ++m; }
    }
    for (int32_t s = 0; s < p->ns; ++s) {
        int32_t a = p->springs[2 * (int64_t)s], b = p->springs[2 * (int64_t)s + 1];
        e[m].r = a; e[m].c = b; ++m;
        e[m].r = b; e[m].c = a; ++m;
    }
    for (int32_t q = 0; q < p->np; ++q) {
        int32_t a = p->pairs[2 * (int64_t)q], b = p->pairs[2 * (int64_t)q + 1];
        e[m].r = a; e[m].c = b; ++m;
        e[m].r = b; e[m].c = a; ++m;
    }
    for (int32_t q = 0; q < p->nvf; ++q) {
        int32_t v = p->vf[2 * (int64_t)q], f = p->vf[2 * (int64_t)q + 1];
        for (int i = 0; i < 3; ++i) {
            int32_t t = p->faces[3 * (int64_t)f + i];
            e[m].r = v; e[m].c = t; ++m;
            e[m].r = t; e[m].c = v; ++m;
        }
    }
    for (int32_t q = 0; q < p->nq; ++q) {
        const int32_t *t = p->quads + 4 * (int64_t)q;
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j)
                if (i != j) { e[m].r = t[i]; e[m].c = t[j]; ++m; }
    }
    qsort(e, (size_t)m, sizeof(rc_pair), cmp_rc);
    *count = m;
    return e;
}

int64_t oracle_pattern_nnzb(const oracle_problem *p)
{
    if (check_problem(p)) return -1;
    int64_t m;
    rc_pair *e = directed_pairs(p, &m);
    if (!e) return -2;
    int64_t u = 0;
    for (int64_t i = 0; i < m; ++i)
        if (i == 0 || cmp_rc(&e[i], &e[i - 1]) != 0) ++u;
    free(e);
    return u;
}

int oracle_pattern(const oracle_problem *p, int32_t *row_ptr, int32_t *col_idx)
{
    if (check_problem(p) || !row_ptr || !col_idx) return -1;
    int64_t m;
    rc_pair *e = directed_pairs(p, &m);
    if (!e) return -2;
    for (int32_t v = 0; v <= p->nv; ++v) row_ptr[v] = 0;
    int64_t u = 0;
    for (int64_t i = 0; i < m; ++i) {
        if (i > 0 && cmp_rc(&e[i], &e[i - 1]) == 0) continue;
        col_idx[u++] = e[i].c;
        row_ptr[e[i].r + 1] += 1;
    }
    for (int32_t v = 0; v < p->nv; ++v) row_ptr[v + 1] += row_ptr[v];
    free(e);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Radial two-vertex terms psi(l), l = |xa - xb|                            */
/* ------------------------------------------------------------------------ */

/* With n = (xa - xb) / l:  g_a = psi' n,  g_b = -g_a,
 * K = psi'' n n^T + (psi' / l)(I - n n^T),  H = [[K, -K], [-K, K]]. */
static void radial_local(const double *xa, const double *xb, double psi,
                         double dpsi, double ddpsi, double *E, double *g6,
                         double *H36)
{
    double d[3] = {xa[0] - xb[0], xa[1] - xb[1], xa[2] - xb[2]};
    double l = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    double n[3] = {d[0] / l, d[1] / l, d[2] / l};
    *E = psi;
    for (int i = 0; i < 3; ++i) {
        g6[i] = dpsi * n[i];
        g6[3 + i] = -dpsi * n[i];
    }
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double nn = n[i] * n[j]; /* same product for (i,j) and (j,i) */
            double K = ddpsi * nn + (dpsi / l) * ((i == j ? 1.0 : 0.0) - nn);
            H36[6 * i + j] = K;
            H36[6 * (i + 3) + (j + 3)] = K;
            H36[6 * i + (j + 3)] = -K;
            H36[6 * (i + 3) + j] = -K;
        }
}

/* Mass-spring term 0.5 k (l - L)^2. */
void oracle_spring_local(const double *xa, const double *xb, double rest,
                         double k, double *E, double *g6, double *H36)
{
    double d[3] = {xa[0] - xb[0], xa[1] - xb[1], xa[2] - xb[2]};
    double l = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    double s = l - rest;
    radial_local(xa, xb, 0.5 * k * s * s, k * s, k, E, g6, H36);
}

/* Log barrier b(d) = -kappa (d - dhat)^2 ln(d / dhat) for d < dhat, else 0.
 *   b'  = -kappa [2 (d - dhat) ln(d/dhat) + (d - dhat)^2 / d]
 *   b'' = -kappa [2 ln(d/dhat) + 4 (d - dhat)/d - (d - dhat)^2 / d^2]      */
void oracle_barrier_scalar(double d, double kappa, double dhat, double *b,
                           double *db, double *ddb)
{
    if (d >= dhat) { *b = 0.0; *db = 0.0; *ddb = 0.0; return; }
    double t = d - dhat, lg = log(d / dhat);
    *b = -kappa * t * t * lg;
    *db = -kappa * (2.0 * t * lg + t * t / d);
    *ddb = -kappa * (2.0 * lg + 4.0 * t / d - t * t / (d * d));
}

void oracle_barrier_local(const double *xa, const double *xb, double kappa,
                          double dhat, double *E, double *g6, double *H36)
{
    double d[3] = {xa[0] - xb[0], xa[1] - xb[1], xa[2] - xb[2]};
    double l = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    double b, db, ddb;
    oracle_barrier_scalar(l, kappa, dhat, &b, &db, &ddb);
    if (l >= dhat) {
        *E = 0.0;
        memset(g6, 0, 6 * sizeof(double));
        memset(H36, 0, 36 * sizeof(double));
        return;
    }
    radial_local(xa, xb, b, db, ddb, E, g6, H36);
}

/* Inertia 0.5 c |x - x_tilde|^2: g = c (x - x_tilde), H = c I. */
void oracle_inertia_local(const double *xv, const double *xt, double c,
                          double *E, double *g3, double *H9)
{
    double e = 0.0;
    for (int i = 0; i < 3; ++i) {
        double d = xv[i] - xt[i];
        e += d * d;
        g3[i] = c * d;
        for (int j = 0; j < 3; ++j) H9[3 * i + j] = (i == j) ? c : 0.0;
    }
    *E = 0.5 * c * e;
}

/* ------------------------------------------------------------------------ */
/* Face: symmetric Dirichlet E = A (tr C + tr C / det C), C = F^T F,        */
/* F = [x1 - x0, x2 - x0] Dm^{-1}  (3x2)                                    */
/* ------------------------------------------------------------------------ */

/* F[r][c] for r in 0..2 (space), c in 0..1 (material). */
static void face_F(const double *x0, const double *x1, const double *x2,
                   const double *Mi, double F[3][2])
{
    for (int r = 0; r < 3; ++r) {
        double d0 = x1[r] - x0[r], d1 = x2[r] - x0[r];
        F[r][0] = d0 * Mi[0] + d1 * Mi[2];
        F[r][1] = d0 * Mi[1] + d1 * Mi[3];
    }
}

/* Closed-form energy and gradient.
 *   dE/dF = A [2F + 2F/det C - (tr C / det C^2) 2 F adj(C)]
 * with adj(C) = [[C11, -C01], [-C01, C00]];  dE/dD = dE/dF Dm^{-T};
 * g1 = column 0 of dE/dD, g2 = column 1, g0 = -(g1 + g2).               */
static void face_energy_grad(const double *x0, const double *x1,
                             const double *x2, const double *Mi, double A,
                             double *E, double *g9)
{
    double F[3][2];
    face_F(x0, x1, x2, Mi, F);
    double C00 = 0, C01 = 0, C11 = 0;
    for (int r = 0; r < 3; ++r) {
        C00 += F[r][0] * F[r][0];
        C01 += F[r][0] * F[r][1];
        C11 += F[r][1] * F[r][1];
    }
    double tr = C00 + C11, det = C00 * C11 - C01 * C01;
    *E = A * (tr + tr / det);
    if (!g9) return;
    double adj[2][2] = {{C11, -C01}, {-C01, C00}};
    double P[3][2];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 2; ++c) {
            double Fadj = F[r][0] * adj[0][c] + F[r][1] * adj[1][c];
            P[r][c] = A * (2.0 * F[r][c] + 2.0 * F[r][c] / det -
                           (tr / (det * det)) * 2.0 * Fadj);
        }
    for (int r = 0; r < 3; ++r) {
        /* dE/dD[r][k] = sum_c P[r][c] * Mi[k][c] */
        double gd0 = P[r][0] * Mi[0] + P[r][1] * Mi[1];
        double gd1 = P[r][0] * Mi[2] + P[r][1] * Mi[3];
        g9[3 + r] = gd0;
        g9[6 + r] = gd1;
        g9[r] = -(gd0 + gd1);
    }
}

/* Hyper-dual numbers a + b e1 + c e2 + d e1 e2 with e1^2 = e2^2 = 0
 * (Fike and Alonso, "The development of hyper-dual numbers for exact
 * second-derivative calculations", AIAA 2011).  Seeding x with e1 along
 * direction p and e2 along direction q makes the e1 e2 part of E(x) equal
 * p^T (d2E/dx2) q exactly. */
typedef struct { double a, b, c, d; } hd;

static hd hd_make(double a, double b, double c) { hd r = {a, b, c, 0.0}; return r; }
static hd hd_add(hd x, hd y) { hd r = {x.a + y.a, x.b + y.b, x.c + y.c, x.d + y.d}; return r; }
static hd hd_sub(hd x, hd y) { hd r = {x.a - y.a, x.b - y.b, x.c - y.c, x.d - y.d}; return r; }
static hd hd_mul(hd x, hd y)
{
    hd r = {x.a * y.a, x.a * y.b + x.b * y.a, x.a * y.c + x.c * y.a,
            x.a * y.d + x.b * y.c + x.c * y.b + x.d * y.a};
    return r;
}
static hd hd_scale(hd x, double s) { hd r = {s * x.a, s * x.b, s * x.c, s * x.d}; return r; }
/* 1/y: f = 1/a, f' = -1/a^2, f'' = 2/a^3. */
static hd hd_inv(hd y)
{
    double ia = 1.0 / y.a;
    hd r = {ia, -y.b * ia * ia, -y.c * ia * ia,
            -y.d * ia * ia + 2.0 * y.b * y.c * ia * ia * ia};
    return r;
}

/* E at the nine hyper-dual coordinates X[3*i + r] (vertex i, axis r). */
static hd face_energy_hd(const hd *X, const double *Mi, double A)
{
    hd F[3][2];
    for (int r = 0; r < 3; ++r) {
        hd d0 = hd_sub(X[3 + r], X[r]);
        hd d1 = hd_sub(X[6 + r], X[r]);
        F[r][0] = hd_add(hd_scale(d0, Mi[0]), hd_scale(d1, Mi[2]));
        F[r][1] = hd_add(hd_scale(d0, Mi[1]), hd_scale(d1, Mi[3]));
    }
    hd C00 = hd_make(0, 0, 0), C01 = hd_make(0, 0, 0), C11 = hd_make(0, 0, 0);
    for (int r = 0; r < 3; ++r) {
        C00 = hd_add(C00, hd_mul(F[r][0], F[r][0]));
        C01 = hd_add(C01, hd_mul(F[r][0], F[r][1]));
        C11 = hd_add(C11, hd_mul(F[r][1], F[r][1]));
    }
    hd tr = hd_add(C00, C11);
    hd det = hd_sub(hd_mul(C00, C11), hd_mul(C01, C01));
    return hd_scale(hd_add(tr, hd_mul(tr, hd_inv(det))), A);
}

static void face_seed(const double *x0, const double *x1, const double *x2,
                      int p, int q, hd *X)
{
    const double *xs[3] = {x0, x1, x2};
    for (int i = 0; i < 9; ++i)
        X[i] = hd_make(xs[i / 3][i % 3], i == p ? 1.0 : 0.0, i == q ? 1.0 : 0.0);
}

void oracle_face_local(const double *x0, const double *x1, const double *x2,
                       const double *dm_inv, double area, double *E,
                       double *g9, double *H81)
{
    face_energy_grad(x0, x1, x2, dm_inv, area, E, g9);
    hd X[9];
    for (int p = 0; p < 9; ++p)
        for (int q = p; q < 9; ++q) {
            face_seed(x0, x1, x2, p, q, X);
            hd e = face_energy_hd(X, dm_inv, area);
            H81[9 * p + q] = e.d;
            H81[9 * q + p] = e.d;
        }
}

void oracle_face_grad_hyperdual(const double *x0, const double *x1,
                                const double *x2, const double *dm_inv,
                                double area, double *g9)
{
    hd X[9];
    for (int p = 0; p < 9; ++p) {
        face_seed(x0, x1, x2, p, -1, X);
        g9[p] = face_energy_hd(X, dm_inv, area).b;
    }
}

/* ------------------------------------------------------------------------ */
/* Face: as-rigid-as-possible E = A sum_i (sigma_i - 1)^2 over the two      */
/* singular values of the same F.  With C = F^T F:                          */
/*   sigma_1^2 + sigma_2^2 = tr C,  sigma_1 sigma_2 = sqrt(det C),          */
/*   so sigma_1 + sigma_2 = sqrt(tr C + 2 sqrt(det C)) and                  */
/*   E = A (tr C - 2 (sigma_1 + sigma_2) + 2).                              */
/* ------------------------------------------------------------------------ */

static hd hd_sqrt(hd x);

static hd arap_energy_hd(const hd *X, const double *Mi, double A)
{
    hd F[3][2];
    for (int r = 0; r < 3; ++r) {
        hd d0 = hd_sub(X[3 + r], X[r]);
        hd d1 = hd_sub(X[6 + r], X[r]);
        F[r][0] = hd_add(hd_scale(d0, Mi[0]), hd_scale(d1, Mi[2]));
        F[r][1] = hd_add(hd_scale(d0, Mi[1]), hd_scale(d1, Mi[3]));
    }
    hd C00 = hd_make(0, 0, 0), C01 = hd_make(0, 0, 0), C11 = hd_make(0, 0, 0);
    for (int r = 0; r < 3; ++r) {
        C00 = hd_add(C00, hd_mul(F[r][0], F[r][0]));
        C01 = hd_add(C01, hd_mul(F[r][0], F[r][1]));
        C11 = hd_add(C11, hd_mul(F[r][1], F[r][1]));
    }
    hd tr = hd_add(C00, C11);
    hd det = hd_sub(hd_mul(C00, C11), hd_mul(C01, C01));
    hd ssum = hd_sqrt(hd_add(tr, hd_scale(hd_sqrt(det), 2.0)));
    return hd_scale(hd_add(hd_sub(tr, hd_scale(ssum, 2.0)), hd_make(2.0, 0.0, 0.0)), A);
}

void oracle_arap_local(const double *x0, const double *x1, const double *x2,
                       const double *dm_inv, double area, double *E,
                       double *g9, double *H81)
{
    hd X[9];
    for (int p = 0; p < 9; ++p)
        for (int q = p; q < 9; ++q) {
            face_seed(x0, x1, x2, p, q, X);
            hd e = arap_energy_hd(X, dm_inv, area);
            H81[9 * p + q] = e.d;
            H81[9 * q + p] = e.d;
            if (p == q) {
                g9[p] = e.b;
                *E = e.a;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Quad planarity: 0.5 kq D^2, D = det[x1 - x0, x2 - x0, x3 - x0]            */
/* (the triple product (x1 - x0) . ((x2 - x0) x (x3 - x0)))                 */
/* ------------------------------------------------------------------------ */

static hd quad_energy_hd(const hd *X, double kq)
{
    hd a[3], b[3], c[3];
    for (int r = 0; r < 3; ++r) {
        a[r] = hd_sub(X[3 + r], X[r]);
        b[r] = hd_sub(X[6 + r], X[r]);
        c[r] = hd_sub(X[9 + r], X[r]);
    }
    hd bxc0 = hd_sub(hd_mul(b[1], c[2]), hd_mul(b[2], c[1]));
    hd bxc1 = hd_sub(hd_mul(b[2], c[0]), hd_mul(b[0], c[2]));
    hd bxc2 = hd_sub(hd_mul(b[0], c[1]), hd_mul(b[1], c[0]));
    hd D = hd_add(hd_add(hd_mul(a[0], bxc0), hd_mul(a[1], bxc1)), hd_mul(a[2], bxc2));
    return hd_scale(hd_mul(D, D), 0.5 * kq);
}

void oracle_quad_local(const double *x0, const double *x1, const double *x2,
                       const double *x3, double kq, double *E, double *g12, double *H144)
{
    const double *xs[4] = {x0, x1, x2, x3};
    hd X[12];
    for (int a = 0; a < 12; ++a)
        for (int b = a; b < 12; ++b) {
            for (int i = 0; i < 12; ++i)
                X[i] = hd_make(xs[i / 3][i % 3], i == a ? 1.0 : 0.0, i == b ? 1.0 : 0.0);
            hd e = quad_energy_hd(X, kq);
            H144[12 * a + b] = e.d;
            H144[12 * b + a] = e.d;
            if (a == b) {
                g12[a] = e.b;
                *E = e.a;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Vertex-face contact: barrier of the point-triangle distance              */
/* ------------------------------------------------------------------------ */

static double dot3(const double *a, const double *b)
{
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2];
}

/* Region of the triangle's closest point to p, from the signs of the
 * projections of p onto the edge directions (the Voronoi regions of the
 * three vertices, three edges and the face). */
int oracle_vf_distance_type(const double *p, const double *t0, const double *t1,
                            const double *t2)
{
    double e01[3], e02[3], q0[3], q1[3], q2[3];
    for (int i = 0; i < 3; ++i) {
        e01[i] = t1[i] - t0[i];
        e02[i] = t2[i] - t0[i];
        q0[i] = p[i] - t0[i];
        q1[i] = p[i] - t1[i];
        q2[i] = p[i] - t2[i];
    }
    /* projections onto e01 and e02 measured from each vertex */
    double a1 = dot3(e01, q0), a2 = dot3(e02, q0);
    if (a1 <= 0.0 && a2 <= 0.0) return 0;
    double b1 = dot3(e01, q1), b2 = dot3(e02, q1);
    if (b1 >= 0.0 && b2 <= b1) return 1;
    double c1 = dot3(e01, q2), c2 = dot3(e02, q2);
    if (c2 >= 0.0 && c1 <= c2) return 2;
    /* edge regions: the barycentric weight of the opposite vertex is <= 0
     * while p projects inside the edge */
    if (a1 * b2 - b1 * a2 <= 0.0 && a1 >= 0.0 && b1 <= 0.0) return 3;          /* (t0,t1) */
    if (b1 * c2 - c1 * b2 <= 0.0 && b2 - b1 >= 0.0 && c1 - c2 >= 0.0) return 4; /* (t1,t2) */
    if (c1 * a2 - a1 * c2 <= 0.0 && a2 >= 0.0 && c2 <= 0.0) return 5;          /* (t2,t0) */
    return 6;
}

static hd hd_sqrt(hd x)
{
    double s = sqrt(x.a), d1 = 0.5 / s, d2 = -0.25 / (s * x.a);
    hd r = {s, d1 * x.b, d1 * x.c, d1 * x.d + d2 * x.b * x.c};
    return r;
}

static hd hd_log(hd x)
{
    double d1 = 1.0 / x.a, d2 = -d1 * d1;
    hd r = {log(x.a), d1 * x.b, d1 * x.c, d1 * x.d + d2 * x.b * x.c};
    return r;
}

static hd hd_dot3(const hd *a, const hd *b)
{
    return hd_add(hd_add(hd_mul(a[0], b[0]), hd_mul(a[1], b[1])), hd_mul(a[2], b[2]));
}

static void hd_cross3(const hd *a, const hd *b, hd *c)
{
    c[0] = hd_sub(hd_mul(a[1], b[2]), hd_mul(a[2], b[1]));
    c[1] = hd_sub(hd_mul(a[2], b[0]), hd_mul(a[0], b[2]));
    c[2] = hd_sub(hd_mul(a[0], b[1]), hd_mul(a[1], b[0]));
}

/* Barrier of the distance of the given type, at hyper-dual coordinates
 * X[0..2] = p, X[3..5] = t0, X[6..8] = t1, X[9..11] = t2. */
static hd vf_energy_hd(const hd *X, int type, double kappa, double dhat)
{
    const hd *P = X, *T[3] = {X + 3, X + 6, X + 9};
    hd d;
    if (type <= 2) {                       /* |p - t_i| */
        hd q[3];
        for (int i = 0; i < 3; ++i) q[i] = hd_sub(P[i], T[type][i]);
        d = hd_sqrt(hd_dot3(q, q));
    } else if (type <= 5) {                /* |(p - t_i) x (t_j - t_i)| / |t_j - t_i| */
        int i = type - 3, j = (type - 2) % 3;
        hd q[3], e[3], c[3];
        for (int k = 0; k < 3; ++k) {
            q[k] = hd_sub(P[k], T[i][k]);
            e[k] = hd_sub(T[j][k], T[i][k]);
        }
        hd_cross3(q, e, c);
        d = hd_sqrt(hd_mul(hd_dot3(c, c), hd_inv(hd_dot3(e, e))));
    } else {                               /* |(p - t0) . n| / |n| */
        hd e1[3], e2[3], n[3], q[3];
        for (int k = 0; k < 3; ++k) {
            e1[k] = hd_sub(T[1][k], T[0][k]);
            e2[k] = hd_sub(T[2][k], T[0][k]);
            q[k] = hd_sub(P[k], T[0][k]);
        }
        hd_cross3(e1, e2, n);
        hd s = hd_dot3(q, n);
        d = hd_sqrt(hd_mul(hd_mul(s, s), hd_inv(hd_dot3(n, n))));
    }
    if (!(d.a < dhat)) return hd_make(0.0, 0.0, 0.0);
    hd t = hd_sub(d, hd_make(dhat, 0.0, 0.0));
    hd lg = hd_log(hd_scale(d, 1.0 / dhat));
    return hd_scale(hd_mul(hd_mul(t, t), lg), -kappa);
}

void oracle_vf_local(const double *p, const double *t0, const double *t1,
                     const double *t2, double kappa, double dhat, double *E,
                     double *g12, double *H144)
{
    const double *xs[4] = {p, t0, t1, t2};
    const int type = oracle_vf_distance_type(p, t0, t1, t2);
    hd X[12];
    for (int a = 0; a < 12; ++a)
        for (int b = a; b < 12; ++b) {
            for (int i = 0; i < 12; ++i)
                X[i] = hd_make(xs[i / 3][i % 3], i == a ? 1.0 : 0.0, i == b ? 1.0 : 0.0);
            hd e = vf_energy_hd(X, type, kappa, dhat);
            H144[12 * a + b] = e.d;
            H144[12 * b + a] = e.d;
            if (a == b) {
                g12[a] = e.b;
                *E = e.a;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Assembly: g = sum_j S_j^T g_j,  H = sum_j S_j^T H_j S_j                  */
/* ------------------------------------------------------------------------ */

static int64_t find_block(const int32_t *row_ptr, const int32_t *col_idx,
                          int32_t a, int32_t b)
{
    int64_t lo = row_ptr[a], hi = row_ptr[a + 1];
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (col_idx[mid] < b) lo = mid + 1;
        else hi = mid;
    }
    if (lo < row_ptr[a + 1] && col_idx[lo] == b) return lo;
    return -1;
}

/* Scatter one element with m vertices vid[0..m-1] and local g (3m), H
 * (3m x 3m, row-major) into the global arrays.  Returns -1 if a block the
 * element touches is missing from the pattern. */
static int scatter(const int32_t *row_ptr, const int32_t *col_idx, int m,
                   const int32_t *vid, const double *gl, const double *Hl,
                   double *g, double *hvals)
{
    int w = 3 * m;
    for (int i = 0; i < m; ++i)
        for (int r = 0; r < 3; ++r) g[3 * (int64_t)vid[i] + r] += gl[3 * i + r];
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < m; ++j) {
            int64_t k = find_block(row_ptr, col_idx, vid[i], vid[j]);
            if (k < 0) return -1;
            for (int r = 0; r < 3; ++r)
                for (int c = 0; c < 3; ++c)
                    hvals[9 * k + 3 * r + c] += Hl[w * (3 * i + r) + 3 * j + c];
        }
    return 0;
}

int oracle_eval(const oracle_problem *p, const int32_t *row_ptr,
                const int32_t *col_idx, const double *x, double *energy,
                double *g, double *hvals)
{
    if (check_problem(p) || !row_ptr || !col_idx || !x || !energy || !g || !hvals)
        return -1;
    int64_t nnzb = row_ptr[p->nv];
    memset(g, 0, 3 * (size_t)p->nv * sizeof(double));
    memset(hvals, 0, 9 * (size_t)nnzb * sizeof(double));
    double E = 0.0;
    double e, gl[12], Hl[144];
    int32_t vid[4];

    for (int32_t s = 0; s < p->ns; ++s) {
        vid[0] = p->springs[2 * (int64_t)s];
        vid[1] = p->springs[2 * (int64_t)s + 1];
        oracle_spring_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                            p->rest_len[s], p->k, &e, gl, Hl);
        E += e;
        if (scatter(row_ptr, col_idx, 2, vid, gl, Hl, g, hvals)) return -3;
    }
    if (p->inertia) {
        for (int32_t v = 0; v < p->nv; ++v) {
            vid[0] = v;
            oracle_inertia_local(x + 3 * (int64_t)v, p->x_tilde + 3 * (int64_t)v,
                                 p->c, &e, gl, Hl);
            E += e;
            if (scatter(row_ptr, col_idx, 1, vid, gl, Hl, g, hvals)) return -3;
        }
    }
    if (p->face_energy) {
        for (int32_t f = 0; f < p->nf; ++f) {
            for (int i = 0; i < 3; ++i) vid[i] = p->faces[3 * (int64_t)f + i];
            if (p->face_energy == 2)
                oracle_arap_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                                  x + 3 * (int64_t)vid[2], p->dm_inv + 4 * (int64_t)f,
                                  p->area[f], &e, gl, Hl);
            else
                oracle_face_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                                  x + 3 * (int64_t)vid[2], p->dm_inv + 4 * (int64_t)f,
                                  p->area[f], &e, gl, Hl);
            E += e;
            if (scatter(row_ptr, col_idx, 3, vid, gl, Hl, g, hvals)) return -3;
        }
    }
    for (int32_t q = 0; q < p->np; ++q) {
        vid[0] = p->pairs[2 * (int64_t)q];
        vid[1] = p->pairs[2 * (int64_t)q + 1];
        if (vid[0] == vid[1]) return -1;
        oracle_barrier_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                             p->kappa, p->dhat, &e, gl, Hl);
        E += e;
        if (scatter(row_ptr, col_idx, 2, vid, gl, Hl, g, hvals)) return -3;
    }
    for (int32_t q = 0; q < p->nvf; ++q) {
        vid[0] = p->vf[2 * (int64_t)q];
        for (int i = 0; i < 3; ++i) vid[1 + i] = p->faces[3 * (int64_t)p->vf[2 * (int64_t)q + 1] + i];
        oracle_vf_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                        x + 3 * (int64_t)vid[2], x + 3 * (int64_t)vid[3], p->kappa, p->dhat,
                        &e, gl, Hl);
        E += e;
        if (scatter(row_ptr, col_idx, 4, vid, gl, Hl, g, hvals)) return -3;
    }
    for (int32_t q = 0; q < p->nq; ++q) {
        for (int i = 0; i < 4; ++i) vid[i] = p->quads[4 * (int64_t)q + i];
        oracle_quad_local(x + 3 * (int64_t)vid[0], x + 3 * (int64_t)vid[1],
                          x + 3 * (int64_t)vid[2], x + 3 * (int64_t)vid[3], p->kq, &e, gl, Hl);
        E += e;
        if (scatter(row_ptr, col_idx, 4, vid, gl, Hl, g, hvals)) return -3;
    }
    *energy = E;
    return 0;
}

int oracle_bsr_spmv(int32_t nv, const int32_t *row_ptr, const int32_t *col_idx,
                    const double *hvals, const double *v, double *y)
{
    if (nv < 0 || !row_ptr || !col_idx || !hvals || !v || !y) return -1;
    for (int32_t a = 0; a < nv; ++a) {
        double acc[3] = {0.0, 0.0, 0.0};
        for (int64_t k = row_ptr[a]; k < row_ptr[a + 1]; ++k) {
            const double *B = hvals + 9 * k;
            const double *vb = v + 3 * (int64_t)col_idx[k];
            for (int r = 0; r < 3; ++r)
                acc[r] += B[3 * r] * vb[0] + B[3 * r + 1] * vb[1] + B[3 * r + 2] * vb[2];
        }
        for (int r = 0; r < 3; ++r) y[3 * (int64_t)a + r] = acc[r];
    }
    return 0;
}

int oracle_hvp(const oracle_problem *p, const int32_t *row_ptr,
               const int32_t *col_idx, const double *x, const double *v,
               double *y)
{
    if (check_problem(p) || !row_ptr || !col_idx || !x || !v || !y) return -1;
    int64_t nnzb = row_ptr[p->nv];
    double *g = (double *)malloc(3 * (size_t)(p->nv > 0 ? p->nv : 1) * sizeof(double));
    double *hv = (double *)malloc(9 * (size_t)(nnzb > 0 ? nnzb : 1) * sizeof(double));
    if (!g || !hv) { free(g); free(hv); return -2; }
    double E;
    int rc = oracle_eval(p, row_ptr, col_idx, x, &E, g, hv);
    if (rc == 0) rc = oracle_bsr_spmv(p->nv, row_ptr, col_idx, hv, v, y);
    free(g);
    free(hv);
    return rc;
}
