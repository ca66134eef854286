/*
 * Host-only exercise of the CPU oracle (oracle/oracle.c) for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: a small grid carrying
 * every term kind (springs, inertia, symmetric-Dirichlet and ARAP faces,
 * vertex-vertex pairs, vertex-face contacts, planarity quads) goes through
 * the pattern, the evaluation, the Hessian-vector product and the block
 * SpMV; malformed problems must be rejected with a negative code.  Checks
 * that need no second implementation: every value is finite, H is
 * symmetric, the HVP equals the SpMV of the assembled H.  Prints one line
 * per failed check and exits non-zero if any failed.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int g_fail = 0;
#define CHECK(cond, ...)                              \
    do {                                              \
        if (!(cond)) {                                \
            ++g_fail;                                 \
            printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            printf(__VA_ARGS__);                      \
            printf("\n");                             \
        }                                             \
    } while (0)

static unsigned long long g_state = 88172645463325252ull;
static double urand(void) /* xorshift64, in [0, 1) */
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (double)(g_state >> 11) / 9007199254740992.0;
}

enum { N = 6, NV = N * N };

static int32_t vid(int i, int j) { return i * N + j; }

static int finite_all(const double *a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int64_t find_blk(const int32_t *rp, const int32_t *ci, int32_t a, int32_t b)
{
    for (int32_t k = rp[a]; k < rp[a + 1]; ++k)
        if (ci[k] == b) return k;
    return -1;
}

static void run(int face_energy)
{
    const double h = 1.0 / (N - 1);
    double X[3 * NV], x[3 * NV], xt[3 * NV];
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            const int32_t v = vid(i, j);
            X[3 * v] = j * h;
            X[3 * v + 1] = i * h;
            X[3 * v + 2] = 0.0;
        }
    for (int k = 0; k < 3 * NV; ++k) {
        x[k] = X[k] + 0.05 * h * (urand() - 0.5);
        xt[k] = X[k] + 0.02 * h * (urand() - 0.5);
    }
    int32_t faces[2 * (N - 1) * (N - 1) * 3];
    int32_t nf = 0;
    for (int i = 0; i + 1 < N; ++i)
        for (int j = 0; j + 1 < N; ++j) {
            const int32_t a = vid(i, j), b = vid(i, j + 1), c = vid(i + 1, j), d = vid(i + 1, j + 1);
            faces[3 * nf] = a, faces[3 * nf + 1] = b, faces[3 * nf + 2] = d, ++nf;
            faces[3 * nf] = a, faces[3 * nf + 1] = d, faces[3 * nf + 2] = c, ++nf;
        }
    double dm_inv[4 * 2 * (N - 1) * (N - 1)], area[2 * (N - 1) * (N - 1)];
    for (int32_t f = 0; f < nf; ++f) {
        const double *p0 = X + 3 * faces[3 * f], *p1 = X + 3 * faces[3 * f + 1],
                     *p2 = X + 3 * faces[3 * f + 2];
        const double e00 = p1[0] - p0[0], e10 = p1[1] - p0[1];
        const double e01 = p2[0] - p0[0], e11 = p2[1] - p0[1];
        const double det = e00 * e11 - e01 * e10;
        dm_inv[4 * f] = e11 / det;
        dm_inv[4 * f + 1] = -e01 / det;
        dm_inv[4 * f + 2] = -e10 / det;
        dm_inv[4 * f + 3] = e00 / det;
        area[f] = 0.5 * fabs(det);
    }
    int32_t springs[2 * 2 * N * (N - 1)];
    double rest[2 * N * (N - 1)];
    int32_t ns = 0;
    for (int i = 0; i < N; ++i)
        for (int j = 0; j + 1 < N; ++j) {
            springs[2 * ns] = vid(i, j), springs[2 * ns + 1] = vid(i, j + 1), rest[ns] = h, ++ns;
            springs[2 * ns] = vid(j, i), springs[2 * ns + 1] = vid(j + 1, i), rest[ns] = h, ++ns;
        }
    const int32_t pairs[] = {vid(0, 0), vid(3, 3), vid(5, 1), vid(2, 4)};
    const int32_t vf[] = {vid(0, 5), 12, vid(5, 5), 3};
    const int32_t quads[] = {vid(1, 1), vid(1, 2), vid(2, 1), vid(2, 2)};
    oracle_problem p;
    memset(&p, 0, sizeof(p));
    p.nv = NV;
    p.nf = nf;
    p.faces = faces;
    p.ns = ns;
    p.springs = springs;
    p.rest_len = rest;
    p.k = 100.0;
    p.inertia = 1;
    p.c = 10.0;
    p.x_tilde = xt;
    p.face_energy = face_energy;
    p.dm_inv = dm_inv;
    p.area = area;
    p.np = 2;
    p.pairs = pairs;
    p.kappa = 1.0;
    p.dhat = 4.0; /* every pair and contact within the barrier's support */
    p.nvf = 2;
    p.vf = vf;
    p.nq = 1;
    p.quads = quads;
    p.kq = 5.0;

    const int64_t nnzb = oracle_pattern_nnzb(&p);
    CHECK(nnzb > NV, "face_energy %d: nnzb %lld", face_energy, (long long)nnzb);
    if (nnzb <= 0) return;
    int32_t *rp = malloc(sizeof(int32_t) * (NV + 1));
    int32_t *ci = malloc(sizeof(int32_t) * (size_t)nnzb);
    double *hv = malloc(sizeof(double) * 9 * (size_t)nnzb);
    double g[3 * NV], v[3 * NV], y1[3 * NV], y2[3 * NV], E = 0.0;
    CHECK(oracle_pattern(&p, rp, ci) == 0, "pattern");
    CHECK(rp[0] == 0 && rp[NV] == nnzb, "row_ptr ends");
    for (int32_t a = 0; a < NV; ++a)
        for (int32_t k = rp[a] + 1; k < rp[a + 1]; ++k) CHECK(ci[k - 1] < ci[k], "row %d sorted", a);
    CHECK(oracle_eval(&p, rp, ci, x, &E, g, hv) == 0, "eval");
    CHECK(isfinite(E) && finite_all(g, 3 * NV) && finite_all(hv, 9 * nnzb), "finite values");
    for (int32_t a = 0; a < NV; ++a)
        for (int32_t k = rp[a]; k < rp[a + 1]; ++k) {
            const int64_t kt = find_blk(rp, ci, ci[k], a);
            CHECK(kt >= 0, "transpose block of (%d, %d)", a, ci[k]);
            if (kt < 0) continue;
            for (int r = 0; r < 3; ++r)
                for (int c = 0; c < 3; ++c) {
                    const double u = hv[9 * k + 3 * r + c], w = hv[9 * kt + 3 * c + r];
                    CHECK(fabs(u - w) <= 1e-9 * (1.0 + fabs(u)), "H symmetric at (%d, %d)", a, ci[k]);
                }
        }
    for (int k = 0; k < 3 * NV; ++k) v[k] = urand() - 0.5;
    CHECK(oracle_hvp(&p, rp, ci, x, v, y1) == 0, "hvp");
    CHECK(oracle_bsr_spmv(NV, rp, ci, hv, v, y2) == 0, "spmv");
    double num = 0.0, den = 0.0;
    for (int k = 0; k < 3 * NV; ++k) {
        num += (y1[k] - y2[k]) * (y1[k] - y2[k]);
        den += y2[k] * y2[k];
    }
    CHECK(sqrt(num) <= 1e-12 * sqrt(den), "HVP against SpMV: %g", sqrt(num / den));

    /* malformed problems: rejected, nothing written out of bounds */
    oracle_problem bad = p;
    int32_t badf[2 * (N - 1) * (N - 1) * 3];
    memcpy(badf, faces, sizeof(int32_t) * 3 * (size_t)nf);
    badf[7] = NV;
    bad.faces = badf;
    CHECK(oracle_pattern_nnzb(&bad) < 0, "face index out of range accepted");
    bad = p;
    const int32_t badpair[] = {0, 0, 1, 2};
    bad.pairs = badpair;
    CHECK(oracle_pattern_nnzb(&bad) < 0, "pair (i, i) accepted");
    bad = p;
    int32_t bads[2 * 2 * N * (N - 1)];
    memcpy(bads, springs, sizeof(int32_t) * 2 * (size_t)ns);
    bads[3] = bads[2];
    bad.springs = bads;
    CHECK(oracle_pattern_nnzb(&bad) < 0, "spring (i, i) accepted");
    bad = p;
    const int32_t badvf[] = {faces[0], 0, 1, 2};
    bad.vf = badvf;
    CHECK(oracle_pattern_nnzb(&bad) < 0, "contact with its own face accepted");
    bad = p;
    bad.nv = -1;
    CHECK(oracle_pattern_nnzb(&bad) < 0, "negative nv accepted");
    free(rp);
    free(ci);
    free(hv);
}

int main(void)
{
    run(1);
    run(2);
    if (g_fail) {
        printf("%d checks failed\n", g_fail);
        return 1;
    }
    printf("all oracle checks passed\n");
    return 0;
}
