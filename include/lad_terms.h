/*
 * lad_terms.h -- the term front end of liblad.so: energies given as lists
 * of user terms, each a local energy over a fixed stencil of 1 to 4
 * vertices, compiled into the library as term sets.
 *
 * Source: page "Locality-Aware Automatic Differentiation on the GPU for
 * Mesh-Based Computations", section "Method": the user writes only local
 * energy terms defined on vertices, edges, faces or their neighbourhoods;
 * the system analyses each term's stencil, dimension and derivative needs,
 * preallocates the block-CSR pattern from the topology, evaluates and
 * differentiates every term in forward mode, and assembles
 *     g = sum_j S_j^T g_j,   H = sum_j S_j^T H_j S_j,
 * or applies H without storing it.  A term is a C++ struct with its arity
 * and constant count fixed at compile time and its energy written once as
 * a template over the number type (see the package's csrc/user_terms.h);
 * a set is a compile-time list of such terms (csrc/lad_terms.hip), and all
 * terms of a set are evaluated in one fused pass unless the caller asks
 * for one launch per term.
 *
 * Sets compiled into the library (per-element constants in brackets):
 *   LAD_TERMS_CLOTH       spring: 2 vertices, 0.5 k (|x0 - x1| - L)^2
 *                           [L, k];
 *                         inertia: 1 vertex, 0.5 c |x - xt|^2
 *                           [xt_x, xt_y, xt_z, c]
 *   LAD_TERMS_ARAP        arap_face: 3 vertices, A sum_i (sigma_i - 1)^2
 *                           over the singular values of
 *                           F = [x1 - x0, x2 - x0] Dm^-1 (3 x 2)
 *                           [Dm^-1 row-major (4), rest area A]
 *   LAD_TERMS_SYMDIR      symmetric_dirichlet_face: 3 vertices,
 *                           A (tr C + tr C / det C), C = F^T F  [as arap_face]
 *   LAD_TERMS_ARAP_CLOTH  arap_face, spring, inertia
 *   LAD_TERMS_CLOTH_QUAD  spring, inertia, and
 *                         quad_planarity: 4 vertices,
 *                           0.5 k det[x1 - x0, x2 - x0, x3 - x0]^2  [k]
 *
 * Layout and conventions are those of lad.h: x, v, g, y are [nv][3] of the
 * dtype; H values are [nnzb][3][3] row-major blocks in the pattern's
 * order; the pattern has full symmetric storage, columns ascending, the
 * diagonal always present, and row a holds every vertex that shares an
 * element of any term with a.  Inputs must be finite and no element
 * degenerate for its term (e.g. a zero-area face).
 *
 * Errors: every call returns lad_status (lad.h); arguments are checked on
 * the host before anything is enqueued.  Streams: eval and hvp enqueue on
 * the caller's stream and never synchronise; build synchronises its stream.
 */
#ifndef LAD_TERMS_H
#define LAD_TERMS_H

#include <stdint.h>

#include "lad.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LAD_TERMS_CLOTH = 1,
    LAD_TERMS_ARAP = 2,
    LAD_TERMS_SYMDIR = 3,
    LAD_TERMS_ARAP_CLOTH = 4,
    LAD_TERMS_CLOTH_QUAD = 5
};

/* The elements of one term of a set. */
typedef struct {
    int32_t count;              /* elements, >= 0                               */
    const int32_t *elems;       /* host [count][arity] vertex ids in [0, nv),
                                   distinct within an element                   */
    const double *consts;       /* host [count][nconst], finite (converted to
                                   the dtype); may be NULL when nconst is 0      */
} lad_term_block;

typedef struct {
    int32_t nv;                 /* vertices, >= 1                               */
    int32_t dtype;              /* LAD_F32 or LAD_F64                           */
    int32_t set;                /* LAD_TERMS_*                                  */
    int32_t fused;              /* 1: all terms in one launch (the default
                                   choice); 0: one launch per term, each later
                                   one adding into g and H                      */
    int32_t nblocks;            /* must equal the set's number of terms         */
    const lad_term_block *blocks; /* host [nblocks], in the set's term order    */
} lad_terms_desc;

typedef struct lad_terms_ctx lad_terms_ctx;

/*
 * The terms of a set: *nterms gets their number; for term index `term`
 * (0-based, < *nterms) *arity, *nconst and *name (a static string) get its
 * stencil width, constant count and name.  Any output may be NULL.  Pure
 * host call.  Errors: LAD_ERR_ARG (unknown set, term out of range).
 */
lad_status lad_terms_describe(int32_t set, int32_t term, int32_t *nterms, int32_t *arity,
                              int32_t *nconst, const char **name);

/*
 * Build a context: validate the elements, derive the block pattern on the
 * GPU from every element's vertex pairs (key design 3), plan 64-row chunks,
 * and upload the elements, their constants and each row's incidence list.
 * Synchronises `hip_stream`; on success *out owns device memory until
 * lad_terms_destroy.  Errors: LAD_ERR_ARG (bad sizes or set, nblocks not
 * the set's term count, NULL arrays, a vertex id out of range or repeated
 * within an element, a non-finite constant, a row of more than 256 blocks,
 * nnzb * 9 >= 2^31), LAD_ERR_OOM, LAD_ERR_HIP.
 */
lad_status lad_terms_build(const lad_terms_desc *desc, void *hip_stream, lad_terms_ctx **out);

/*
 * Energy, gradient and block-CSR Hessian of the set's terms at x.
 *   d_x      device [nv][3] dtype.
 *   d_energy device double, overwritten with F(x); or NULL (not summed).
 *   d_grad   device [nv][3] dtype, fully overwritten.
 *   d_hvals  device [hvals_capacity_blocks][3][3] dtype; the first nnzb
 *            blocks are fully overwritten.  Capacity must be >= nnzb.
 * Every value is written by one lane in a fixed order (bitwise
 * reproducible).  Asynchronous.  Errors: LAD_ERR_ARG (NULL x, grad or
 * hvals; capacity too small).
 */
lad_status lad_terms_eval(lad_terms_ctx *ctx, const void *d_x, double *d_energy, void *d_grad,
                          void *d_hvals, int64_t hvals_capacity_blocks, void *hip_stream);

/*
 * y = H(x) v for the set's terms, with H never stored.  d_x, d_v, d_y are
 * device [nv][3] dtype; d_y is fully overwritten and must not alias d_x or
 * d_v.  Asynchronous.  Errors: LAD_ERR_ARG.
 */
lad_status lad_terms_hvp(lad_terms_ctx *ctx, const void *d_x, const void *d_v, void *d_y,
                         void *hip_stream);

/*
 * The pattern: *nnzb gets its block count, *d_row_ptr ([nv+1]) and
 * *d_col_idx ([nnzb]) library-owned DEVICE pointers valid until
 * lad_terms_destroy.  Pure host call.  Errors: LAD_ERR_ARG.
 */
lad_status lad_terms_get_pattern(lad_terms_ctx *ctx, int64_t *nnzb, const int32_t **d_row_ptr,
                                 const int32_t **d_col_idx);

/*
 * Copy the pattern into caller-owned DEVICE buffers (d_row_ptr [nv+1],
 * d_col_idx [nnzb] with nnzb <= col_capacity) on `hip_stream`, then
 * synchronise it; *nnzb gets the block count.  Errors: LAD_ERR_ARG (NULL
 * pointer), LAD_ERR_CAPACITY (col_capacity < nnzb; nothing copied),
 * LAD_ERR_HIP.
 */
lad_status lad_terms_copy_pattern(lad_terms_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                                  int32_t *d_col_idx, int64_t col_capacity, int64_t *nnzb);

/* Message for the last host-side error of this context ("" if none); with
 * ctx == NULL, of the last failed lad_terms_build in this thread. */
const char *lad_terms_last_error(const lad_terms_ctx *ctx);

/* Host synchronisations this context has made so far (the build's, and one
 * per lad_terms_copy_pattern; lad_terms_eval and lad_terms_hvp make none).
 * Returns -1 for ctx == NULL.  Makes no GPU call. */
int64_t lad_terms_host_syncs(const lad_terms_ctx *ctx);

void lad_terms_destroy(lad_terms_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif
