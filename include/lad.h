/*
 * lad.h -- locality-aware per-element automatic differentiation of mesh
 * energies on AMD Instinct MI355X (gfx950): the C ABI of liblad.so.
 *
 * The library evaluates a partially separable objective
 *     F(x) = sum_j f_j(x_j)
 * over a triangle mesh, differentiates every local term j in forward mode
 * (second-order dual numbers in registers), and assembles on the GPU
 *     g = sum_j S_j^T g_j         (global gradient)
 *     H = sum_j S_j^T H_j S_j     (3x3-block CSR Hessian)
 * together with a matrix-free Hessian-vector product and double-buffered
 * insertion of runtime vertex-vertex contact pairs.
 * Source: page "Locality-Aware Automatic Differentiation on the GPU for
 * Mesh-Based Computations" (Mahmoud, Goel, Ragan-Kelley, Solomon), section
 * "Method" and its key designs 1-4.
 *
 * Terms supported (each switched on in lad_mesh_desc):
 *   spring   0.5 k (|x_a - x_b| - L_s)^2                 per spring s=(a,b)
 *   inertia  0.5 c |x_v - xt_v|^2                          per vertex v
 *   face     A_f (tr C + tr C / det C),  C = F^T F,        per triangle f
 *            F = [x1 - x0, x2 - x0] Dm_f^{-1}  (symmetric Dirichlet)
 *   pair     -kappa (d - dhat)^2 ln(d / dhat) for d < dhat, else 0,
 *            d = |x_i - x_j|                               per inserted pair
 *
 * Data layout (all device arrays are caller-owned unless stated):
 *   x, v, g, y : [nv][3] of the context dtype (float or double), DOF 3v+c.
 *   hvals      : [capacity][3][3] of the dtype; block k of the active pattern
 *                holds d2F / dx_{row,r} dx_{col_idx[k],c} at 9k + 3r + c.
 *   pattern    : row_ptr int32 [nv+1], col_idx int32 [nnzb]; rows are
 *                vertices, columns ascending, full symmetric storage, the
 *                diagonal block always present.  Row a holds {a}, every
 *                vertex sharing a face or a spring with a, and a's current
 *                pair partners.
 *
 * Errors: every call returns lad_status; nothing throws across the ABI.
 * Arguments are checked on the host before anything is enqueued; a failed
 * call enqueues nothing and leaves outputs and the pattern untouched.  Pair
 * indices live on the device and are checked there: a bad pair set leaves
 * the previous pattern active and is reported by lad_device_status.
 *
 * Streams: every call enqueues on the caller's HIP stream (hipStream_t passed
 * as void*; NULL is the null stream).  lad_eval_energy_grad_hess (and its
 * _noalloc variant), lad_hvp and lad_insert_pairs never synchronise with
 * the host.  lad_build_pattern,
 * lad_get_pattern, lad_get_info and lad_device_status synchronise that stream.
 *
 * Threading: one context must not be used by two host threads at once.
 */
#ifndef LAD_H
#define LAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lad_ctx lad_ctx;

typedef enum {
    LAD_OK = 0,
    LAD_ERR_ARG = -1,       /* bad argument (null pointer, size, index)     */
    LAD_ERR_CAPACITY = -2,  /* more pairs or blocks than reserved storage   */
    LAD_ERR_OOM = -3,       /* device or host allocation failed             */
    LAD_ERR_HIP = -4,       /* a HIP runtime call failed                     */
    LAD_ERR_STATE = -5,     /* call not valid in the context's state        */
    LAD_ERR_PAIRS = -6,     /* device-side check rejected a pair set        */
    LAD_ERR_NONFINITE = -7  /* debug check: an output held a NaN or an inf  */
} lad_status;

typedef enum { LAD_F32 = 0, LAD_F64 = 1 } lad_dtype;

/* Mesh and energy terms.  All pointers are HOST pointers, read during
 * lad_build_pattern and not retained (the library copies what it needs).
 * Per-element constants are given in fp64 and rounded once to the dtype. */
typedef struct {
    int32_t nv;                 /* vertices, >= 1                              */
    int32_t nf;                 /* triangles, >= 0                             */
    const int32_t *faces;       /* [nf][3] vertex ids (counter-clockwise)      */

    lad_dtype dtype;            /* arithmetic and storage type of x, g, H, v, y */
    int32_t deterministic;      /* 1: bitwise reproducible run to run required */
                                /*    (every path but the two atomic patch      */
                                /*    assemblies is; those reject it)           */
    int32_t patch_lds_bytes;    /* LDS budget per patch; 0 = library default    */
    int32_t pair_capacity;      /* max pairs per lad_insert_pairs, >= 0         */

    int32_t ns;                 /* springs, >= 0 (0 = no spring term)          */
    const int32_t *springs;     /* [ns][2] vertex ids, a != b                  */
    const double *rest_len;     /* [ns] rest lengths L_s                       */
    double k;                   /* spring stiffness                            */

    int32_t inertia;            /* 1 = inertia term on every vertex            */
    double c;                   /* inertia weight (mass / dt^2)                */
    const double *x_tilde;      /* [nv][3] inertial target positions           */

    int32_t face_energy;        /* 1 = symmetric-Dirichlet term on every face  */
    const double *dm_inv;       /* [nf][4] row-major 2x2 inverse rest edge matrix */
    const double *area;         /* [nf] rest areas                              */

    double kappa;               /* pair barrier stiffness                      */
    double dhat;                /* pair barrier support, > 0 if pair_capacity>0 */

    int32_t eval_path;          /* LAD_PATH_AUTO, LAD_PATH_PATCH, LAD_PATH_ROWS,
                                   LAD_PATH_PATCH_ATOMIC or
                                   LAD_PATH_PATCH_LDS_ATOMIC                  */
    int32_t vf_capacity;        /* max vertex-face contacts per
                                   lad_insert_contacts, >= 0; > 0 needs faces
                                   (nf > 0) and the row path                  */
} lad_mesh_desc;

/* Parallel decomposition of the evaluation and HVP kernels.
 *  LAD_PATH_PATCH  element owner: one workgroup per patch of contiguous rows;
 *                  every element touching an owned row is evaluated once per
 *                  such patch and scattered into the patch's rows, which are
 *                  accumulated in LDS and streamed out.  The scatter runs in
 *                  colour phases (no two elements of a phase share an owned
 *                  vertex): plain LDS adds in a fixed order, bitwise
 *                  reproducible.  Any mix of terms.
 *  LAD_PATH_ROWS   row owner: one lane per block row evaluates every term of
 *                  that row; each block is written once, in a fixed order,
 *                  without atomics.  Requires rest lengths >= 0, at most one
 *                  spring per vertex pair and, with face terms, rows shorter
 *                  than 256 blocks.
 *  LAD_PATH_AUTO   LAD_PATH_ROWS when its requirements hold, else PATCH.
 *  LAD_PATH_PATCH_ATOMIC  the page's own assembly: each element is evaluated
 *                  once, by the patch owning its lowest vertex id; its
 *                  blocks and gradient entries in other patches' rows are
 *                  added with global float atomics into slots that a small
 *                  launch zeroes first (Source: page "Locality-Aware
 *                  Automatic Differentiation on the GPU for Mesh-Based
 *                  Computations", key designs 3 and 4: atomic scatter-add
 *                  into the preallocated pattern).  Results vary in the last
 *                  bits from run to run.  Takes no deterministic mode and no
 *                  contact capacity (LAD_ERR_ARG otherwise).
 *  LAD_PATH_PATCH_LDS_ATOMIC  LAD_PATH_PATCH with the scatter into LDS done
 *                  by LDS float atomics instead of colour phases (the page's
 *                  patch-local accumulation, key design 3); results vary in
 *                  the last bits.  Takes no deterministic mode.  */
enum {
    LAD_PATH_AUTO = 0,
    LAD_PATH_PATCH = 1,
    LAD_PATH_ROWS = 2,
    LAD_PATH_PATCH_ATOMIC = 3,
    LAD_PATH_PATCH_LDS_ATOMIC = 4
};

/* Summary of a context (lad_get_info synchronises the context's stream to
 * read the device-side active pattern size). */
typedef struct {
    int32_t nv;
    int32_t dtype;
    int64_t nnzb_base;          /* blocks of the topology pattern              */
    int64_t nnzb_active;        /* blocks of the active pattern (base + pairs) */
    int64_t hvals_capacity;     /* blocks an hvals buffer must hold            */
    int32_t npairs_active;
    int32_t npatches;           /* patches, or row chunks on the row path      */
    int32_t lds_bytes_eval;     /* dynamic LDS of the eval kernel per workgroup */
    int32_t lds_bytes_hvp;
    int64_t spring_records;     /* element records incl. patch-boundary copies */
    int64_t face_records;
    int32_t max_colors;         /* colour phases of the patch path's assembly  */
    int32_t active_buffer;      /* 0 = topology pattern, 1/2 = pair buffers    */
    int32_t eval_path;          /* the LAD_PATH_* decomposition in use         */
    int32_t grid_eval;          /* workgroups of one evaluation launch         */
    int64_t host_syncs;         /* host synchronisations made so far for this
                                   context, this lad_get_info call included;
                                   lad_eval_energy_grad_hess, lad_hvp and
                                   lad_insert_pairs never add to it          */
    int32_t nvf_active;         /* vertex-face contacts of the active pattern  */
    int32_t pad0;
    double pattern_ms;          /* GPU time of the topology pattern's build in
                                   lad_build_pattern (count, scan, fill, sort
                                   and de-duplication, compaction), from HIP
                                   events around those launches              */
} lad_info;

/*
 * Build a context: validate the mesh, derive the block pattern on the GPU
 * (parallel row count, wave/LDS prefix scan, fill, per-row sort and
 * de-duplication), split the vertices into LDS-sized patches on the host,
 * and upload the per-patch element records.  Source: key design 2 (patches
 * with ribbon vertices staged in on-chip memory) and key design 3 (pattern
 * preallocated at initialisation from the topology with a prefix sum).
 * Synchronises `hip_stream`.  On success *out owns device memory until
 * lad_destroy.  Errors: LAD_ERR_ARG (bad sizes, null arrays for enabled
 * terms, vertex ids out of range, a spring with a == b, nnzb*9 >= 2^31),
 * LAD_ERR_OOM, LAD_ERR_HIP.
 */
lad_status lad_build_pattern(const lad_mesh_desc *desc, void *hip_stream,
                             lad_ctx **out);

/* Read the context summary.  Synchronises the context's build stream. */
lad_status lad_get_info(lad_ctx *ctx, lad_info *info);

/*
 * Active pattern: *nnzb gets its block count; *d_row_ptr and *d_col_idx get
 * library-owned DEVICE pointers, valid until the next lad_insert_pairs or
 * lad_destroy.  This is the pattern the values of lad_eval_energy_grad_hess
 * are laid out in: the block CSR preallocated from the topology (with the
 * current contacts merged in), which a caller hands on to a solver.
 * Source: key design 3 (sparsity pattern preallocated at initialisation,
 * derivatives written straight into it) and key design 4 (the active one
 * of the two pattern buffers).  Synchronises `hip_stream` (which must be
 * the stream the context's calls run on, so that pending inserts are
 * complete).  Errors: LAD_ERR_ARG (NULL argument), LAD_ERR_HIP.
 */
lad_status lad_get_pattern(lad_ctx *ctx, void *hip_stream, int64_t *nnzb,
                           const int32_t **d_row_ptr, const int32_t **d_col_idx);

/*
 * Copy the active pattern into caller-owned DEVICE buffers: d_row_ptr gets
 * nv+1 entries, d_col_idx gets nnzb entries (*nnzb, which must not exceed
 * col_capacity).  Source: key design 3 (the preallocated block CSR handed
 * to the caller) and key design 4 (the active pattern buffer).
 * Synchronises `hip_stream` to read the active buffer, then copies on it
 * and synchronises again.  Errors: LAD_ERR_ARG (NULL pointer),
 * LAD_ERR_CAPACITY (col_capacity < nnzb; nothing copied), LAD_ERR_HIP.
 */
lad_status lad_copy_pattern(lad_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                            int32_t *d_col_idx, int64_t col_capacity, int64_t *nnzb);

/*
 * Energy, gradient and block-CSR Hessian at positions d_x.
 * Source: section "Method" (g = sum S_j^T g_j, H = sum S_j^T H_j S_j) and
 * key design 1 (per-element forward mode; global traffic is one read of the
 * mesh and one write of the derivatives).
 *   d_x      device [nv][3] dtype, read only.
 *   d_energy device double, overwritten with F(x); or NULL, in which case the
 *            energy is not summed (one small kernel launch is saved: the
 *            evaluation itself is then a single launch on the row path,
 *            two with pair capacity, three with vertex-face capacity: the
 *            contact terms, the untouched rows, the rows contacts touch).
 *   d_grad   device [nv][3] dtype, fully overwritten.
 *   d_hvals  device [hvals_capacity][3][3] dtype; the first nnzb_active
 *            blocks are fully overwritten in the active pattern's order.
 *   hvals_capacity_blocks must be >= lad_info.hvals_capacity.
 * Asynchronous on `hip_stream`; no host synchronisation.  Outputs must not
 * alias inputs.  Calls on one context must be ordered (one stream, or
 * streams synchronised by the caller): they share per-context scratch.
 * Errors: LAD_ERR_ARG (null x, grad or hvals; capacity too small).
 */
lad_status lad_eval_energy_grad_hess(lad_ctx *ctx, const void *d_x,
                                     double *d_energy, void *d_grad,
                                     void *d_hvals, int64_t hvals_capacity_blocks,
                                     void *hip_stream);

/*
 * lad_eval_energy_grad_hess for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  The same kernels and the same results, bit for bit; the
 * per-workgroup partial energies (the evaluation's only scratch) go to a
 * static device array of the library instead of the context's buffer.  The
 * call makes no hipMalloc, hipFree or other allocation; its first call on a
 * device looks up that device's copy of the array.
 *   Arguments, layout and ownership as lad_eval_energy_grad_hess.  The
 *   context's device must be the current device.
 *   Limit: at most 32768 partial energies (256 KiB): one per workgroup of
 *   the evaluation's launches, about 2,100 for a row-path context on MI355X
 *   (plus one per 256 contact incidence entries), one per patch on the patch
 *   path.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (two streams, two host threads,
 * two processes' contexts do not share it) race and may return a wrong
 * energy.  Order them on one stream.  No slot is read before the call
 * writes it, so nothing needs clearing between calls.
 * Errors: as lad_eval_energy_grad_hess, plus LAD_ERR_CAPACITY (more partial
 * energies than the array holds), LAD_ERR_STATE (vertex-face capacity, whose
 * per-contact strips are context scratch; or another device current),
 * LAD_ERR_HIP.  Nothing is enqueued on error.
 */
lad_status lad_eval_energy_grad_hess_noalloc(lad_ctx *ctx, const void *d_x,
                                             double *d_energy, void *d_grad,
                                             void *d_hvals, int64_t hvals_capacity_blocks,
                                             void *hip_stream);

/*
 * Matrix-free Hessian-vector product y = H(x) v, H never stored.
 * Source: section "Method" (matrix-free operations on the assembled
 * derivatives) and the parameterisation application in "Results".
 *   d_x, d_v device [nv][3] dtype, read only; d_y device [nv][3] dtype,
 *   fully overwritten.  Asynchronous; no host synchronisation.
 */
lad_status lad_hvp(lad_ctx *ctx, const void *d_x, const void *d_v, void *d_y,
                   void *hip_stream);

/*
 * Vector objective: the least-squares form of the spring and inertia terms,
 *   R_s           = sqrt(k) (|x_a - x_b| - L_s)   rows 0 .. ns-1, springs in
 *                                                  the order of the desc
 *   R_(ns+3v+c)   = sqrt(c) (x_v - xt_v)_c        rows ns .. ns+3nv-1
 *                                                  (inertia on)
 * so that 0.5 |R|^2 is the spring + inertia energy, and its sparse Jacobian
 * J = dR/dx = sum_j P_j^T J_j S_j.  Source: page "Locality-Aware Automatic
 * Differentiation on the GPU for Mesh-Based Computations", section "Method"
 * (vector objectives assemble a sparse Jacobian; local Jacobians by forward
 * mode) and its closing discussion (materialising J explicitly pays off).
 * Available on contexts without face terms and without pair capacity (those
 * energies are not sums of squares): other contexts get LAD_ERR_STATE.
 *
 * Jacobian pattern: CSR, nrows = ns (+ 3 nv) rows, 3 nv columns (DOF 3v+c),
 * nnz = 6 ns (+ 3 nv).  Spring row s holds its two vertices' six DOFs in
 * ascending order at entries 6s .. 6s+5; inertia row ns+i holds DOF i at
 * entry 6 ns + i.  *d_row_ptr and *d_col_idx get library-owned DEVICE
 * pointers valid until lad_destroy; the first call allocates and builds
 * them on the GPU and synchronises `hip_stream`.  Errors: LAD_ERR_ARG,
 * LAD_ERR_STATE (see above, or nnz >= 2^31), LAD_ERR_OOM, LAD_ERR_HIP.
 */
lad_status lad_jacobian_pattern(lad_ctx *ctx, void *hip_stream, int64_t *nrows, int64_t *nnz,
                                const int32_t **d_row_ptr, const int32_t **d_col_idx);

/*
 * Copy the Jacobian pattern into caller-owned DEVICE buffers: d_row_ptr
 * gets nrows+1 entries, d_col_idx gets nnz entries (*nnz, which must not
 * exceed col_capacity).  Builds the pattern first if needed; copies on
 * `hip_stream` and synchronises it.  Errors: as lad_jacobian_pattern, plus
 * LAD_ERR_CAPACITY (col_capacity < nnz; nothing copied).
 */
lad_status lad_copy_jacobian_pattern(lad_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                                     int32_t *d_col_idx, int64_t col_capacity, int64_t *nnz);

/*
 * Residuals and Jacobian values at d_x: d_r device [nrows] dtype and
 * d_jvals device [nnz] dtype, both fully overwritten, the values in the
 * pattern's order (the pattern itself need not have been requested).
 * Asynchronous; no host synchronisation.  Errors: LAD_ERR_ARG,
 * LAD_ERR_STATE, LAD_ERR_HIP.
 */
lad_status lad_residual_jacobian(lad_ctx *ctx, const void *d_x, void *d_r, void *d_jvals,
                                 void *hip_stream);

/*
 * Gauss-Newton product y = J^T (J v) at d_x, matrix-free (J is formed per
 * term in registers and never stored); the positive semi-definite
 * counterpart of lad_hvp for the same spring + inertia energy.  d_x, d_v
 * device [nv][3] dtype, read only; d_y device [nv][3], fully overwritten.
 * Needs the row path (lad_info.eval_path == LAD_PATH_ROWS).  Asynchronous;
 * no host synchronisation.  Errors: LAD_ERR_ARG, LAD_ERR_STATE, LAD_ERR_HIP.
 */
lad_status lad_gauss_newton_product(lad_ctx *ctx, const void *d_x, const void *d_v, void *d_y,
                                    void *hip_stream);

/* Why a Newton-CG solve ended (lad_cg_stats.reason). */
enum { LAD_CG_CONVERGED = 0, LAD_CG_NEG_CURVATURE = 1, LAD_CG_MAX_ITERS = 2 };

typedef struct {
    int32_t iterations;   /* completed CG updates                                */
    int32_t reason;       /* LAD_CG_CONVERGED, LAD_CG_NEG_CURVATURE or
                             LAD_CG_MAX_ITERS                                    */
    double rel_residual;  /* |r| / |g| of the last residual (r = H p + g for the
                             returned p, except after a first-step negative
                             curvature exit, where p = -g and this is 1)      */
    double grad_norm;     /* |g|                                                 */
} lad_cg_stats;

/*
 * Newton direction by truncated conjugate gradients on the matrix-free HVP:
 * approximately solves H(x) p = -g from p = 0 (line-search Newton-CG,
 * Nocedal and Wright, Numerical Optimization, 2nd ed., Algorithm 7.1).
 * Stops when |r| < eps (r = H p + g), returning p; at the first CG
 * direction d with d.H d <= 0, returning -g if that is the first direction
 * and the current p otherwise (a descent direction either way); or after
 * max_iters updates, returning the current p.  eps = eta |g| for eta > 0,
 * else min(0.5, sqrt|g|) |g| (that algorithm's forcing term).  The page
 * "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
 * Computations" presents fast Hessian-vector products as what makes such
 * Newton-type methods practical on large meshes; it fixes no solver.
 *   d_x, d_g  device [nv][3] dtype, read only (g is usually the gradient
 *             from lad_eval_energy_grad_hess at the same x).
 *   d_p       device [nv][3] dtype, fully overwritten; must not alias d_g.
 *   max_iters >= 0; stats: host pointer, or NULL.
 * Dot products are accumulated in fp64 in a fixed order (bitwise
 * reproducible); vector updates are computed in fp64 and rounded to the
 * dtype.  The first call allocates per-context work vectors (up to four
 * [nv][3] arrays and a few KB), kept until lad_destroy.  Synchronises `hip_stream`
 * after every 16 iterations (to stop early) and at the end.  Errors:
 * LAD_ERR_ARG (NULL x, g or p, p == g, max_iters < 0), LAD_ERR_OOM,
 * LAD_ERR_HIP.
 */
lad_status lad_newton_cg(lad_ctx *ctx, const void *d_x, const void *d_g, void *d_p,
                         int32_t max_iters, double eta, lad_cg_stats *stats,
                         void *hip_stream);

/*
 * Replace the runtime contacts: vertex-vertex pairs (barrier of |x_i - x_j|,
 * as lad_insert_pairs) and vertex-face contacts (v, face f) with the same
 * barrier applied to the distance from x_v to the triangle f; the region of
 * the triangle's closest point (vertex, edge interior, face interior) is
 * decided at the positions of each evaluation and d is that region's smooth
 * formula.  The next pattern is topology U {(i,j),(j,i)} for every pair
 * U {(v,t),(t,v) for t in f} for every contact, sorted and de-duplicated;
 * the previous contacts are dropped.  Source: key design 4 (runtime
 * vertex-vertex and vertex-face interactions, double-buffered CSR).
 *   d_pairs  device int32 [npairs][2], 0 <= npairs <= pair_capacity.
 *   d_vf     device int32 [nvf][2] of (vertex, face id), 0 <= nvf <=
 *            vf_capacity; the vertex must not belong to the face.
 * npairs = nvf = 0 restores the topology pattern.  Errors and device-side
 * checks as lad_insert_pairs (LAD_ERR_CAPACITY for either count).
 * Asynchronous.
 */
lad_status lad_insert_contacts(lad_ctx *ctx, const int32_t *d_pairs, int32_t npairs,
                               const int32_t *d_vf, int32_t nvf, void *hip_stream);

/*
 * Replace the runtime vertex-vertex pairs (and drop any vertex-face
 * contacts): the next pattern is
 * topology U {(i,j),(j,i) for every pair}, sorted and de-duplicated; the
 * previous pairs are dropped.  Built on the GPU into the inactive one of two
 * reserved pattern buffers, then made active by a device-side swap (no host
 * round trip).  Source: key design 4 (decoupled discovery and evaluation,
 * double-buffered CSR with reserved storage).
 *   d_pairs  device int32 [npairs][2]; read during the call's kernels only.
 *   npairs   0 <= npairs <= pair_capacity (0 restores the topology pattern).
 * Host errors: LAD_ERR_ARG, LAD_ERR_CAPACITY (npairs > pair_capacity); the
 * pattern is then unchanged.  Device-side checks (index out of range, i == j,
 * staging capacity exceeded, see below) keep the previous pattern and pairs
 * active and latch an error readable with lad_device_status
 * (LAD_ERR_PAIRS for a bad index, LAD_ERR_CAPACITY for staging).
 * Staging capacity: the evaluation stages a group of rows' blocks on chip,
 * so inserted blocks are limited per group as well as in total.  Row path:
 * each chunk of up to 64 consecutive rows (lad_info.npatches chunks) holds
 * at most 512 blocks, topology and inserted together; a chunk of the grid
 * cloths has at most 448 topology blocks, so it takes at least 64 inserted
 * blocks (one per pair endpoint whose partner is new to its row, three for
 * a contact vertex, one per face vertex of a contact).  Patch path: each
 * patch takes max(32, 1/8 of its topology blocks) inserted blocks.
 * Asynchronous; hvals buffers sized to lad_info.hvals_capacity stay valid.
 */
lad_status lad_insert_pairs(lad_ctx *ctx, const int32_t *d_pairs, int32_t npairs,
                            void *hip_stream);

/*
 * Read and clear the device-side error latch set by lad_insert_pairs and
 * lad_insert_contacts and, in debug mode, by the output checks.  *status
 * gets LAD_OK, LAD_ERR_PAIRS (a bad index), LAD_ERR_CAPACITY (staging),
 * LAD_ERR_STATE (an insert whose workgroups did not complete their chain:
 * an internal failure, the insert was not committed) or LAD_ERR_NONFINITE
 * (debug mode), the first of these that applies.  Synchronises
 * `hip_stream`.
 */
lad_status lad_device_status(lad_ctx *ctx, void *hip_stream, int32_t *status);

/*
 * Debug mode, for callers hunting a NaN or an inf.  flags = LAD_DEBUG_NONFINITE
 * makes every later lad_eval_energy_grad_hess (and _noalloc) check its
 * energy, gradient and the active pattern's Hessian blocks, and every
 * lad_hvp its product, on the device after the call's kernels, on the same
 * stream: a value that is not finite latches an error that
 * lad_device_status reports as LAD_ERR_NONFINITE (the calls themselves stay
 * asynchronous and make no host synchronisation; each check reads its
 * outputs once more).  flags = 0 turns it off.  Errors: LAD_ERR_ARG (NULL
 * ctx, unknown flag).  Makes no GPU call.
 */
#define LAD_DEBUG_NONFINITE 1
lad_status lad_set_debug(lad_ctx *ctx, int32_t flags);

/* Message for the last host-side error of this context ("" if none).  The
 * string is owned by the context.  With ctx == NULL: the last error of a
 * failed lad_build_pattern in this thread. */
const char *lad_last_error(const lad_ctx *ctx);

/* Static name of a status code. */
const char *lad_status_string(lad_status s);

/* Release the context and its device memory (synchronises the device).
 * NULL is a no-op.  The pointer is invalid afterwards. */
void lad_destroy(lad_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* LAD_H */
