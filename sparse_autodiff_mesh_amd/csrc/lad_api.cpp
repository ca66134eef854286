// lad_api.cpp -- the C ABI of liblad: argument checks, context lifetime and
// the order of kernel launches.  Every argument is checked on the host
// before anything touches the GPU; the per-step calls enqueue on the
// caller's stream and never synchronise.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstring>
#include <string>
#include <vector>

#include "lad_internal.h"
#include "lad_jacobian.h"
#include "lad_solve.h"

#include <algorithm>

using namespace lad;

struct lad_ctx {
    int32_t device = 0;              // HIP device the context was built on
    int32_t nv = 0;
    lad_dtype dtype = LAD_F32;
    int32_t es = 4;
    int32_t mode = kModeLdsAtomic;   // PatchMode of the patch kernels
    hipStream_t stream = nullptr;
    int64_t nnzb_base = 0, hcap = 0;
    int32_t pair_cap = 0;
    int32_t vf_cap = 0;              // vertex-face contact capacity
    int32_t nf = 0;
    double k = 0, c = 0, kappa = 0, dhat = 0;
    int32_t springs_on = 0, faces_on = 0, inertia_on = 0;
    int32_t npatch = 0, lds_eval = 0, lds_hvp = 0, max_colors = 0;
    int32_t row_lds_blocks = kRowLdsBlocks;  // row path: staging blocks per workgroup
    int64_t nspr_rec = 0, nfac_rec = 0;
    int32_t pair_blocks = 0;
    int32_t row_mode = 0;            // 1: row-owner kernels (LAD_PATH_ROWS)
    bool cols_complete[3] = {true, true, true};  // column array of each pattern buffer complete
    int64_t host_syncs = 0;          // host synchronisations made for this context
    double pattern_ms = 0.0;         // GPU time of the topology pattern's build
    int32_t debug_flags = 0;         // lad_set_debug
    int32_t grid_eval = 0, grid_hvp = 0;
    void *d_slot_rest = nullptr;
    int32_t *d_fptr = nullptr;
    int32_t *d_sl_ptr = nullptr, *d_sl_nb = nullptr, *d_sl_rows = nullptr;
    int16_t *d_sl_d16 = nullptr;
    void *d_sl_rest = nullptr;
    FaceInc *d_finc = nullptr;
    RowFace *d_rfinc = nullptr;
    int32_t *d_sf_ptr = nullptr;
    SliceFace *d_sface = nullptr;
    void *d_face_dm = nullptr, *d_face_area = nullptr;

    std::vector<void *> allocs;
    PatchHdr *d_hdr = nullptr;
    int32_t *d_rib = nullptr;
    SpringRec *d_spr = nullptr;
    void *d_spr_rest = nullptr;
    FaceRec *d_fac = nullptr;
    void *d_fac_dm = nullptr;
    void *d_fac_area = nullptr;
    int32_t *d_col_bounds = nullptr;
    uint16_t *d_diag_rel = nullptr;
    // element-once patches (LAD_PATH_PATCH_ATOMIC): see Plan
    int32_t *d_spr_gblk = nullptr, *d_fac_gblk = nullptr;
    uint8_t *d_blk_flag = nullptr, *d_vtx_flag = nullptr;
    int32_t *d_bnd_blk = nullptr, *d_bnd_vtx = nullptr;
    int32_t nbnd_blk = 0, nbnd_vtx = 0;
    void *d_xt = nullptr;
    DevState *d_state = nullptr;
    double *d_epart = nullptr;
    PatternBufs pat{};
    InsertBufs ins{};
    // vector objective: springs in input order, their rest lengths (dtype),
    // and the Jacobian pattern (built by the first lad_jacobian_pattern call)
    int32_t ns = 0;
    int32_t *d_springs = nullptr;
    int32_t *d_faces = nullptr;      // kept on the device for vertex-face contacts
    void *d_vf_eval = nullptr;       // per contact vertex: local term strips [4 vf_cap][kVfStrip]
    void *d_vf_hvp = nullptr;        // per contact vertex: H_e u_e [4 vf_cap][kVfHvpStrip]
    int32_t *d_vf_ids = nullptr;     // [vf_cap][4]
    int32_t *d_vf_slots = nullptr;   // [4 vf_cap][4]
    void *d_spring_rest = nullptr;
    int32_t *d_jrp = nullptr, *d_jci = nullptr;
    // Newton-CG work space, allocated by the first lad_newton_cg call
    void *cg_r = nullptr, *cg_d = nullptr, *cg_d2 = nullptr, *cg_y = nullptr;
    double *cg_parts = nullptr;      // partial sums of d.Bd
    double *cg_parts2 = nullptr;     // partial sums of r.r
    int32_t cg_nparts = 0;
    CgState *d_cg = nullptr;
    CgState *h_cg = nullptr;         // pinned host copy
    std::string err;
};

namespace {

thread_local std::string g_build_error;

lad_status fail(lad_ctx *ctx, lad_status s, const std::string &msg)
{
    if (ctx) ctx->err = msg;
    else g_build_error = msg;
    return s;
}

lad_status hip_fail(lad_ctx *ctx, hipError_t e, const char *what)
{
    return fail(ctx, LAD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Every host synchronisation the library makes for a context goes through
// here, so lad_get_info can report how many there were.
hipError_t host_sync(lad_ctx *ctx, hipStream_t s)
{
    if (ctx) ++ctx->host_syncs;
    return hipStreamSynchronize(s);
}

template <typename T>
hipError_t dev_alloc(lad_ctx *ctx, T **p, size_t count)
{
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, count > 0 ? count * sizeof(T) : 16);
    if (e == hipSuccess) {
        ctx->allocs.push_back(q);
        *p = static_cast<T *>(q);
    }
    return e;
}

void free_all(lad_ctx *ctx)
{
    for (void *p : ctx->allocs) (void)hipFree(p);
    ctx->allocs.clear();
    if (ctx->h_cg) (void)hipHostFree(ctx->h_cg);
    ctx->h_cg = nullptr;
}

std::string check_desc(const lad_mesh_desc *d)
{
    if (!d) return "desc is NULL";
    if (d->nv <= 0) return "nv must be >= 1";
    if (d->nf < 0 || d->ns < 0) return "nf and ns must be >= 0";
    if (d->dtype != LAD_F32 && d->dtype != LAD_F64) return "dtype must be LAD_F32 or LAD_F64";
    if (d->pair_capacity < 0) return "pair_capacity must be >= 0";
    if (d->vf_capacity < 0) return "vf_capacity must be >= 0";
    if (int64_t(d->pair_capacity) + d->vf_capacity > int64_t(kInsMaxWg) * kThreads)
        return "pair_capacity + vf_capacity must be at most " +
               std::to_string(int64_t(kInsMaxWg) * kThreads);
    if (d->vf_capacity > 0 && d->nf == 0) return "vertex-face contacts need faces";
    if (d->vf_capacity > 0 && (d->eval_path == LAD_PATH_PATCH ||
                               d->eval_path == LAD_PATH_PATCH_LDS_ATOMIC))
        return "vertex-face contacts need the row path";
    if (d->eval_path != LAD_PATH_AUTO && d->eval_path != LAD_PATH_PATCH &&
        d->eval_path != LAD_PATH_ROWS && d->eval_path != LAD_PATH_PATCH_ATOMIC &&
        d->eval_path != LAD_PATH_PATCH_LDS_ATOMIC)
        return "eval_path must be LAD_PATH_AUTO, LAD_PATH_PATCH, LAD_PATH_ROWS, "
               "LAD_PATH_PATCH_ATOMIC or LAD_PATH_PATCH_LDS_ATOMIC";
    if (d->eval_path == LAD_PATH_PATCH_ATOMIC &&
        (d->deterministic || d->pair_capacity > 0 || d->vf_capacity > 0))
        return "LAD_PATH_PATCH_ATOMIC takes no deterministic mode and no contact capacity";
    if (d->eval_path == LAD_PATH_PATCH_LDS_ATOMIC && d->deterministic)
        return "LAD_PATH_PATCH_LDS_ATOMIC takes no deterministic mode";
    if (d->patch_lds_bytes < 0 || d->patch_lds_bytes > kMaxPatchLds)
        return "patch_lds_bytes must be in [0, " + std::to_string(kMaxPatchLds) + "]";
    if (d->nf > 0 && !d->faces) return "faces is NULL";
    for (int64_t f = 0; f < d->nf; ++f) {
        const int32_t *t = d->faces + 3 * f;
        for (int i = 0; i < 3; ++i)
            if (t[i] < 0 || t[i] >= d->nv) return "face vertex id out of range";
        if (t[0] == t[1] || t[1] == t[2] || t[0] == t[2]) return "face with a repeated vertex";
    }
    if (d->ns > 0) {
        if (!d->springs || !d->rest_len) return "springs or rest_len is NULL";
        for (int64_t s = 0; s < d->ns; ++s) {
            const int32_t a = d->springs[2 * s], b = d->springs[2 * s + 1];
            if (a < 0 || a >= d->nv || b < 0 || b >= d->nv) return "spring vertex id out of range";
            if (a == b) return "spring with a == b";
            if (!std::isfinite(d->rest_len[s])) return "non-finite rest length";
        }
        if (!std::isfinite(d->k)) return "non-finite k";
    }
    if (d->inertia) {
        if (!d->x_tilde) return "x_tilde is NULL";
        if (!std::isfinite(d->c)) return "non-finite c";
    }
    if (d->face_energy && d->nf > 0 && (!d->dm_inv || !d->area)) return "dm_inv or area is NULL";
    if (d->pair_capacity > 0 || d->vf_capacity > 0) {
        if (!(d->dhat > 0) || !std::isfinite(d->dhat)) return "dhat must be > 0 with contacts";
        if (!std::isfinite(d->kappa)) return "non-finite kappa";
        if (2 * int64_t(d->pair_capacity) + 4 * int64_t(d->vf_capacity) >= (int64_t(1) << 29))
            return "pair_capacity / vf_capacity too large";
    }
    const int64_t raw = int64_t(d->nv) + 6 * int64_t(d->nf) + 2 * int64_t(d->ns);
    if (raw >= (int64_t(1) << 31)) return "mesh too large for int32 pattern indices";
    return "";
}

template <typename T>
std::vector<T> narrow(const double *src, size_t n)
{
    std::vector<T> out(n);
    for (size_t i = 0; i < n; ++i) out[i] = T(src[i]);
    return out;
}

template <typename T>
hipError_t upload(lad_ctx *ctx, T **dst, const std::vector<T> &src, hipStream_t s)
{
    hipError_t e = dev_alloc(ctx, dst, src.size());
    if (e == hipSuccess && !src.empty())
        e = hipMemcpyAsync(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice, s);
    return e;
}

template <typename T>
lad_status upload_constants(lad_ctx *ctx, const lad_mesh_desc *d, const Plan &plan,
                            const RowPlan &rplan, hipStream_t s)
{
    std::vector<T> rest(plan.spr_src.size());
    for (size_t i = 0; i < rest.size(); ++i) rest[i] = T(d->rest_len[plan.spr_src[i]]);
    std::vector<T> dm(plan.fac_src.size() * 4), area(plan.fac_src.size());
    for (size_t i = 0; i < area.size(); ++i) {
        const int64_t f = plan.fac_src[i];
        for (int j = 0; j < 4; ++j) dm[4 * i + j] = T(d->dm_inv[4 * f + j]);
        area[i] = T(d->area[f]);
    }
    T *p = nullptr;
    hipError_t e = upload(ctx, &p, rest, s);
    ctx->d_spr_rest = p;
    if (e == hipSuccess) e = upload(ctx, &p, dm, s);
    ctx->d_fac_dm = p;
    if (e == hipSuccess) e = upload(ctx, &p, area, s);
    ctx->d_fac_area = p;
    if (e == hipSuccess && d->inertia) {
        e = upload(ctx, &p, narrow<T>(d->x_tilde, size_t(d->nv) * 3), s);
        ctx->d_xt = p;
    }
    if (e == hipSuccess && d->ns > 0) {
        e = upload(ctx, &p, narrow<T>(d->rest_len, size_t(d->ns)), s);
        ctx->d_spring_rest = p;
    }
    if (e == hipSuccess && ctx->row_mode) {
        e = upload(ctx, &p, narrow<T>(rplan.slot_rest.data(), rplan.slot_rest.size()), s);
        ctx->d_slot_rest = p;
        if (e == hipSuccess) e = upload(ctx, &ctx->d_sl_ptr, rplan.sl_ptr, s);
        if (e == hipSuccess && !rplan.sl_rows.empty()) e = upload(ctx, &ctx->d_sl_rows, rplan.sl_rows, s);
        if (e == hipSuccess && !rplan.sl_d16.empty()) e = upload(ctx, &ctx->d_sl_d16, rplan.sl_d16, s);
        else if (e == hipSuccess) e = upload(ctx, &ctx->d_sl_nb, rplan.sl_nb, s);
        if (e == hipSuccess) e = upload(ctx, &p, narrow<T>(rplan.sl_rest.data(), rplan.sl_rest.size()), s);
        ctx->d_sl_rest = p;
    }
    if (e == hipSuccess && ctx->row_mode && ctx->faces_on) {
        e = upload(ctx, &p, narrow<T>(d->dm_inv, size_t(d->nf) * 4), s);
        ctx->d_face_dm = p;
        if (e == hipSuccess) e = upload(ctx, &p, narrow<T>(d->area, size_t(d->nf)), s);
        ctx->d_face_area = p;
        if (e == hipSuccess) e = upload(ctx, &ctx->d_fptr, rplan.fptr, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_finc, rplan.finc, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_rfinc, rplan.rfinc, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_sf_ptr, rplan.sf_ptr, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_sface, rplan.sface, s);
    }
    // lifetime of the host vectors: synchronise before they go out of scope
    if (e == hipSuccess) e = host_sync(ctx, s);
    return e == hipSuccess ? LAD_OK : hip_fail(ctx, e, "upload of element constants");
}

template <typename T>
PatchArgs<T> patch_args(const lad_ctx *ctx)
{
    PatchArgs<T> a{};
    a.hdr = ctx->d_hdr;
    a.npatch = ctx->npatch;
    a.rib = ctx->d_rib;
    a.spr = ctx->d_spr;
    a.spr_rest = static_cast<const T *>(ctx->d_spr_rest);
    a.fac = ctx->d_fac;
    a.fac_dm = static_cast<const T *>(ctx->d_fac_dm);
    a.fac_area = static_cast<const T *>(ctx->d_fac_area);
    a.col_bounds = ctx->d_col_bounds;
    a.diag_rel = ctx->d_diag_rel;
    a.x_tilde = static_cast<const T *>(ctx->d_xt);
    a.k = T(ctx->k);
    a.c = T(ctx->c);
    a.springs_on = ctx->springs_on;
    a.faces_on = ctx->faces_on;
    a.inertia_on = ctx->inertia_on;
    a.state = ctx->d_state;
    a.pat = ctx->pat;
    a.spr_gblk = ctx->d_spr_gblk;
    a.fac_gblk = ctx->d_fac_gblk;
    a.blk_flag = ctx->d_blk_flag;
    a.vtx_flag = ctx->d_vtx_flag;
    return a;
}

template <typename T>
RowArgs<T> row_args(const lad_ctx *ctx)
{
    RowArgs<T> a{};
    a.chunk = ctx->d_hdr;
    a.nchunk = ctx->npatch;
    a.nv = ctx->nv;
    a.rp0 = ctx->pat.rp[0];
    a.ci0 = ctx->pat.ci[0];
    a.slot_rest = static_cast<const T *>(ctx->d_slot_rest);
    a.sl_rows = ctx->d_sl_rows;
    a.sl_ptr = ctx->d_sl_ptr;
    a.sl_nb = ctx->d_sl_nb;
    a.sl_d16 = ctx->d_sl_d16;
    a.sl_rest = static_cast<const T *>(ctx->d_sl_rest);
    a.x_tilde = static_cast<const T *>(ctx->d_xt);
    a.fptr = ctx->d_fptr;
    a.finc = ctx->d_finc;
    a.rfinc = ctx->d_rfinc;
    a.sf_ptr = ctx->d_sf_ptr;
    a.sface = ctx->d_sface;
    a.face_dm = static_cast<const T *>(ctx->d_face_dm);
    a.face_area = static_cast<const T *>(ctx->d_face_area);
    a.k = T(ctx->k);
    a.c = T(ctx->c);
    a.kappa = T(ctx->kappa);
    a.dhat = T(ctx->dhat);
    a.springs_on = ctx->springs_on;
    a.inertia_on = ctx->inertia_on;
    a.faces_on = ctx->faces_on;
    a.pairs_on = (ctx->pair_cap > 0 || ctx->vf_cap > 0) ? 1 : 0;
    a.lds_blocks = ctx->row_lds_blocks;
    a.state = ctx->d_state;
    a.pat = ctx->pat;
    a.vf_eval = static_cast<T *>(ctx->d_vf_eval);
    a.vf_hvp = static_cast<T *>(ctx->d_vf_hvp);
    a.vf_ids = ctx->d_vf_ids;
    a.vf_slots = ctx->d_vf_slots;
    a.vf_stride = ctx->vf_cap;
    return a;
}

// Partial energies one evaluation writes: one per workgroup of its launches.
int32_t eval_nparts(const lad_ctx *ctx)
{
    return (ctx->row_mode ? ctx->grid_eval : ctx->npatch) + ctx->pair_blocks;
}

template <typename T>
hipError_t enqueue_eval(lad_ctx *ctx, const void *x, double *energy, void *g, void *hv,
                        double *parts, hipStream_t s)
{
    // Every workgroup stores its partial energy at parts[...] (no slot is
    // read before it is written); one small launch sums them when the
    // caller asked for the energy.
    hipError_t e = hipSuccess;
    int32_t nparts = 0;
    if (ctx->row_mode) {
        // the vertex-face contact terms (one thread each), every row that no
        // contact touches, then the touched rows, which add the contact terms
        if (ctx->vf_cap > 0) e = launch_vf_eval<T>(row_args<T>(ctx), static_cast<const T *>(x), s);
        if (e == hipSuccess)
            e = launch_eval_rows<T>(row_args<T>(ctx), static_cast<const T *>(x),
                                    static_cast<T *>(g), static_cast<T *>(hv),
                                    EnergySink{parts, 0}, ctx->grid_eval, s);
        nparts = ctx->grid_eval;
        // rows touched by pairs, one thread each
        if (e == hipSuccess && ctx->pair_blocks > 0) {
            e = launch_eval_pair_rows<T>(row_args<T>(ctx), static_cast<const T *>(x),
                                         static_cast<T *>(g), static_cast<T *>(hv),
                                         EnergySink{parts, ctx->grid_eval},
                                         ctx->pair_blocks, s);
            nparts += ctx->pair_blocks;
        }
    } else {
        const PatchArgs<T> a = patch_args<T>(ctx);
        // element-once patches add into the boundary slots: zero them first
        if (ctx->mode == kModeBoundaryAtomic)
            e = launch_zero_boundary<T>(ctx->d_bnd_blk, ctx->nbnd_blk, ctx->d_bnd_vtx,
                                        ctx->nbnd_vtx, static_cast<T *>(hv), static_cast<T *>(g),
                                        s);
        if (e == hipSuccess)
            e = launch_eval<T>(a, static_cast<const T *>(x), static_cast<T *>(g),
                               static_cast<T *>(hv), EnergySink{parts, 0}, ctx->mode,
                               ctx->lds_eval, s);
        if (e == hipSuccess && ctx->pair_blocks > 0)
            e = launch_pairs_eval<T>(ctx->d_state, ctx->pat, static_cast<const T *>(x),
                                     static_cast<T *>(g), static_cast<T *>(hv),
                                     EnergySink{parts, ctx->npatch}, ctx->pair_blocks,
                                     T(ctx->kappa), T(ctx->dhat), s);
        nparts = ctx->npatch + ctx->pair_blocks;
    }
    if (e == hipSuccess && energy) e = launch_energy_reduce(parts, nparts, energy, s);
    return e;
}

template <typename T>
hipError_t enqueue_hvp_patch(lad_ctx *ctx, const void *x, const void *v, void *y, hipStream_t s)
{
    const PatchArgs<T> a = patch_args<T>(ctx);
    hipError_t e = hipSuccess;
    if (ctx->mode == kModeBoundaryAtomic)
        e = launch_zero_boundary<T>(nullptr, 0, ctx->d_bnd_vtx, ctx->nbnd_vtx, (T *)nullptr,
                                    static_cast<T *>(y), s);
    if (e == hipSuccess)
        e = launch_hvp<T>(a, static_cast<const T *>(x), static_cast<const T *>(v),
                          static_cast<T *>(y), ctx->mode, ctx->lds_hvp, s);
    if (e == hipSuccess && ctx->pair_blocks > 0)
        e = launch_pairs_hvp<T>(ctx->d_state, ctx->pat, static_cast<const T *>(x),
                                static_cast<const T *>(v), static_cast<T *>(y), ctx->pair_blocks,
                                T(ctx->kappa), T(ctx->dhat), s);
    return e;
}

// Workgroups of the touched-row HVP kernel (a grid-stride loop over the
// pattern's incidence entries); 0 without contact capacity.
int pair_hvp_grid(const lad_ctx *ctx)
{
    return std::min<int32_t>(ctx->pair_blocks, kCgMaxGrid);
}

// y = H v.  The row path can also produce per-workgroup partial sums of
// v.y (into dot_parts, returning their number in *dot_parts_used; 0 means
// the caller must compute v.y itself) and form v itself as a Newton-CG
// direction (cg.r non-null), taking the step that closes the previous
// update first.
template <typename T>
hipError_t enqueue_hvp(lad_ctx *ctx, const void *x, const void *v, void *y, hipStream_t s,
                       double *dot_parts = nullptr, int32_t *dot_parts_used = nullptr,
                       const CgDir<T> &cg = CgDir<T>{})
{
    if (dot_parts_used) *dot_parts_used = 0;
    if (ctx->row_mode) {
        // every row's topology terms; then, with contacts possible, the
        // vertex-face contacts' H_e u_e and the touched rows, which add their
        // contact terms (and their part of v.y after the rows' own)
        RowArgs<T> a = row_args<T>(ctx);
        a.hvp_dot = dot_parts;
        const T *xt = static_cast<const T *>(x);
        hipError_t e = launch_hvp_rows<T>(a, xt, static_cast<const T *>(v), static_cast<T *>(y),
                                          ctx->grid_hvp, s, cg);
        const T *u = cg.r ? cg.d_new : static_cast<const T *>(v);  // the direction as stored
        if (e == hipSuccess && ctx->vf_cap > 0) e = launch_vf_hvp<T>(a, xt, u, cg.st, s);
        const int pg = pair_hvp_grid(ctx);
        if (e == hipSuccess && pg > 0)
            e = launch_hvp_pair_rows<T>(a, xt, u, static_cast<T *>(y),
                                        dot_parts ? dot_parts + ctx->grid_hvp : nullptr, pg,
                                        cg.st, s);
        if (dot_parts_used && dot_parts) *dot_parts_used = ctx->grid_hvp + pg;
        return e;
    }
    return enqueue_hvp_patch<T>(ctx, x, v, y, s);
}

// Iterations enqueued between two host reads of the solve's stop flag.
constexpr int32_t kCgCheck = 16;
// From this many vertices on, the row path forms each Newton-CG direction in
// a launch of its own and runs the plain product on it (one operand array,
// five waves per SIMD); below, the product forms the direction itself from
// r and the previous direction (two operand arrays, four waves per SIMD),
// which saves a launch.  At 1000 x 1000: 45 against 51 us per iteration; at
// 100 x 100: 15.7 against 12.9 us.
constexpr int32_t kCgSplitRows = 65536;

hipError_t cg_workspace(lad_ctx *ctx)
{
    if (ctx->d_cg) return hipSuccess;
    const size_t n = size_t(ctx->nv) * 3;
    const size_t bytes = n * size_t(ctx->es);
    char *r = nullptr, *d = nullptr, *d2 = nullptr, *y = nullptr;
    hipError_t e = dev_alloc(ctx, &r, bytes);
    if (e == hipSuccess) e = dev_alloc(ctx, &d, bytes);
    if (e == hipSuccess && ctx->row_mode) e = dev_alloc(ctx, &d2, bytes);
    if (e == hipSuccess) e = dev_alloc(ctx, &y, bytes);
    const int32_t np = std::max<int32_t>(kCgMaxGrid, ctx->grid_hvp + pair_hvp_grid(ctx));
    double *parts = nullptr, *parts2 = nullptr;
    if (e == hipSuccess) e = dev_alloc(ctx, &parts, size_t(np));
    if (e == hipSuccess) e = dev_alloc(ctx, &parts2, size_t(kCgMaxGrid));
    CgState *st = nullptr;
    if (e == hipSuccess) e = dev_alloc(ctx, &st, 1);
    CgState *h = nullptr;
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&h), sizeof(CgState));
    if (e != hipSuccess) return e;
    ctx->cg_r = r;
    ctx->cg_d = d;
    ctx->cg_d2 = d2;
    ctx->cg_y = y;
    ctx->cg_parts = parts;
    ctx->cg_parts2 = parts2;
    ctx->cg_nparts = np;
    ctx->d_cg = st;
    ctx->h_cg = h;
    return hipSuccess;
}

// Truncated Newton-CG (line-search Newton-CG, Nocedal and Wright,
// Algorithm 7.1).  Iteration j: the direction (after the step that closes
// update j - 1: convergence or beta) d = -r + beta d, y = H d and the
// partial sums of d.y; then update j (after its step: the negative-
// curvature exit or alpha) p += alpha d, r += alpha y with the partial sums
// of r.r.  Each step is taken by every workgroup of the kernel that needs
// it, so the row path runs two launches per iteration (the direction and
// the d.y sums are fused into the HVP, d alternating between two buffers),
// or on large meshes three (the direction, the HVP with the d.y sums, the
// update); the patch path runs the direction, its HVP, the d.y sums and the
// update.
// One launch after the last iteration closes it.  All scalars stay on the
// device; the host reads the stop flag every kCgCheck iterations and the
// final state.
template <typename T>
hipError_t enqueue_newton_cg(lad_ctx *ctx, const void *x, const void *gv, void *pv,
                             int32_t max_iters, double eta, hipStream_t s)
{
    hipError_t e = cg_workspace(ctx);
    if (e != hipSuccess) return e;
    const int64_t n = int64_t(ctx->nv) * 3;
    const int grid = cg_vec_grid(n);
    const T *g = static_cast<const T *>(gv);
    T *p = static_cast<T *>(pv);
    T *r = static_cast<T *>(ctx->cg_r), *d = static_cast<T *>(ctx->cg_d),
      *y = static_cast<T *>(ctx->cg_y);
    CgState *st = ctx->d_cg;
    e = launch_cg_init<T>(g, p, r, d, n, ctx->cg_parts2, grid, s);
    if (e == hipSuccess) e = launch_cg_start(ctx->cg_parts2, grid, st, eta, max_iters, s);
    int32_t done = 0;
    while (e == hipSuccess && done < max_iters) {
        const int32_t nb = std::min(kCgCheck, max_iters - done);
        for (int32_t it = 0; it < nb && e == hipSuccess; ++it) {
            const int32_t j = done + it;
            int32_t nparts = 0;
            T *dj = d;  // this iteration's direction
            if (ctx->row_mode && ctx->nv >= kCgSplitRows) {
                // d_j = -r + beta d_(j-1) in its own launch (the first
                // direction, -g, is the init kernel's), then the plain
                // product, which also writes the partial sums of d.y and
                // stops with the solve
                if (j > 0) e = launch_cg_dir<T>(r, d, n, grid, ctx->cg_parts2, grid, st, j, s);
                CgDir<T> only_stop;
                only_stop.st = st;
                if (e == hipSuccess)
                    e = enqueue_hvp<T>(ctx, x, d, y, s, ctx->cg_parts, &nparts, only_stop);
            } else if (ctx->row_mode) {
                // d_j = -r + beta d_(j-1) inside the HVP; beta is 0 on the
                // first iteration, where d_(-1) = -g from the init kernel
                T *d_old = j % 2 == 0 ? d : static_cast<T *>(ctx->cg_d2);
                dj = j % 2 == 0 ? static_cast<T *>(ctx->cg_d2) : d;
                CgDir<T> cg;
                cg.r = r;
                cg.d_old = d_old;
                cg.d_new = dj;
                cg.st = st;
                cg.rr_parts = ctx->cg_parts2;
                cg.n_rr = grid;
                cg.iter = j;
                e = enqueue_hvp<T>(ctx, x, nullptr, y, s, ctx->cg_parts, &nparts, cg);
            } else {
                if (j > 0) e = launch_cg_dir<T>(r, d, n, grid, ctx->cg_parts2, grid, st, j, s);
                if (e == hipSuccess) e = enqueue_hvp<T>(ctx, x, d, y, s);
                nparts = grid;
                if (e == hipSuccess) e = launch_cg_dot<T>(d, y, n, ctx->cg_parts, grid, st, s);
            }
            if (e == hipSuccess)
                e = launch_cg_update<T>(p, r, dj, y, n, ctx->cg_parts, nparts, ctx->cg_parts2,
                                        grid, st, j, s);
        }
        done += nb;
        if (e == hipSuccess && done < max_iters) {
            e = hipMemcpyAsync(ctx->h_cg, st, sizeof(CgState), hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = host_sync(ctx, s);
            if (e == hipSuccess && ctx->h_cg->stop) break;
        }
    }
    if (e == hipSuccess) e = launch_cg_close(ctx->cg_parts2, grid, st, done, s);
    if (e == hipSuccess) e = launch_cg_final<T>(g, p, n, grid, st, s);
    if (e == hipSuccess) e = hipMemcpyAsync(ctx->h_cg, st, sizeof(CgState), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    return e;
}

lad_status build(const lad_mesh_desc *d, hipStream_t s, lad_ctx *ctx)
{
    hipError_t e = hipGetDevice(&ctx->device);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipGetDevice");
    const int32_t nv = d->nv;
    ctx->nv = nv;
    ctx->dtype = d->dtype;
    ctx->es = d->dtype == LAD_F64 ? 8 : 4;
    // the patch path's assembly: colour phases unless an atomic one is asked
    // for (on gfx950 they are several times faster than LDS float atomics)
    ctx->mode = d->eval_path == LAD_PATH_PATCH_ATOMIC       ? kModeBoundaryAtomic
                : d->eval_path == LAD_PATH_PATCH_LDS_ATOMIC ? kModeLdsAtomic
                                                            : kModeColour;
    ctx->stream = s;
    ctx->pair_cap = d->pair_capacity;
    ctx->vf_cap = d->vf_capacity;
    ctx->nf = d->nf;
    ctx->k = d->k;
    ctx->c = d->c;
    ctx->kappa = d->kappa;
    ctx->dhat = d->dhat;
    ctx->springs_on = d->ns > 0;
    ctx->faces_on = d->face_energy && d->nf > 0;
    ctx->inertia_on = d->inertia ? 1 : 0;

    // ---- topology pattern on the GPU
    std::vector<void *> temps;
    auto tmp_alloc = [&](int32_t **p, size_t n) {
        void *q = nullptr;
        hipError_t r = hipMalloc(&q, (n > 0 ? n : 1) * sizeof(int32_t));
        if (r == hipSuccess) {
            temps.push_back(q);
            *p = static_cast<int32_t *>(q);
        }
        return r;
    };
    auto free_temps = [&]() {
        for (void *q : temps) (void)hipFree(q);
        temps.clear();
    };
    const int64_t raw = int64_t(nv) + 6 * int64_t(d->nf) + 2 * int64_t(d->ns);
    int32_t *d_faces = nullptr, *d_springs = nullptr;
    PatternScratch sc{};
    // the faces stay on the device when vertex-face contacts may reference them
    e = d->vf_capacity > 0 ? dev_alloc(ctx, &d_faces, size_t(d->nf) * 3)
                           : tmp_alloc(&d_faces, size_t(d->nf) * 3);
    if (d->vf_capacity > 0) ctx->d_faces = d_faces;
    // the springs stay on the device for the vector objective
    if (e == hipSuccess) e = dev_alloc(ctx, &d_springs, size_t(d->ns) * 2);
    ctx->d_springs = d_springs;
    ctx->ns = d->ns;
    if (e == hipSuccess) e = tmp_alloc(&sc.cnt, nv);
    if (e == hipSuccess) e = tmp_alloc(&sc.off, size_t(nv) + 1);
    if (e == hipSuccess) e = tmp_alloc(&sc.raw, size_t(raw));
    if (e == hipSuccess) e = tmp_alloc(&sc.cur, nv);
    if (e == hipSuccess) e = tmp_alloc(&sc.ucnt, nv);
    if (e == hipSuccess) e = tmp_alloc(&sc.tmp, size_t(scan_tmp_size(nv)));
    int32_t *d_rp0 = nullptr, *d_ci0 = nullptr;
    if (e == hipSuccess) e = dev_alloc(ctx, &d_rp0, size_t(nv) + 1);
    if (e != hipSuccess) {
        free_temps();
        return fail(ctx, LAD_ERR_OOM, std::string("device allocation: ") + hipGetErrorString(e));
    }
    if (d->nf > 0)
        e = hipMemcpyAsync(d_faces, d->faces, size_t(d->nf) * 3 * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && d->ns > 0)
        e = hipMemcpyAsync(d_springs, d->springs, size_t(d->ns) * 2 * 4, hipMemcpyHostToDevice, s);
    // HIP events around the pattern launches (count .. scan here, the
    // compaction below) time the build on the GPU
    hipEvent_t ev[4] = {};
    bool timed = true;
    for (hipEvent_t &x : ev) timed = timed && hipEventCreate(&x) == hipSuccess;
    auto drop_events = [&]() {
        for (hipEvent_t &x : ev)
            if (x) (void)hipEventDestroy(x);
    };
    if (timed && e == hipSuccess) (void)hipEventRecord(ev[0], s);
    if (e == hipSuccess) e = launch_pattern_count(nv, d->nf, d_faces, d->ns, d_springs, sc, s);
    if (e == hipSuccess) e = launch_pattern_fill(nv, d->nf, d_faces, d->ns, d_springs, sc, s);
    if (e == hipSuccess) e = launch_pattern_unique(nv, sc, s);
    if (e == hipSuccess) e = launch_scan(sc.ucnt, d_rp0, nv, sc.tmp, s);
    if (timed && e == hipSuccess) (void)hipEventRecord(ev[1], s);
    std::vector<int32_t> h_rp(size_t(nv) + 1);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h_rp.data(), d_rp0, h_rp.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) {
        free_temps();
        drop_events();
        return hip_fail(ctx, e, "pattern build");
    }
    const int64_t nnzb = h_rp[nv];
    ctx->nnzb_base = nnzb;
    ctx->hcap = nnzb + 2 * int64_t(d->pair_capacity) + 6 * int64_t(d->vf_capacity);
    if (ctx->hcap * 9 >= (int64_t(1) << 31)) {
        free_temps();
        drop_events();
        return fail(ctx, LAD_ERR_ARG, "pattern too large for int32 value indices");
    }
    e = dev_alloc(ctx, &d_ci0, size_t(nnzb));
    if (timed && e == hipSuccess) (void)hipEventRecord(ev[2], s);
    if (e == hipSuccess) e = launch_pattern_compact(nv, sc, d_rp0, d_ci0, s);
    if (timed && e == hipSuccess) (void)hipEventRecord(ev[3], s);
    std::vector<int32_t> h_ci(static_cast<size_t>(nnzb));
    if (e == hipSuccess && nnzb > 0)
        e = hipMemcpyAsync(h_ci.data(), d_ci0, h_ci.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    free_temps();
    if (e == hipSuccess && timed) {
        float a = 0.f, b = 0.f;
        if (hipEventElapsedTime(&a, ev[0], ev[1]) == hipSuccess &&
            hipEventElapsedTime(&b, ev[2], ev[3]) == hipSuccess)
            ctx->pattern_ms = double(a) + double(b);
    }
    drop_events();
    if (e != hipSuccess) return hip_fail(ctx, e, "pattern compaction");

    // ---- patches (host)
    PlanInput in;
    in.nv = nv;
    in.nf = d->nf;
    in.faces = d->faces;
    in.ns = d->ns;
    in.springs = d->springs;
    in.face_energy = ctx->faces_on;
    in.row_ptr = h_rp.data();
    in.col_idx = h_ci.data();
    in.elem_size = ctx->es;
    in.lds_budget = d->patch_lds_bytes > 0 ? d->patch_lds_bytes : kDefaultPatchLds;
    in.element_once = ctx->mode == kModeBoundaryAtomic ? 1 : 0;
    Plan plan;
    RowPlan rplan;
    std::string why = "patch path requested";
    if (d->eval_path == LAD_PATH_AUTO || d->eval_path == LAD_PATH_ROWS)
        why = build_row_plan(in, d->rest_len, rplan);
    if (d->eval_path == LAD_PATH_ROWS && !why.empty())
        return fail(ctx, LAD_ERR_ARG, "row path not applicable: " + why);
    ctx->row_mode = why.empty() ? 1 : 0;
    if (!ctx->row_mode && d->vf_capacity > 0)
        return fail(ctx, LAD_ERR_ARG, "vertex-face contacts need the row path: " + why);
    if (ctx->row_mode) {
        plan.hdr = rplan.chunk;
        // the face kernel without contact capacity stages half chunks
        ctx->row_lds_blocks = (ctx->faces_on && d->pair_capacity == 0 && d->vf_capacity == 0)
                                  ? half_chunk_blocks(rplan.chunk, h_rp.data())
                                  : kRowLdsBlocks;
        ctx->lds_eval = ctx->es == 8 ? rows_lds_bytes<double>(ctx->row_lds_blocks)
                                     : rows_lds_bytes<float>(ctx->row_lds_blocks);
        ctx->lds_hvp = 0;
        ctx->nspr_rec = d->ns;
        ctx->nfac_rec = ctx->faces_on ? d->nf : 0;
    } else {
        std::string msg = build_plan(in, plan);
        if (!msg.empty()) return fail(ctx, LAD_ERR_ARG, "patcher: " + msg);
        ctx->lds_eval = plan.lds_eval;
        ctx->lds_hvp = plan.lds_hvp;
        ctx->max_colors = plan.max_colors;
        ctx->nspr_rec = int64_t(plan.spr.size());
        ctx->nfac_rec = int64_t(plan.fac.size());
    }
    ctx->npatch = int32_t(plan.hdr.size());

    e = upload(ctx, &ctx->d_hdr, plan.hdr, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_rib, plan.rib, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_spr, plan.spr, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_fac, plan.fac, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_col_bounds, plan.col_bounds, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_diag_rel, plan.diag_rel, s);
    if (e == hipSuccess && ctx->mode == kModeBoundaryAtomic) {
        e = upload(ctx, &ctx->d_spr_gblk, plan.spr_gblk, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_fac_gblk, plan.fac_gblk, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_blk_flag, plan.blk_flag, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_vtx_flag, plan.vtx_flag, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_bnd_blk, plan.bnd_blk, s);
        if (e == hipSuccess) e = upload(ctx, &ctx->d_bnd_vtx, plan.bnd_vtx, s);
        ctx->nbnd_blk = int32_t(plan.bnd_blk.size());
        ctx->nbnd_vtx = int32_t(plan.bnd_vtx.size());
    }
    // with pair capacity: the insertion's tiles (whole row chunks on the row
    // path, for its capacity check; fixed row blocks on the patch path)
    // (the pointers are stored in ctx->ins after that struct is reset below)
    InsertTiles itiles;
    int32_t *d_tile_row = nullptr, *d_tile_unit = nullptr, *d_row_tile = nullptr,
            *d_row_unit = nullptr;
    if (e == hipSuccess && (d->pair_capacity > 0 || d->vf_capacity > 0)) {
        const std::string msg = build_insert_tiles(plan.hdr, nv, ctx->row_mode, itiles);
        if (!msg.empty()) return fail(ctx, LAD_ERR_ARG, "insertion tiles: " + msg);
        e = upload(ctx, &d_tile_row, itiles.tile_row, s);
        if (e == hipSuccess) e = upload(ctx, &d_tile_unit, itiles.tile_unit, s);
        if (e == hipSuccess) e = upload(ctx, &d_row_tile, itiles.row_tile, s);
        if (e == hipSuccess && ctx->row_mode) e = upload(ctx, &d_row_unit, itiles.row_unit, s);
    }
    if (e != hipSuccess) return hip_fail(ctx, e, "upload of patch tables");
    lad_status st = ctx->dtype == LAD_F64 ? upload_constants<double>(ctx, d, plan, rplan, s)
                                          : upload_constants<float>(ctx, d, plan, rplan, s);
    if (st != LAD_OK) return st;
    if (ctx->row_mode) {
        e = ctx->dtype == LAD_F64
                ? rows_grid<double>(ctx->row_lds_blocks, ctx->npatch, ctx->faces_on,
                                    ctx->pair_cap > 0 || ctx->vf_cap > 0,
                                    &ctx->grid_eval, &ctx->grid_hvp)
                : rows_grid<float>(ctx->row_lds_blocks, ctx->npatch, ctx->faces_on,
                                   ctx->pair_cap > 0 || ctx->vf_cap > 0,
                                   &ctx->grid_eval, &ctx->grid_hvp);
        if (e != hipSuccess) return hip_fail(ctx, e, "occupancy query");
    } else {
        ctx->grid_eval = ctx->npatch;
        ctx->grid_hvp = ctx->npatch;
    }

    // ---- pattern buffers, device state, scratch
    std::memset(&ctx->pat, 0, sizeof(ctx->pat));
    std::memset(&ctx->ins, 0, sizeof(ctx->ins));
    ctx->ins.tile_row = d_tile_row;
    ctx->ins.tile_unit = d_tile_unit;
    ctx->ins.row_tile = d_row_tile;
    ctx->ins.row_unit = d_row_unit;
    ctx->ins.ntiles = int32_t(itiles.tile_row.empty() ? 0 : itiles.tile_row.size() - 1);
    ctx->pat.rp[0] = d_rp0;
    ctx->pat.ci[0] = d_ci0;
    ctx->ins.rp[0] = d_rp0;
    ctx->ins.ci[0] = d_ci0;
    e = dev_alloc(ctx, &ctx->d_state, 1);
    DevState hs{};
    hs.nnzb[0] = int32_t(nnzb);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ctx->d_state, &hs, sizeof(hs), hipMemcpyHostToDevice, s);
    if (e == hipSuccess && (d->pair_capacity > 0 || d->vf_capacity > 0)) {
        // incidence entries: 2 per pair, 4 per vertex-face contact
        const size_t ninc = 2 * size_t(d->pair_capacity) + 4 * size_t(d->vf_capacity);
        for (int b = 1; b <= 2 && e == hipSuccess; ++b) {
            e = dev_alloc(ctx, &ctx->ins.rp[b], size_t(nv) + 1);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.ci[b], size_t(ctx->hcap));
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pairs[b], 2 * size_t(d->pair_capacity));
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.vf[b], 2 * size_t(d->vf_capacity));
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pinc_ptr[b], size_t(nv) + 1);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pinc[b], ninc);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pinc_row[b], ninc);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pnew[b], 3 * ninc);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.trow[b], ninc);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.pslot[b], ninc);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.rins1[b], size_t(nv));
        }
        const size_t nt = size_t(ctx->ins.ntiles);
        const size_t nel = size_t(d->pair_capacity) + size_t(d->vf_capacity);
        ctx->ins.max_wg = int32_t((nel + kThreads - 1) / kThreads);
        const size_t wg = size_t(ctx->ins.max_wg);
        if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.tstat, nt * kStatStride);
        if (e == hipSuccess) e = hipMemsetAsync(ctx->ins.tstat, 0, nt * kStatStride * 8, s);
        if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.hist, nt * wg);
        if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.hoff, nt * wg);
        if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.seg, 2 * wg * size_t(kInsWgEnt));
        if (e == hipSuccess) e = dev_alloc(ctx, &ctx->ins.erank, wg * size_t(kInsWgEnt));
        for (int b = 1; b <= 2; ++b) {
            ctx->pat.rp[b] = ctx->ins.rp[b];
            ctx->pat.ci[b] = ctx->ins.ci[b];
            ctx->pat.pairs[b] = ctx->ins.pairs[b];
            ctx->pat.pinc_ptr[b] = ctx->ins.pinc_ptr[b];
            ctx->pat.pinc[b] = ctx->ins.pinc[b];
            ctx->pat.pinc_row[b] = ctx->ins.pinc_row[b];
            ctx->pat.trow[b] = ctx->ins.trow[b];
            ctx->pat.pnew[b] = ctx->ins.pnew[b];
            ctx->pat.pslot[b] = ctx->ins.pslot[b];
            ctx->pat.rins1[b] = ctx->ins.rins1[b];
            ctx->pat.vf[b] = ctx->ins.vf[b];
        }
        ctx->ins.faces = ctx->d_faces;
        ctx->pat.faces = ctx->d_faces;
        if (e == hipSuccess && d->vf_capacity > 0) {
            char *ve = nullptr, *vh = nullptr;
            const size_t strips = 4 * size_t(d->vf_capacity);
            e = dev_alloc(ctx, &ve, strips * size_t(kVfStrip) * size_t(ctx->es));
            if (e == hipSuccess) e = dev_alloc(ctx, &vh, strips * size_t(kVfHvpStrip) * size_t(ctx->es));
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->d_vf_ids, strips);
            if (e == hipSuccess) e = dev_alloc(ctx, &ctx->d_vf_slots, 4 * strips);
            ctx->d_vf_eval = ve;
            ctx->d_vf_hvp = vh;
        }
        ctx->pair_blocks = int32_t((ninc + kThreads - 1) / kThreads);
    }
    if (e == hipSuccess)
        e = dev_alloc(ctx, &ctx->d_epart,
                      size_t(std::max(ctx->npatch, ctx->grid_eval) + ctx->pair_blocks));
    if (e == hipSuccess && !ctx->row_mode && (ctx->lds_eval > 64 * 1024 || ctx->lds_hvp > 64 * 1024))
        e = raise_lds_limits(std::max(ctx->lds_eval, ctx->lds_hvp));
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "allocation of pattern buffers");
    return LAD_OK;
}

lad_status check_vector_objective(lad_ctx *ctx)
{
    if (ctx->faces_on || ctx->pair_cap > 0 || ctx->vf_cap > 0)
        return fail(ctx, LAD_ERR_STATE,
                    "the vector objective covers spring and inertia terms; this context has face "
                    "or pair terms");
    const int64_t nnz = 6 * int64_t(ctx->ns) + (ctx->inertia_on ? 3 * int64_t(ctx->nv) : 0);
    if (nnz >= (int64_t(1) << 31))
        return fail(ctx, LAD_ERR_STATE, "Jacobian too large for int32 indices");
    return LAD_OK;
}

template <typename T>
hipError_t enqueue_residual_jacobian(lad_ctx *ctx, const void *x, void *r, void *jv,
                                            hipStream_t s)
{
    const int64_t irows = ctx->inertia_on ? 3 * int64_t(ctx->nv) : 0;
    return launch_residual_jacobian<T>(ctx->ns, ctx->d_springs,
                                       static_cast<const T *>(ctx->d_spring_rest),
                                       T(std::sqrt(ctx->k)), irows, static_cast<const T *>(x),
                                       static_cast<const T *>(ctx->d_xt), T(std::sqrt(ctx->c)),
                                       static_cast<T *>(r), static_cast<T *>(jv), s);
}

template <typename T>
hipError_t enqueue_gauss_newton(lad_ctx *ctx, const void *x, const void *v, void *y,
                                       hipStream_t s)
{
    return launch_gauss_newton_rows<T>(row_args<T>(ctx), T(std::sqrt(ctx->k)), T(std::sqrt(ctx->c)),
                                       static_cast<const T *>(x), static_cast<const T *>(v),
                                       static_cast<T *>(y), ctx->grid_hvp, s);
}

}  // namespace

namespace lad {

lad_status eval_with_parts(lad_ctx *ctx, const void *d_x, double *d_energy, void *d_grad,
                           void *d_hvals, int64_t hvals_capacity_blocks, double *parts,
                           hipStream_t s)
{
    if (!d_x || !d_grad || !d_hvals) return fail(ctx, LAD_ERR_ARG, "NULL buffer");
    if (hvals_capacity_blocks < ctx->hcap)
        return fail(ctx, LAD_ERR_ARG, "hvals capacity below " + std::to_string(ctx->hcap) + " blocks");
    hipError_t e = ctx->dtype == LAD_F64
                       ? enqueue_eval<double>(ctx, d_x, d_energy, d_grad, d_hvals, parts, s)
                       : enqueue_eval<float>(ctx, d_x, d_energy, d_grad, d_hvals, parts, s);
    if (e == hipSuccess && (ctx->debug_flags & LAD_DEBUG_NONFINITE))
        e = launch_check_finite(ctx->d_state, d_energy, d_grad, 3 * int64_t(ctx->nv), d_hvals,
                                ctx->es, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "eval launch");
    return LAD_OK;
}

int32_t eval_scratch_doubles(const lad_ctx *ctx) { return eval_nparts(ctx); }

int32_t ctx_device(const lad_ctx *ctx) { return ctx->device; }

int32_t ctx_vf_capacity(const lad_ctx *ctx) { return ctx->vf_cap; }

lad_status ctx_fail(lad_ctx *ctx, lad_status st, const char *msg) { return fail(ctx, st, msg); }

}  // namespace lad

extern "C" {

lad_status lad_build_pattern(const lad_mesh_desc *desc, void *hip_stream, lad_ctx **out)
{
    if (!out) return fail(nullptr, LAD_ERR_ARG, "out is NULL");
    *out = nullptr;
    const std::string msg = check_desc(desc);
    if (!msg.empty()) return fail(nullptr, LAD_ERR_ARG, msg);
    lad_ctx *ctx = new (std::nothrow) lad_ctx();
    if (!ctx) return fail(nullptr, LAD_ERR_OOM, "host allocation failed");
    const lad_status s = build(desc, static_cast<hipStream_t>(hip_stream), ctx);
    if (s != LAD_OK) {
        g_build_error = ctx->err;
        (void)host_sync(ctx, static_cast<hipStream_t>(hip_stream));
        free_all(ctx);
        delete ctx;
        return s;
    }
    g_build_error.clear();
    *out = ctx;
    return LAD_OK;
}

lad_status lad_get_info(lad_ctx *ctx, lad_info *info)
{
    if (!ctx || !info) return fail(ctx, LAD_ERR_ARG, "ctx or info is NULL");
    DevState hs{};
    hipError_t e = hipMemcpyAsync(&hs, ctx->d_state, sizeof(hs), hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = host_sync(ctx, ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_get_info");
    std::memset(info, 0, sizeof(*info));
    info->nv = ctx->nv;
    info->dtype = ctx->dtype;
    info->nnzb_base = ctx->nnzb_base;
    info->nnzb_active = hs.active == 0 ? ctx->nnzb_base : hs.nnzb[hs.active];
    info->hvals_capacity = ctx->hcap;
    info->npairs_active = hs.active == 0 ? 0 : hs.np[hs.active];
    info->nvf_active = hs.active == 0 ? 0 : hs.nvf[hs.active];
    info->npatches = ctx->npatch;
    info->lds_bytes_eval = ctx->lds_eval;
    info->lds_bytes_hvp = ctx->lds_hvp;
    info->spring_records = ctx->nspr_rec;
    info->face_records = ctx->nfac_rec;
    info->max_colors = ctx->max_colors;
    info->pattern_ms = ctx->pattern_ms;
    info->active_buffer = hs.active;
    info->eval_path = ctx->row_mode                         ? LAD_PATH_ROWS
                      : ctx->mode == kModeBoundaryAtomic ? LAD_PATH_PATCH_ATOMIC
                      : ctx->mode == kModeLdsAtomic      ? LAD_PATH_PATCH_LDS_ATOMIC
                                                         : LAD_PATH_PATCH;
    info->grid_eval = ctx->grid_eval;
    info->host_syncs = ctx->host_syncs;
    return LAD_OK;
}

lad_status lad_get_pattern(lad_ctx *ctx, void *hip_stream, int64_t *nnzb,
                           const int32_t **d_row_ptr, const int32_t **d_col_idx)
{
    if (!ctx || !nnzb || !d_row_ptr || !d_col_idx) return fail(ctx, LAD_ERR_ARG, "NULL argument");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    DevState hs{};
    hipError_t e = hipMemcpyAsync(&hs, ctx->d_state, sizeof(hs), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_get_pattern");
    const int a = hs.active;
    if (a < 0 || a > 2) return fail(ctx, LAD_ERR_STATE, "corrupt device state");
    *nnzb = a == 0 ? ctx->nnzb_base : hs.nnzb[a];
    if (!ctx->cols_complete[a]) {
        e = launch_complete_cols(ctx->d_state, ctx->ins, ctx->d_hdr, ctx->npatch, s);
        if (e == hipSuccess) e = host_sync(ctx, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "lad_get_pattern");
        ctx->cols_complete[a] = true;
    }
    *d_row_ptr = ctx->pat.rp[a];
    *d_col_idx = ctx->pat.ci[a];
    return LAD_OK;
}

lad_status lad_copy_pattern(lad_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                            int32_t *d_col_idx, int64_t col_capacity, int64_t *nnzb)
{
    if (!ctx || !d_row_ptr || !d_col_idx || !nnzb) return fail(ctx, LAD_ERR_ARG, "NULL argument");
    const int32_t *rp = nullptr, *ci = nullptr;
    lad_status st = lad_get_pattern(ctx, hip_stream, nnzb, &rp, &ci);
    if (st != LAD_OK) return st;
    if (*nnzb > col_capacity) return fail(ctx, LAD_ERR_CAPACITY, "col_capacity below nnzb");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipMemcpyAsync(d_row_ptr, rp, (size_t(ctx->nv) + 1) * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && *nnzb > 0)
        e = hipMemcpyAsync(d_col_idx, ci, size_t(*nnzb) * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_copy_pattern");
    return LAD_OK;
}

lad_status lad_eval_energy_grad_hess(lad_ctx *ctx, const void *d_x, double *d_energy,
                                     void *d_grad, void *d_hvals,
                                     int64_t hvals_capacity_blocks, void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    return lad::eval_with_parts(ctx, d_x, d_energy, d_grad, d_hvals, hvals_capacity_blocks,
                                ctx->d_epart, static_cast<hipStream_t>(hip_stream));
}

lad_status lad_hvp(lad_ctx *ctx, const void *d_x, const void *d_v, void *d_y, void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!d_x || !d_v || !d_y) return fail(ctx, LAD_ERR_ARG, "NULL buffer");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ctx->dtype == LAD_F64 ? enqueue_hvp<double>(ctx, d_x, d_v, d_y, s)
                                         : enqueue_hvp<float>(ctx, d_x, d_v, d_y, s);
    if (e == hipSuccess && (ctx->debug_flags & LAD_DEBUG_NONFINITE))
        e = launch_check_finite(ctx->d_state, nullptr, d_y, 3 * int64_t(ctx->nv), nullptr, ctx->es,
                                s);
    if (e != hipSuccess) return hip_fail(ctx, e, "hvp launch");
    return LAD_OK;
}

lad_status lad_newton_cg(lad_ctx *ctx, const void *d_x, const void *d_g, void *d_p,
                         int32_t max_iters, double eta, lad_cg_stats *stats, void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!d_x || !d_g || !d_p) return fail(ctx, LAD_ERR_ARG, "NULL buffer");
    if (d_p == d_g) return fail(ctx, LAD_ERR_ARG, "d_p must not alias d_g");
    if (max_iters < 0) return fail(ctx, LAD_ERR_ARG, "max_iters must be >= 0");
    if (!std::isfinite(eta)) return fail(ctx, LAD_ERR_ARG, "eta must be finite");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ctx->dtype == LAD_F64
                       ? enqueue_newton_cg<double>(ctx, d_x, d_g, d_p, max_iters, eta, s)
                       : enqueue_newton_cg<float>(ctx, d_x, d_g, d_p, max_iters, eta, s);
    if (e == hipErrorOutOfMemory) return fail(ctx, LAD_ERR_OOM, "Newton-CG work space");
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_newton_cg");
    if (stats) {
        const CgState &h = *ctx->h_cg;
        stats->iterations = h.iter;
        stats->reason = h.reason;
        stats->grad_norm = h.gnorm;
        stats->rel_residual = (h.reason == LAD_CG_NEG_CURVATURE && h.iter == 0) ? 1.0
                              : h.gnorm > 0.0 ? std::sqrt(h.rrv[h.iter & 1]) / h.gnorm
                                              : 0.0;
    }
    return LAD_OK;
}

lad_status lad_jacobian_pattern(lad_ctx *ctx, void *hip_stream, int64_t *nrows, int64_t *nnz,
                                const int32_t **d_row_ptr, const int32_t **d_col_idx)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!nrows || !nnz || !d_row_ptr || !d_col_idx) return fail(ctx, LAD_ERR_ARG, "NULL argument");
    lad_status st = check_vector_objective(ctx);
    if (st != LAD_OK) return st;
    const int64_t irows = ctx->inertia_on ? 3 * int64_t(ctx->nv) : 0;
    const int64_t m = int64_t(ctx->ns) + irows, n = 6 * int64_t(ctx->ns) + irows;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (!ctx->d_jrp) {
        int32_t *rp = nullptr, *ci = nullptr;
        hipError_t e = dev_alloc(ctx, &rp, size_t(m) + 1);
        if (e == hipSuccess) e = dev_alloc(ctx, &ci, size_t(n));
        if (e != hipSuccess) return fail(ctx, LAD_ERR_OOM, "Jacobian pattern");
        e = launch_jacobian_pattern(ctx->ns, ctx->d_springs, irows, rp, ci, s);
        if (e == hipSuccess) e = host_sync(ctx, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "Jacobian pattern");
        ctx->d_jrp = rp;
        ctx->d_jci = ci;
    }
    *nrows = m;
    *nnz = n;
    *d_row_ptr = ctx->d_jrp;
    *d_col_idx = ctx->d_jci;
    return LAD_OK;
}

lad_status lad_copy_jacobian_pattern(lad_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                                     int32_t *d_col_idx, int64_t col_capacity, int64_t *nnz)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!d_row_ptr || !d_col_idx || !nnz) return fail(ctx, LAD_ERR_ARG, "NULL argument");
    int64_t m = 0, n = 0;
    const int32_t *rp = nullptr, *ci = nullptr;
    lad_status st = lad_jacobian_pattern(ctx, hip_stream, &m, &n, &rp, &ci);
    if (st != LAD_OK) return st;
    *nnz = n;
    if (col_capacity < n)
        return fail(ctx, LAD_ERR_CAPACITY, "col_capacity below nnz " + std::to_string(n));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipMemcpyAsync(d_row_ptr, rp, size_t(m + 1) * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && n > 0)
        e = hipMemcpyAsync(d_col_idx, ci, size_t(n) * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_copy_jacobian_pattern");
    return LAD_OK;
}

lad_status lad_residual_jacobian(lad_ctx *ctx, const void *d_x, void *d_r, void *d_jvals,
                                 void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!d_x || !d_r || !d_jvals) return fail(ctx, LAD_ERR_ARG, "NULL buffer");
    lad_status st = check_vector_objective(ctx);
    if (st != LAD_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ctx->dtype == LAD_F64 ? enqueue_residual_jacobian<double>(ctx, d_x, d_r, d_jvals, s)
                                         : enqueue_residual_jacobian<float>(ctx, d_x, d_r, d_jvals, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "residual/Jacobian launch");
    return LAD_OK;
}

lad_status lad_gauss_newton_product(lad_ctx *ctx, const void *d_x, const void *d_v, void *d_y,
                                    void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (!d_x || !d_v || !d_y) return fail(ctx, LAD_ERR_ARG, "NULL buffer");
    lad_status st = check_vector_objective(ctx);
    if (st != LAD_OK) return st;
    if (!ctx->row_mode)
        return fail(ctx, LAD_ERR_STATE, "the Gauss-Newton product needs the row path");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ctx->dtype == LAD_F64 ? enqueue_gauss_newton<double>(ctx, d_x, d_v, d_y, s)
                                         : enqueue_gauss_newton<float>(ctx, d_x, d_v, d_y, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "Gauss-Newton launch");
    return LAD_OK;
}

lad_status lad_insert_contacts(lad_ctx *ctx, const int32_t *d_pairs, int32_t npairs,
                               const int32_t *d_vf, int32_t nvf, void *hip_stream)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (npairs < 0 || nvf < 0) return fail(ctx, LAD_ERR_ARG, "npairs and nvf must be >= 0");
    if (npairs > ctx->pair_cap)
        return fail(ctx, LAD_ERR_CAPACITY,
                    "npairs " + std::to_string(npairs) + " exceeds pair_capacity " +
                        std::to_string(ctx->pair_cap));
    if (nvf > ctx->vf_cap)
        return fail(ctx, LAD_ERR_CAPACITY,
                    "nvf " + std::to_string(nvf) + " exceeds vf_capacity " +
                        std::to_string(ctx->vf_cap));
    if (npairs > 0 && !d_pairs) return fail(ctx, LAD_ERR_ARG, "d_pairs is NULL");
    if (nvf > 0 && !d_vf) return fail(ctx, LAD_ERR_ARG, "d_vf is NULL");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool none = npairs == 0 && nvf == 0;
    hipError_t e = none ? launch_restore_topology(ctx->d_state, s)
                        : launch_insert(ctx->d_state, d_pairs, npairs, d_vf, nvf, ctx->nv,
                                        ctx->nf, ctx->ins, ctx->d_hdr, ctx->npatch,
                                        ctx->row_mode ? 0 : 1, s);
    // the row path leaves the untouched rows' columns of the new buffer
    // unwritten until the pattern is read
    if (ctx->row_mode && !none) ctx->cols_complete[1] = ctx->cols_complete[2] = false;
    if (e != hipSuccess) return hip_fail(ctx, e, "insert launch");
    return LAD_OK;
}

lad_status lad_insert_pairs(lad_ctx *ctx, const int32_t *d_pairs, int32_t npairs, void *hip_stream)
{
    return lad_insert_contacts(ctx, d_pairs, npairs, nullptr, 0, hip_stream);
}

lad_status lad_device_status(lad_ctx *ctx, void *hip_stream, int32_t *status)
{
    if (!ctx || !status) return fail(ctx, LAD_ERR_ARG, "NULL argument");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    DevState hs{};
    hipError_t e = hipMemcpyAsync(&hs, ctx->d_state, sizeof(hs), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    const int32_t zero = 0;
    if (e == hipSuccess && hs.err_latched != 0)
        e = hipMemcpyAsync(reinterpret_cast<char *>(ctx->d_state) + offsetof(DevState, err_latched),
                           &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "lad_device_status");
    const int32_t b = hs.err_latched;
    *status = (b & 1)   ? LAD_ERR_PAIRS
              : (b & 2) ? LAD_ERR_CAPACITY
              : (b & 4) ? LAD_ERR_STATE
              : (b & 8) ? LAD_ERR_NONFINITE
                        : LAD_OK;
    return LAD_OK;
}

lad_status lad_set_debug(lad_ctx *ctx, int32_t flags)
{
    if (!ctx) return fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (flags & ~LAD_DEBUG_NONFINITE) return fail(ctx, LAD_ERR_ARG, "unknown debug flag");
    ctx->debug_flags = flags;
    return LAD_OK;
}

const char *lad_last_error(const lad_ctx *ctx) { return ctx ? ctx->err.c_str() : g_build_error.c_str(); }

const char *lad_status_string(lad_status s)
{
    switch (s) {
    case LAD_OK: return "LAD_OK";
    case LAD_ERR_ARG: return "LAD_ERR_ARG";
    case LAD_ERR_CAPACITY: return "LAD_ERR_CAPACITY";
    case LAD_ERR_OOM: return "LAD_ERR_OOM";
    case LAD_ERR_HIP: return "LAD_ERR_HIP";
    case LAD_ERR_STATE: return "LAD_ERR_STATE";
    case LAD_ERR_PAIRS: return "LAD_ERR_PAIRS";
    case LAD_ERR_NONFINITE: return "LAD_ERR_NONFINITE";
    }
    return "LAD_ERR_UNKNOWN";
}

void lad_destroy(lad_ctx *ctx)
{
    if (!ctx) return;
    (void)host_sync(ctx, ctx->stream);
    free_all(ctx);
    delete ctx;
}

}  // extern "C"
