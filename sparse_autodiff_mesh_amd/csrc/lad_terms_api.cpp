// lad_terms_api.cpp -- the C ABI of the term front end (include/lad_terms.h):
// argument checks, pattern and incidence construction, and launch order.
// Every argument is checked on the host before anything touches the GPU;
// eval and hvp enqueue on the caller's stream and never synchronise.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "lad_terms.h"
#include "lad_terms_internal.h"

using namespace lad;
using namespace lad::terms;

struct lad_terms_ctx {
    int32_t nv = 0;
    lad_dtype dtype = LAD_F32;
    int32_t es = 4;
    int32_t set = 0;
    int32_t fused = 1;
    int32_t nterms = 0;
    TermInfo info[kMaxTerms] = {};
    int64_t nnzb = 0;
    int32_t nchunk = 0, lds_blocks = 0, lds_bytes = 0;
    int32_t grid_eval = 0, grid_hvp = 0;
    int32_t *d_rp = nullptr, *d_ci = nullptr, *d_diag = nullptr;
    PatchHdr *d_chunk = nullptr;
    int32_t *d_inc_ptr[kMaxTerms] = {};
    TermInc *d_inc[kMaxTerms] = {};
    unsigned char *d_inl[kMaxTerms] = {};   // inline records (small stencils)
    unsigned char *d_inl_sl[kMaxTerms] = {};  // the same, transposed per slice
    int32_t *d_sl_ptr[kMaxTerms] = {};        // and the slices' offsets
    int32_t *d_elems[kMaxTerms] = {};
    void *d_consts[kMaxTerms] = {};
    double *d_epart = nullptr;
    std::vector<void *> allocs;
    std::string err;
    int64_t host_syncs = 0;  // host synchronisations made for this context
};

namespace {

thread_local std::string g_terms_build_error;

constexpr int32_t kChunkRows = kRowThreads;
constexpr int32_t kChunkBlocks = 512;   // LDS staging per workgroup, in blocks
constexpr int32_t kMaxRowBlocks = 256;  // column offsets are stored in 8 bits

// Every host synchronisation of this front end goes through here and is
// counted (lad_terms_host_syncs).
hipError_t host_sync(lad_terms_ctx *ctx, hipStream_t s)
{
    if (ctx) ++ctx->host_syncs;
    return hipStreamSynchronize(s);
}

lad_status fail(lad_terms_ctx *ctx, lad_status s, const std::string &msg)
{
    if (ctx) ctx->err = msg;
    else g_terms_build_error = msg;
    return s;
}

template <typename P>
hipError_t dev_alloc(lad_terms_ctx *ctx, P **p, size_t bytes)
{
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes > 0 ? bytes : 16);
    if (e == hipSuccess) {
        ctx->allocs.push_back(q);
        *p = static_cast<P *>(q);
    }
    return e;
}

void free_all(lad_terms_ctx *ctx)
{
    for (void *p : ctx->allocs) (void)hipFree(p);
    ctx->allocs.clear();
}

template <typename P>
hipError_t upload(lad_terms_ctx *ctx, P **dst, const std::vector<P> &src, hipStream_t s)
{
    hipError_t e = dev_alloc(ctx, dst, src.size() * sizeof(P));
    if (e == hipSuccess && !src.empty())
        e = hipMemcpyAsync(*dst, src.data(), src.size() * sizeof(P), hipMemcpyHostToDevice, s);
    return e;
}

std::string check_desc(const lad_terms_desc *d, int nterms, const TermInfo *info)
{
    if (!d) return "desc is NULL";
    if (d->nv <= 0) return "nv must be >= 1";
    if (d->dtype != LAD_F32 && d->dtype != LAD_F64) return "dtype must be LAD_F32 or LAD_F64";
    if (nterms == 0) return "unknown term set " + std::to_string(d->set);
    if (d->fused != 0 && d->fused != 1) return "fused must be 0 or 1";
    if (d->nblocks != nterms)
        return "nblocks must be " + std::to_string(nterms) + " for this set";
    if (!d->blocks) return "blocks is NULL";
    for (int t = 0; t < nterms; ++t) {
        const lad_term_block &b = d->blocks[t];
        const int K = info[t].arity, NC = info[t].nconst;
        const std::string who = std::string("term ") + info[t].name + ": ";
        if (b.count < 0) return who + "count must be >= 0";
        if (b.count == 0) continue;
        if (!b.elems) return who + "elems is NULL";
        if (NC > 0 && !b.consts) return who + "consts is NULL";
        for (int64_t e = 0; e < b.count; ++e) {
            const int32_t *v = b.elems + e * K;
            for (int i = 0; i < K; ++i) {
                if (v[i] < 0 || v[i] >= d->nv) return who + "vertex id out of range";
                for (int j = 0; j < i; ++j)
                    if (v[j] == v[i]) return who + "an element repeats a vertex";
            }
            for (int q = 0; q < NC; ++q)
                if (!std::isfinite(b.consts[e * NC + q])) return who + "non-finite constant";
        }
    }
    return "";
}

// Position of column b in row a of the pattern, or -1.
int32_t find_pos(const std::vector<int32_t> &rp, const std::vector<int32_t> &ci, int32_t a,
                 int32_t b)
{
    const auto lo = ci.begin() + rp[size_t(a)], hi = ci.begin() + rp[size_t(a) + 1];
    const auto it = std::lower_bound(lo, hi, b);
    return (it != hi && *it == b) ? int32_t(it - lo) : -1;
}

template <typename T>
lad_status build_typed(lad_terms_ctx *ctx, const lad_terms_desc *d, hipStream_t s)
{
    const int32_t nv = d->nv;
    // ---- pattern on the GPU from every element's vertex pairs
    std::vector<int32_t> pairs;
    for (int t = 0; t < ctx->nterms; ++t) {
        const lad_term_block &b = d->blocks[t];
        const int K = ctx->info[t].arity;
        for (int64_t e = 0; e < b.count; ++e)
            for (int i = 0; i < K; ++i)
                for (int j = i + 1; j < K; ++j) {
                    pairs.push_back(b.elems[e * K + i]);
                    pairs.push_back(b.elems[e * K + j]);
                }
    }
    const int64_t npairs = int64_t(pairs.size() / 2);
    if (int64_t(nv) + 2 * npairs >= (int64_t(1) << 31))
        return fail(nullptr, LAD_ERR_ARG, "too many element vertex pairs for int32 indices");
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
    PatternScratch sc{};
    int32_t *d_pairs = nullptr;
    hipError_t e = tmp_alloc(&d_pairs, pairs.size());
    if (e == hipSuccess) e = tmp_alloc(&sc.cnt, size_t(nv));
    if (e == hipSuccess) e = tmp_alloc(&sc.off, size_t(nv) + 1);
    if (e == hipSuccess) e = tmp_alloc(&sc.raw, size_t(nv) + 2 * size_t(npairs));
    if (e == hipSuccess) e = tmp_alloc(&sc.cur, size_t(nv));
    if (e == hipSuccess) e = tmp_alloc(&sc.ucnt, size_t(nv));
    if (e == hipSuccess) e = tmp_alloc(&sc.tmp, size_t(scan_tmp_size(nv)));
    if (e == hipSuccess) e = dev_alloc(ctx, &ctx->d_rp, (size_t(nv) + 1) * 4);
    if (e != hipSuccess) {
        free_temps();
        return fail(nullptr, LAD_ERR_OOM, std::string("device allocation: ") + hipGetErrorString(e));
    }
    if (!pairs.empty())
        e = hipMemcpyAsync(d_pairs, pairs.data(), pairs.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_pattern_count(nv, 0, nullptr, int32_t(npairs), d_pairs, sc, s);
    if (e == hipSuccess) e = launch_pattern_fill(nv, 0, nullptr, int32_t(npairs), d_pairs, sc, s);
    if (e == hipSuccess) e = launch_pattern_unique(nv, sc, s);
    if (e == hipSuccess) e = launch_scan(sc.ucnt, ctx->d_rp, nv, sc.tmp, s);
    std::vector<int32_t> rp(static_cast<size_t>(nv) + 1);
    if (e == hipSuccess)
        e = hipMemcpyAsync(rp.data(), ctx->d_rp, rp.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) {
        free_temps();
        return fail(nullptr, LAD_ERR_HIP, std::string("pattern build: ") + hipGetErrorString(e));
    }
    ctx->nnzb = rp[size_t(nv)];
    if (ctx->nnzb * 9 >= (int64_t(1) << 31)) {
        free_temps();
        return fail(nullptr, LAD_ERR_ARG, "pattern too large for int32 value indices");
    }
    e = dev_alloc(ctx, &ctx->d_ci, size_t(ctx->nnzb) * 4);
    if (e == hipSuccess) e = launch_pattern_compact(nv, sc, ctx->d_rp, ctx->d_ci, s);
    std::vector<int32_t> ci(static_cast<size_t>(ctx->nnzb));
    if (e == hipSuccess && !ci.empty())
        e = hipMemcpyAsync(ci.data(), ctx->d_ci, ci.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    free_temps();
    if (e != hipSuccess)
        return fail(nullptr, LAD_ERR_HIP, std::string("pattern compaction: ") + hipGetErrorString(e));

    // ---- diagonal offsets, row length limit, chunks
    std::vector<int32_t> diag(static_cast<size_t>(nv));
    for (int32_t a = 0; a < nv; ++a) {
        if (rp[size_t(a) + 1] - rp[size_t(a)] > kMaxRowBlocks)
            return fail(nullptr, LAD_ERR_ARG,
                        "vertex " + std::to_string(a) + " has a row of more than " +
                            std::to_string(kMaxRowBlocks) + " blocks");
        diag[size_t(a)] = find_pos(rp, ci, a, a);
    }
    std::vector<PatchHdr> chunks;
    int32_t maxblk = 0;
    for (int32_t v0 = 0; v0 < nv;) {
        int32_t n = 0, blk = 0;
        while (n < kChunkRows && v0 + n < nv) {
            const int32_t len = rp[size_t(v0 + n) + 1] - rp[size_t(v0 + n)];
            if (blk + len > kChunkBlocks) break;
            blk += len;
            ++n;
        }
        PatchHdr h;
        std::memset(&h, 0, sizeof(h));
        h.v0 = v0;
        h.nown = n;
        h.blk0 = rp[size_t(v0)];
        h.nblk = blk;
        h.amap_cap = kChunkBlocks;
        chunks.push_back(h);
        maxblk = std::max(maxblk, blk);
        v0 += n;
    }
    ctx->nchunk = int32_t(chunks.size());
    ctx->lds_blocks = std::max<int32_t>(maxblk, 1);
    ctx->lds_bytes = int32_t(((int64_t(ctx->lds_blocks) * 9 * int64_t(sizeof(T)) + 16) + 15) &
                             ~int64_t(15));

    // ---- per term: incidence (rows in vertex order, elements by id), elements, constants
    e = upload(ctx, &ctx->d_diag, diag, s);
    if (e == hipSuccess) e = upload(ctx, &ctx->d_chunk, chunks, s);
    // first writer of every block of each row, in term order, then record
    // order (records of a row are filled in element order)
    std::vector<unsigned char> written(static_cast<size_t>(ctx->nnzb), 0);
    for (int t = 0; t < ctx->nterms && e == hipSuccess; ++t) {
        const lad_term_block &b = d->blocks[t];
        const int K = ctx->info[t].arity, NC = ctx->info[t].nconst;
        std::vector<int32_t> ptr(size_t(nv) + 1, 0);
        for (int64_t el = 0; el < int64_t(b.count) * K; ++el) ptr[size_t(b.elems[el]) + 1] += 1;
        for (int32_t a = 0; a < nv; ++a) ptr[size_t(a) + 1] += ptr[size_t(a)];
        std::vector<TermInc> inc(static_cast<size_t>(ptr[size_t(nv)]));
        std::vector<int32_t> cur(ptr.begin(), ptr.end() - 1);
        for (int64_t el = 0; el < b.count; ++el) {
            const int32_t *v = b.elems + el * K;
            for (int i = 0; i < K; ++i) {
                const int32_t a = v[i];
                TermInc r;
                r.e = int32_t(el);
                r.pk = uint32_t(i);
                for (int q = 1; q < K; ++q) {
                    const int32_t pos = find_pos(rp, ci, a, v[(i + q) % K]);
                    if (pos < 0) return fail(nullptr, LAD_ERR_HIP, "element block missing from pattern");
                    r.pk |= uint32_t(pos) << (8 * q);
                    unsigned char &wr = written[size_t(rp[size_t(a)] + pos)];
                    if (!wr) {
                        r.pk |= 1u << (1 + q);
                        wr = 1;
                    }
                }
                inc[size_t(cur[size_t(a)]++)] = r;
            }
        }
        e = upload(ctx, &ctx->d_inc_ptr[t], ptr, s);
        if (K <= kInlineVerts) {
            // each record carries the element's other vertex and constants
            // (InlineRec<T, NC>: pk, other, c[NC], padded to 8 bytes); rows
            // in order for the explicit pass, and for the product
            // transposed per slice of kTermSliceRows rows: slice q holds
            // kTermSliceRows x (its rows' largest count) records, record j
            // of row a at sl_ptr[q] + kTermSliceRows j + a % kTermSliceRows
            // (padding records are zero and never evaluated)
            const size_t rb = inline_rec_bytes<T>(NC);
            std::vector<unsigned char> rows(inc.size() * rb, 0);
            const int64_t nsl = (int64_t(nv) + kTermSliceRows - 1) / kTermSliceRows;
            std::vector<int32_t> slp(size_t(nsl) + 1, 0);
            for (int64_t q = 0; q < nsl; ++q) {
                int32_t w = 0;
                for (int64_t a = q * kTermSliceRows;
                     a < std::min<int64_t>(nv, (q + 1) * kTermSliceRows); ++a)
                    w = std::max(w, ptr[size_t(a) + 1] - ptr[size_t(a)]);
                const int64_t end = int64_t(slp[size_t(q)]) + int64_t(kTermSliceRows) * w;
                if (end > INT32_MAX) return fail(nullptr, LAD_ERR_CAPACITY, "too many element records");
                slp[size_t(q) + 1] = int32_t(end);
            }
            std::vector<unsigned char> recs(size_t(slp[size_t(nsl)]) * rb, 0);
            for (int32_t a = 0; a < nv; ++a)
            for (int32_t k = ptr[size_t(a)]; k < ptr[size_t(a) + 1]; ++k) {
                const int64_t j = k - ptr[size_t(a)];  // the record's place in its row
                const int64_t slot = slp[size_t(a / kTermSliceRows)] + j * kTermSliceRows +
                                     a % kTermSliceRows;
                unsigned char *r = rows.data() + size_t(k) * rb;
                const int64_t el = inc[k].e;
                const int i = int(inc[k].pk & 3u);
                const int32_t other = K == 2 ? b.elems[el * 2 + (1 - i)] : 0;
                std::memcpy(r, &inc[k].pk, 4);
                std::memcpy(r + 4, &other, 4);
                for (int q = 0; q < NC; ++q) {
                    const T c = T(b.consts[el * NC + q]);
                    std::memcpy(r + 8 + size_t(q) * sizeof(T), &c, sizeof(T));
                }
                std::memcpy(recs.data() + size_t(slot) * rb, r, rb);
            }
            if (e == hipSuccess) e = upload(ctx, &ctx->d_inl[t], rows, s);
            if (e == hipSuccess) e = upload(ctx, &ctx->d_inl_sl[t], recs, s);
            if (e == hipSuccess) e = upload(ctx, &ctx->d_sl_ptr[t], slp, s);
        } else {
            std::vector<int32_t> elems(b.elems, b.elems + int64_t(b.count) * K);
            std::vector<T> consts(size_t(b.count) * size_t(NC));
            for (size_t q = 0; q < consts.size(); ++q) consts[q] = T(b.consts[q]);
            if (e == hipSuccess) e = upload(ctx, &ctx->d_inc[t], inc, s);
            if (e == hipSuccess) e = upload(ctx, &ctx->d_elems[t], elems, s);
            T *dc = nullptr;
            if (e == hipSuccess) e = upload(ctx, &dc, consts, s);
            ctx->d_consts[t] = dc;
        }
    }
    if (e == hipSuccess)
        e = terms_grid<T>(ctx->set, ctx->lds_bytes, ctx->nchunk, nv, &ctx->grid_eval,
                          &ctx->grid_hvp);
    if (e == hipSuccess)
        e = dev_alloc(ctx, &ctx->d_epart, size_t(ctx->nterms) * size_t(ctx->grid_eval) * 8);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return fail(nullptr, LAD_ERR_HIP, std::string("upload: ") + hipGetErrorString(e));
    return LAD_OK;
}

template <typename T>
TermsArgs<T> args_of(const lad_terms_ctx *ctx)
{
    TermsArgs<T> a{};
    a.chunk = ctx->d_chunk;
    a.nchunk = ctx->nchunk;
    a.nv = ctx->nv;
    a.rp = ctx->d_rp;
    a.ci = ctx->d_ci;
    a.diag = ctx->d_diag;
    a.lds_blocks = ctx->lds_blocks;
    for (int t = 0; t < ctx->nterms; ++t) {
        a.t[t].inc_ptr = ctx->d_inc_ptr[t];
        a.t[t].inc = ctx->d_inc[t];
        a.t[t].inl = ctx->d_inl[t];
        a.t[t].inl_sl = ctx->d_inl_sl[t];
        a.t[t].sl_ptr = ctx->d_sl_ptr[t];
        a.t[t].elems = ctx->d_elems[t];
        a.t[t].consts = static_cast<const T *>(ctx->d_consts[t]);
    }
    return a;
}

}  // namespace

extern "C" {

lad_status lad_terms_describe(int32_t set, int32_t term, int32_t *nterms, int32_t *arity,
                              int32_t *nconst, const char **name)
{
    TermInfo info[kMaxTerms];
    const int n = set_terms(set, info);
    if (n == 0) return LAD_ERR_ARG;
    if (nterms) *nterms = n;
    if (term < 0 || term >= n) return (arity || nconst || name) ? LAD_ERR_ARG : LAD_OK;
    if (arity) *arity = info[term].arity;
    if (nconst) *nconst = info[term].nconst;
    if (name) *name = info[term].name;
    return LAD_OK;
}

lad_status lad_terms_build(const lad_terms_desc *desc, void *hip_stream, lad_terms_ctx **out)
{
    g_terms_build_error.clear();
    if (!out) return fail(nullptr, LAD_ERR_ARG, "out is NULL");
    *out = nullptr;
    TermInfo info[kMaxTerms];
    const int nterms = desc ? set_terms(desc->set, info) : 0;
    const std::string why = check_desc(desc, nterms, info);
    if (!why.empty()) return fail(nullptr, LAD_ERR_ARG, why);
    lad_terms_ctx *ctx = new lad_terms_ctx();
    ctx->nv = desc->nv;
    ctx->dtype = lad_dtype(desc->dtype);
    ctx->es = desc->dtype == LAD_F64 ? 8 : 4;
    ctx->set = desc->set;
    ctx->fused = desc->fused;
    ctx->nterms = nterms;
    for (int t = 0; t < nterms; ++t) ctx->info[t] = info[t];
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const lad_status st = desc->dtype == LAD_F64 ? build_typed<double>(ctx, desc, s)
                                                 : build_typed<float>(ctx, desc, s);
    if (st != LAD_OK) {
        free_all(ctx);
        delete ctx;
        return st;
    }
    *out = ctx;
    return LAD_OK;
}

lad_status lad_terms_eval(lad_terms_ctx *ctx, const void *d_x, double *d_energy, void *d_grad,
                          void *d_hvals, int64_t hvals_capacity_blocks, void *hip_stream)
{
    if (!ctx) return LAD_ERR_ARG;
    if (!d_x || !d_grad || !d_hvals) return fail(ctx, LAD_ERR_ARG, "x, grad or hvals is NULL");
    if (hvals_capacity_blocks < ctx->nnzb)
        return fail(ctx, LAD_ERR_ARG, "hvals capacity " + std::to_string(hvals_capacity_blocks) +
                                          " < nnzb " + std::to_string(ctx->nnzb));
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (ctx->dtype == LAD_F64)
        e = launch_terms_eval<double>(ctx->set, ctx->fused, args_of<double>(ctx),
                                      static_cast<const double *>(d_x), static_cast<double *>(d_grad),
                                      static_cast<double *>(d_hvals), EnergySink{ctx->d_epart, 0},
                                      ctx->grid_eval, ctx->lds_bytes, s);
    else
        e = launch_terms_eval<float>(ctx->set, ctx->fused, args_of<float>(ctx),
                                     static_cast<const float *>(d_x), static_cast<float *>(d_grad),
                                     static_cast<float *>(d_hvals), EnergySink{ctx->d_epart, 0},
                                     ctx->grid_eval, ctx->lds_bytes, s);
    const int32_t nparts = (ctx->fused || ctx->nterms == 1) ? ctx->grid_eval
                                                             : ctx->nterms * ctx->grid_eval;
    if (e == hipSuccess && d_energy) e = launch_energy_reduce(ctx->d_epart, nparts, d_energy, s);
    if (e != hipSuccess) return fail(ctx, LAD_ERR_HIP, std::string("eval: ") + hipGetErrorString(e));
    return LAD_OK;
}

lad_status lad_terms_hvp(lad_terms_ctx *ctx, const void *d_x, const void *d_v, void *d_y,
                         void *hip_stream)
{
    if (!ctx) return LAD_ERR_ARG;
    if (!d_x || !d_v || !d_y) return fail(ctx, LAD_ERR_ARG, "x, v or y is NULL");
    if (d_y == d_x || d_y == d_v) return fail(ctx, LAD_ERR_ARG, "y must not alias x or v");
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (ctx->dtype == LAD_F64)
        e = launch_terms_hvp<double>(ctx->set, ctx->fused, args_of<double>(ctx),
                                     static_cast<const double *>(d_x),
                                     static_cast<const double *>(d_v), static_cast<double *>(d_y),
                                     ctx->grid_hvp, s);
    else
        e = launch_terms_hvp<float>(ctx->set, ctx->fused, args_of<float>(ctx),
                                    static_cast<const float *>(d_x),
                                    static_cast<const float *>(d_v), static_cast<float *>(d_y),
                                    ctx->grid_hvp, s);
    if (e != hipSuccess) return fail(ctx, LAD_ERR_HIP, std::string("hvp: ") + hipGetErrorString(e));
    return LAD_OK;
}

lad_status lad_terms_get_pattern(lad_terms_ctx *ctx, int64_t *nnzb, const int32_t **d_row_ptr,
                                 const int32_t **d_col_idx)
{
    if (!ctx) return LAD_ERR_ARG;
    if (!nnzb || !d_row_ptr || !d_col_idx) return fail(ctx, LAD_ERR_ARG, "NULL output");
    *nnzb = ctx->nnzb;
    *d_row_ptr = ctx->d_rp;
    *d_col_idx = ctx->d_ci;
    return LAD_OK;
}

lad_status lad_terms_copy_pattern(lad_terms_ctx *ctx, void *hip_stream, int32_t *d_row_ptr,
                                  int32_t *d_col_idx, int64_t col_capacity, int64_t *nnzb)
{
    if (!ctx) return LAD_ERR_ARG;
    if (!d_row_ptr || !d_col_idx || !nnzb) return fail(ctx, LAD_ERR_ARG, "NULL pointer");
    *nnzb = ctx->nnzb;
    if (col_capacity < ctx->nnzb)
        return fail(ctx, LAD_ERR_CAPACITY, "col_capacity " + std::to_string(col_capacity) +
                                               " < nnzb " + std::to_string(ctx->nnzb));
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipMemcpyAsync(d_row_ptr, ctx->d_rp, (size_t(ctx->nv) + 1) * 4,
                                  hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(d_col_idx, ctx->d_ci, size_t(ctx->nnzb) * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = host_sync(ctx, s);
    if (e != hipSuccess) return fail(ctx, LAD_ERR_HIP, std::string("copy: ") + hipGetErrorString(e));
    return LAD_OK;
}

const char *lad_terms_last_error(const lad_terms_ctx *ctx)
{
    return ctx ? ctx->err.c_str() : g_terms_build_error.c_str();
}

int64_t lad_terms_host_syncs(const lad_terms_ctx *ctx) { return ctx ? ctx->host_syncs : -1; }

void lad_terms_destroy(lad_terms_ctx *ctx)
{
    if (!ctx) return;
    free_all(ctx);
    delete ctx;
}

}  // extern "C"
