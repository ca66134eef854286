// lad_patch.cpp -- host-side mesh patcher.
//
// Splits the vertices into patches sized for one workgroup's LDS and emits,
// per patch, the element records its kernel evaluates.  Source: page
// "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", key design 2 (mesh cut into patches that fit the memory
// hierarchy, one thread block per patch, ribbon/ghost elements for
// cross-patch neighbours, patch-local staging of connectivity and
// attributes).
//
// Design on gfx950 (differs from the page's RXMesh patches):
//  * A patch owns a CONTIGUOUS range of vertex ids, so the block-CSR rows it
//    owns form one contiguous range of the Hessian value array: the kernel
//    accumulates that whole range in LDS and writes it back as one coalesced
//    stream, and no block is ever zero-filled or atomically updated in HBM.
//  * Owner computes: every element that touches an owned vertex is evaluated
//    by that patch, and only the owned rows are written.  Elements on a patch
//    boundary are evaluated once per patch that owns one of their vertices;
//    ribbon vertices are the non-owned vertices of those elements.
//  * Records inside a patch are greedily coloured so that no two elements of
//    one colour share an owned vertex.  The default assembly runs the
//    colours one after another with plain LDS read-add-write (a fixed
//    summation order); the LDS-atomic assembly uses LDS float atomics, and
//    the same order keeps lanes of one wave off the same addresses.
//  * Element-once plans (the page's own decomposition, key designs 3-4:
//    assembly by atomic scatter-add into the preallocated pattern) keep
//    each element in one patch only, the one owning its lowest vertex id.
//    Its contributions to the rows of other patches go to HBM with global
//    atomics; the plan lists those rows' blocks and vertices so they can be
//    zeroed before the kernel and added to (not stored) by their owner.
#include <algorithm>
#include <climits>
#include <cstring>

#include "lad_internal.h"

namespace lad {

static int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

int32_t amap_capacity(int nblk) { return nblk + std::max(32, nblk / 8); }

// Region order must match the carving in the kernels.
int64_t lds_eval_bytes(int es, int nblk, int nown, int nloc, int amap_cap)
{
    int64_t b = 0;
    b += align16((int64_t(nblk) * 9 + 4) * es);  // H chunk (+ vector pad)
    b += align16(int64_t(nown) * 3 * es + 4 * es);  // g chunk (+ vector pad)
    b += align16(int64_t(nloc) * 3 * es);        // staged positions
    b += align16(int64_t(nown) * 2);             // diagonal block table
    b += align16(int64_t(amap_cap) * 2);         // active->base block map
    b += 64;                                     // energy reduction
    return b;
}

int64_t lds_hvp_bytes(int es, int nown, int nloc)
{
    int64_t b = 0;
    b += align16(int64_t(nloc) * 3 * es);        // x
    b += align16(int64_t(nloc) * 3 * es);        // v
    b += align16(int64_t(nown) * 3 * es);        // y accumulators
    b += 64;
    return b;
}

namespace {

int32_t find_pos(const int32_t *row_ptr, const int32_t *col_idx, int32_t a, int32_t b)
{
    const int32_t *lo = col_idx + row_ptr[a], *hi = col_idx + row_ptr[a + 1];
    const int32_t *it = std::lower_bound(lo, hi, b);
    if (it == hi || *it != b) return -1;
    return int32_t(it - lo);
}

// Greedy colouring of records that touch `m` owned vertices each.  `owned`
// returns the owned-local ids of record r (negative = not owned).  Returns
// the colour count, or -1 if more than kMaxColors are needed.
template <class OwnedFn>
int colour_records(int nrec, int nown, int m, OwnedFn owned, std::vector<int> &colour)
{
    constexpr int W = kMaxColors / 64;
    std::vector<uint64_t> used(size_t(nown) * W, 0);
    colour.assign(nrec, 0);
    int ncol = 0;
    int ids[3];
    for (int r = 0; r < nrec; ++r) {
        owned(r, ids);
        uint64_t mask[W] = {};
        for (int i = 0; i < m; ++i)
            if (ids[i] >= 0)
                for (int w = 0; w < W; ++w) mask[w] |= used[size_t(ids[i]) * W + w];
        int c = -1;
        for (int w = 0; w < W && c < 0; ++w)
            if (~mask[w]) c = 64 * w + __builtin_ctzll(~mask[w]);
        if (c < 0) return -1;
        colour[r] = c;
        for (int i = 0; i < m; ++i)
            if (ids[i] >= 0) used[size_t(ids[i]) * W + c / 64] |= uint64_t(1) << (c % 64);
        ncol = std::max(ncol, c + 1);
    }
    return ncol;
}

}  // namespace

std::string build_plan(const PlanInput &in, Plan &out)
{
    const int32_t nv = in.nv;
    const int es = in.elem_size;
    const int32_t *rp = in.row_ptr, *ci = in.col_idx;
    out = Plan();
    out.elem_size = es;
    if (nv <= 0) return "nv must be positive";

    // ---- 1. patch boundaries: greedy over vertex ids under the LDS budget
    std::vector<int32_t> stamp(nv, -1);
    std::vector<int32_t> starts;
    {
        int32_t pid = 0, nown = 0, nblk = 0, nloc = 0;
        starts.push_back(0);
        for (int32_t v = 0; v < nv; ++v) {
            const int32_t len = rp[v + 1] - rp[v];
            int32_t fresh = 0;
            for (int32_t k = rp[v]; k < rp[v + 1]; ++k) fresh += stamp[ci[k]] != pid;
            auto fits = [&](int32_t o, int32_t b, int32_t l) {
                return b <= kMaxLocal - 1 && l <= kMaxLocal - 1 &&
                       amap_capacity(b) <= kMaxLocal &&
                       lds_eval_bytes(es, b, o, l, amap_capacity(b)) <= in.lds_budget;
            };
            if (nown > 0 && !fits(nown + 1, nblk + len, nloc + fresh)) {
                ++pid;
                starts.push_back(v);
                nown = nblk = nloc = 0;
                fresh = len;  // nothing stamped with the new id yet
            }
            if (!fits(nown + 1, nblk + len, nloc + fresh))
                return "vertex " + std::to_string(v) + " has a row too long for the LDS budget";
            for (int32_t k = rp[v]; k < rp[v + 1]; ++k) stamp[ci[k]] = pid;
            nown += 1;
            nblk += len;
            nloc += fresh;
        }
        starts.push_back(nv);
    }
    const int32_t np = int32_t(starts.size()) - 1;
    out.vpatch.resize(nv);
    for (int32_t p = 0; p < np; ++p)
        for (int32_t v = starts[p]; v < starts[p + 1]; ++v) out.vpatch[v] = p;

    // ---- 2. element -> patch incidence (counting sort by patch): every
    // patch owning one of the element's vertices, or with element_once the
    // patch of its lowest vertex id only (patches are ascending id ranges)
    const bool once = in.element_once != 0;
    auto patches_of = [&](const int32_t *ev, int m, int32_t *ps) {
        int cnt = 0;
        if (once) {
            int32_t lo = ev[0];
            for (int i = 1; i < m; ++i) lo = std::min(lo, ev[i]);
            ps[cnt++] = out.vpatch[lo];
            return cnt;
        }
        for (int i = 0; i < m; ++i) {
            int32_t p = out.vpatch[ev[i]];
            bool dup = false;
            for (int j = 0; j < cnt; ++j) dup |= ps[j] == p;
            if (!dup) ps[cnt++] = p;
        }
        return cnt;
    };
    auto emit_lists = [&](int32_t ne, int m, const int32_t *ev, std::vector<int32_t> &off,
                          std::vector<int32_t> &lst) {
        off.assign(size_t(np) + 1, 0);
        int32_t ps[3];
        for (int32_t e = 0; e < ne; ++e) {
            const int cnt = patches_of(ev + int64_t(e) * m, m, ps);
            for (int j = 0; j < cnt; ++j) off[ps[j] + 1] += 1;
        }
        for (int32_t p = 0; p < np; ++p) off[p + 1] += off[p];
        lst.assign(off[np], 0);
        std::vector<int32_t> cur(off.begin(), off.end() - 1);
        for (int32_t e = 0; e < ne; ++e) {
            const int cnt = patches_of(ev + int64_t(e) * m, m, ps);
            for (int j = 0; j < cnt; ++j) lst[cur[ps[j]]++] = e;
        }
    };
    std::vector<int32_t> soff, slst, foff, flst;
    if (in.ns > 0) emit_lists(in.ns, 2, in.springs, soff, slst);
    else soff.assign(size_t(np) + 1, 0);
    if (in.face_energy && in.nf > 0) emit_lists(in.nf, 3, in.faces, foff, flst);
    else foff.assign(size_t(np) + 1, 0);

    // ---- 3. per patch: local numbering, records, colours, LDS sizes
    std::vector<int32_t> local(nv, -1);
    std::fill(stamp.begin(), stamp.end(), -1);
    out.hdr.resize(np);
    out.diag_rel.assign(nv, kNone);
    out.spr.reserve(slst.size());
    out.spr_src.reserve(slst.size());
    out.fac.reserve(flst.size());
    out.fac_src.reserve(flst.size());
    std::vector<int> colour;
    std::vector<int32_t> order;
    if (once) {
        out.blk_flag.assign(size_t(rp[nv]), 0);
        out.vtx_flag.assign(size_t(nv), 0);
        out.spr_gblk.reserve(2 * slst.size());
        out.fac_gblk.reserve(9 * flst.size());
    }
    // global block (a, b), flagged as receiving a foreign contribution
    auto foreign_blk = [&](int32_t a, int32_t b) -> int32_t {
        const int32_t pos = find_pos(rp, ci, a, b);
        if (pos < 0) return -1;
        out.blk_flag[size_t(rp[a] + pos)] = 1;
        out.vtx_flag[size_t(a)] = 1;
        return rp[a] + pos;
    };
    for (int32_t p = 0; p < np; ++p) {
        PatchHdr &h = out.hdr[p];
        std::memset(&h, 0, sizeof(h));
        const int32_t v0 = starts[p], v1 = starts[p + 1], nown = v1 - v0;
        h.v0 = v0;
        h.nown = nown;
        h.blk0 = rp[v0];
        h.nblk = rp[v1] - rp[v0];
        // local ids: owned first, then ribbon (ascending global id)
        std::vector<int32_t> rib;
        for (int32_t v = v0; v < v1; ++v) {
            stamp[v] = p;
            local[v] = v - v0;
        }
        auto add_rib = [&](int32_t u) {
            if (stamp[u] != p) {
                stamp[u] = p;
                rib.push_back(u);
            }
        };
        if (once) {
            // the non-owned vertices of the patch's own elements
            for (int32_t i = soff[p]; i < soff[p + 1]; ++i)
                for (int j = 0; j < 2; ++j) add_rib(in.springs[2 * int64_t(slst[i]) + j]);
            for (int32_t i = foff[p]; i < foff[p + 1]; ++i)
                for (int j = 0; j < 3; ++j) add_rib(in.faces[3 * int64_t(flst[i]) + j]);
        } else {
            for (int32_t v = v0; v < v1; ++v)
                for (int32_t k = rp[v]; k < rp[v + 1]; ++k) add_rib(ci[k]);
        }
        std::sort(rib.begin(), rib.end());
        for (size_t i = 0; i < rib.size(); ++i) local[rib[i]] = nown + int32_t(i);
        h.rib_off = int32_t(out.rib.size());
        h.nrib = int32_t(rib.size());
        out.rib.insert(out.rib.end(), rib.begin(), rib.end());
        const int32_t nloc = nown + h.nrib;

        for (int32_t v = v0; v < v1; ++v) {
            int32_t pos = find_pos(rp, ci, v, v);
            if (pos < 0) return "diagonal block missing";
            out.diag_rel[v] = uint16_t(rp[v] - h.blk0 + pos);
        }
        auto slot = [&](int32_t a, int32_t b) -> uint16_t {
            if (a < v0 || a >= v1) return kNone;
            int32_t pos = find_pos(rp, ci, a, b);
            return pos < 0 ? kNone : uint16_t(rp[a] - h.blk0 + pos);
        };

        // springs
        h.col_off = int32_t(out.col_bounds.size());
        {
            const int32_t n = soff[p + 1] - soff[p];
            const int32_t *lst = slst.data() + soff[p];
            int nc = colour_records(n, nown, 2, [&](int r, int *ids) {
                const int32_t *s = in.springs + 2 * int64_t(lst[r]);
                for (int i = 0; i < 2; ++i) {
                    int32_t l = local[s[i]];
                    ids[i] = l < nown ? l : -1;
                }
            }, colour);
            if (nc < 0) return "too many spring colours in a patch";
            order.resize(n);
            for (int32_t r = 0; r < n; ++r) order[r] = r;
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t x, int32_t y) { return colour[x] < colour[y]; });
            h.spr_off = int32_t(out.spr.size());
            h.nspr = n;
            h.nspr_col = nc;
            int32_t c = -1;
            for (int32_t i = 0; i < n; ++i) {
                const int32_t r = order[i];
                while (c < colour[r]) {
                    out.col_bounds.push_back(i);
                    ++c;
                }
                const int32_t s = lst[r];
                const int32_t a = in.springs[2 * int64_t(s)], b = in.springs[2 * int64_t(s) + 1];
                SpringRec rec;
                rec.lab = uint32_t(local[a]) | (uint32_t(local[b]) << 16);
                uint16_t sab = slot(a, b), sba = slot(b, a);
                if ((a >= v0 && a < v1 && sab == kNone) || (b >= v0 && b < v1 && sba == kNone))
                    return "spring block missing from pattern";
                rec.blk = uint32_t(sab) | (uint32_t(sba) << 16);
                out.spr.push_back(rec);
                out.spr_src.push_back(s);
                if (once) {
                    const bool fa = a < v0 || a >= v1, fb = b < v0 || b >= v1;
                    int32_t g0 = -1, g1 = -1;
                    if (fa || fb) {
                        const int32_t f = fa ? a : b, o = fa ? b : a;
                        g0 = foreign_blk(f, f);
                        g1 = foreign_blk(f, o);
                        if (g0 < 0 || g1 < 0) return "spring block missing from pattern";
                    }
                    out.spr_gblk.push_back(g0);
                    out.spr_gblk.push_back(g1);
                }
            }
            if (n > 0) out.col_bounds.push_back(n);
            else h.nspr_col = 0;
            out.max_colors = std::max(out.max_colors, h.nspr_col);
        }
        // faces
        {
            const int32_t n = foff[p + 1] - foff[p];
            const int32_t *lst = flst.data() + foff[p];
            int nc = colour_records(n, nown, 3, [&](int r, int *ids) {
                const int32_t *t = in.faces + 3 * int64_t(lst[r]);
                for (int i = 0; i < 3; ++i) {
                    int32_t l = local[t[i]];
                    ids[i] = l < nown ? l : -1;
                }
            }, colour);
            if (nc < 0) return "too many face colours in a patch";
            order.resize(n);
            for (int32_t r = 0; r < n; ++r) order[r] = r;
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t x, int32_t y) { return colour[x] < colour[y]; });
            h.fac_off = int32_t(out.fac.size());
            h.nfac = n;
            h.nfac_col = nc;
            int32_t c = -1;
            for (int32_t i = 0; i < n; ++i) {
                const int32_t r = order[i];
                while (c < colour[r]) {
                    out.col_bounds.push_back(i);
                    ++c;
                }
                const int32_t f = lst[r];
                const int32_t *t = in.faces + 3 * int64_t(f);
                FaceRec rec;
                for (int a = 0; a < 3; ++a) {
                    rec.l[a] = uint16_t(local[t[a]]);
                    for (int b = 0; b < 3; ++b) {
                        uint16_t s = slot(t[a], t[b]);
                        if (t[a] >= v0 && t[a] < v1 && s == kNone)
                            return "face block missing from pattern";
                        rec.blk[3 * a + b] = s;
                        if (once) {
                            int32_t gb = -1;
                            if (t[a] < v0 || t[a] >= v1) {
                                gb = foreign_blk(t[a], t[b]);
                                if (gb < 0) return "face block missing from pattern";
                            }
                            out.fac_gblk.push_back(gb);
                        }
                    }
                }
                out.fac.push_back(rec);
                out.fac_src.push_back(f);
            }
            if (n > 0) out.col_bounds.push_back(n);
            else h.nfac_col = 0;
            out.max_colors = std::max(out.max_colors, h.nfac_col);
        }
        h.amap_cap = amap_capacity(h.nblk);
        h.lds_eval = int32_t(lds_eval_bytes(es, h.nblk, nown, nloc, h.amap_cap));
        h.lds_hvp = int32_t(lds_hvp_bytes(es, nown, nloc));
        out.lds_eval = std::max(out.lds_eval, h.lds_eval);
        out.lds_hvp = std::max(out.lds_hvp, h.lds_hvp);
    }
    if (once) {
        for (int32_t b = 0; b < rp[nv]; ++b)
            if (out.blk_flag[size_t(b)]) out.bnd_blk.push_back(b);
        for (int32_t v = 0; v < nv; ++v)
            if (out.vtx_flag[size_t(v)]) out.bnd_vtx.push_back(v);
    }
    return "";
}

int32_t half_chunk_blocks(const std::vector<PatchHdr> &chunks, const int32_t *rp)
{
    const int32_t half = kRowsPerChunk / 2;
    int32_t most = 1;
    for (const PatchHdr &c : chunks)
        for (int32_t h0 = 0; h0 < c.nown; h0 += half) {
            const int32_t a = c.v0 + h0, b = c.v0 + std::min(c.nown, h0 + half);
            most = std::max(most, rp[b] - rp[a]);
        }
    return most;
}

// The rows of the product kernels' slices when the face term is on:
// patches of kSliceRows vertices grown breadth first over the pattern's
// adjacency (each patch seeded at the lowest vertex no patch holds yet,
// neighbours taken in column order, a new seed whenever the search runs
// dry, so every slice but the last is full).  A slice lists every face
// incident to its rows once, and a compact patch touches about 2.5 faces
// per row where 64 consecutive rows of a mesh numbered line by line touch
// 4 (512 x 512 grid: 159 against 257 faces per slice).  Padding: -1.
static void bfs_slice_rows(int32_t nv, const int32_t *rp, const int32_t *ci,
                           std::vector<int32_t> &rows)
{
    const int64_t nsl = (int64_t(nv) + kSliceRows - 1) / kSliceRows;
    rows.assign(size_t(nsl * kSliceRows), -1);
    std::vector<uint8_t> taken(size_t(nv), 0);
    std::vector<int32_t> queue;
    queue.reserve(kSliceRows);
    int32_t cursor = 0;
    for (int64_t t = 0; t < nsl; ++t) {
        int32_t n = 0;
        size_t head = 0;
        queue.clear();
        while (n < kSliceRows) {
            if (head == queue.size()) {  // the search ran dry: a new seed
                while (cursor < nv && taken[size_t(cursor)]) ++cursor;
                if (cursor == nv) break;
                taken[size_t(cursor)] = 1;
                queue.push_back(cursor);
            }
            const int32_t v = queue[head++];
            rows[size_t(t * kSliceRows + n++)] = v;
            // take a neighbour only while the patch has room for it, so
            // every vertex taken is placed
            for (int32_t k = rp[v]; k < rp[v + 1]; ++k) {
                const int32_t w = ci[k];
                if (taken[size_t(w)] || n + int32_t(queue.size() - head) >= kSliceRows) continue;
                taken[size_t(w)] = 1;
                queue.push_back(w);
            }
        }
    }
}

std::string build_row_plan(const PlanInput &in, const double *rest_len, RowPlan &out)
{
    const int32_t nv = in.nv;
    const int32_t *rp = in.row_ptr, *ci = in.col_idx;
    out = RowPlan();
    const int64_t nnzb = rp[nv];
    out.slot_rest.assign(size_t(nnzb), -1.0);
    for (int64_t s = 0; s < in.ns; ++s) {
        const int32_t a = in.springs[2 * s], b = in.springs[2 * s + 1];
        const double L = rest_len[s];
        if (!(L >= 0.0)) return "a spring has a negative rest length";
        const int32_t pab = find_pos(rp, ci, a, b), pba = find_pos(rp, ci, b, a);
        if (pab < 0 || pba < 0) return "spring block missing from pattern";
        double &sab = out.slot_rest[size_t(rp[a] + pab)];
        double &sba = out.slot_rest[size_t(rp[b] + pba)];
        if (sab >= 0.0 || sba >= 0.0) return "two springs join the same vertex pair";
        sab = L;
        sba = L;
    }
    const bool faces = in.face_energy && in.nf > 0;
    if (faces) bfs_slice_rows(nv, rp, ci, out.sl_rows);
    // row of lane l of product slice t, -1 for padding
    auto slice_row = [&](int64_t t, int64_t l) -> int32_t {
        if (!out.sl_rows.empty()) return out.sl_rows[size_t(t * kSliceRows + l)];
        const int64_t a = t * kSliceRows + l;
        return a < nv ? int32_t(a) : -1;
    };
    {
        // spring slices: each row's spring neighbours in column order
        const int64_t nsl = (int64_t(nv) + kSliceRows - 1) / kSliceRows;
        out.sl_ptr.assign(size_t(nsl) + 1, 0);
        int64_t tot = 0;
        for (int64_t t = 0; t < nsl; ++t) {
            int32_t w = 0;
            for (int64_t l = 0; l < kSliceRows; ++l) {
                const int32_t a = slice_row(t, l);
                if (a < 0) continue;
                int32_t n = 0;
                for (int64_t k = rp[a]; k < rp[a + 1]; ++k)
                    n += (ci[k] != a && out.slot_rest[size_t(k)] >= 0.0) ? 1 : 0;
                w = std::max(w, n);
            }
            tot += int64_t(kSliceRows) * w;
            if (tot > INT32_MAX) return "too many springs for the spring slices";
            out.sl_ptr[size_t(t) + 1] = int32_t(tot);
        }
        out.sl_nb.assign(size_t(tot), 0);
        out.sl_rest.assign(size_t(tot), -1.0);
        for (int64_t t = 0; t < nsl; ++t) {
            const int64_t w = (out.sl_ptr[size_t(t) + 1] - out.sl_ptr[size_t(t)]) / kSliceRows;
            for (int64_t l = 0; l < kSliceRows; ++l) {
                const int32_t a = slice_row(t, l);
                const int64_t e0 = out.sl_ptr[size_t(t)] + l;
                int64_t j = 0;
                if (a >= 0)
                    for (int64_t k = rp[a]; k < rp[a + 1]; ++k)
                        if (ci[k] != a && out.slot_rest[size_t(k)] >= 0.0) {
                            out.sl_nb[size_t(e0 + kSliceRows * j)] = ci[k];
                            out.sl_rest[size_t(e0 + kSliceRows * j)] = out.slot_rest[size_t(k)];
                            ++j;
                        }
                for (; j < w; ++j) out.sl_nb[size_t(e0 + kSliceRows * j)] = a >= 0 ? a : nv - 1;
            }
        }
        // 16-bit differences from the row (the last row for padding), when
        // all fit
        auto entry_row = [&](int64_t t, int64_t e) -> int64_t {
            const int32_t a = slice_row(t, (e - out.sl_ptr[size_t(t)]) % kSliceRows);
            return a >= 0 ? a : nv - 1;
        };
        bool narrow = true;
        for (int64_t t = 0; t < nsl && narrow; ++t)
            for (int64_t e = out.sl_ptr[size_t(t)]; e < out.sl_ptr[size_t(t) + 1]; ++e) {
                const int64_t a = entry_row(t, e);
                const int64_t d = int64_t(out.sl_nb[size_t(e)]) - a;
                if (d < INT16_MIN || d > INT16_MAX) {
                    narrow = false;
                    break;
                }
            }
        if (narrow) {
            out.sl_d16.resize(size_t(tot));
            for (int64_t t = 0; t < nsl; ++t)
                for (int64_t e = out.sl_ptr[size_t(t)]; e < out.sl_ptr[size_t(t) + 1]; ++e) {
                    const int64_t a = entry_row(t, e);
                    out.sl_d16[size_t(e)] = int16_t(int64_t(out.sl_nb[size_t(e)]) - a);
                }
        }
    }
    if (faces) {
        // per-row incidence, rows in vertex order, faces by id within a row
        out.fptr.assign(size_t(nv) + 1, 0);
        for (int64_t f = 0; f < in.nf; ++f)
            for (int k = 0; k < 3; ++k) out.fptr[size_t(in.faces[3 * f + k]) + 1] += 1;
        for (int32_t v = 0; v < nv; ++v) out.fptr[v + 1] += out.fptr[v];
        out.finc.resize(size_t(out.fptr[nv]));
        std::vector<int32_t> cur(out.fptr.begin(), out.fptr.end() - 1);
        for (int64_t f = 0; f < in.nf; ++f) {
            const int32_t *t = in.faces + 3 * f;
            for (int i = 0; i < 3; ++i) {
                const int32_t a = t[i];
                FaceInc e;
                e.f = int32_t(f);
                e.o1 = t[(i + 1) % 3];
                e.o2 = t[(i + 2) % 3];
                e.pk = uint32_t(i);
                for (int k = 0; k < 3; ++k) {
                    const int32_t pos = find_pos(rp, ci, a, t[k]);
                    if (pos < 0) return "face block missing from pattern";
                    if (pos >= kMaxRowFaceSlots) return "a row is too long for the row path's face terms";
                    e.pk |= uint32_t(pos) << (8 * k + 8);
                }
                out.finc[size_t(cur[a]++)] = e;
            }
        }
        // each slice's face list: every row's first incident face (by id),
        // then every row's second, ..., each face once; then every row's
        // faces by their position in that list
        const int64_t nsl = (int64_t(nv) + kSliceRows - 1) / kSliceRows;
        out.sf_ptr.assign(size_t(nsl) + 1, 0);
        out.rfinc.resize(out.finc.size());
        std::vector<int32_t> where(size_t(in.nf), -1);   // position in the current list
        std::vector<int64_t> owner(size_t(in.nf), -1);   // slice that listed the face
        for (int64_t t = 0; t < nsl; ++t) {
            int32_t maxdeg = 0;
            for (int64_t l = 0; l < kSliceRows; ++l) {
                const int32_t a = slice_row(t, l);
                if (a >= 0) maxdeg = std::max(maxdeg, out.fptr[a + 1] - out.fptr[a]);
            }
            int64_t nl = 0;
            for (int32_t rank = 0; rank < maxdeg; ++rank)
                for (int64_t l = 0; l < kSliceRows; ++l) {
                    const int32_t a = slice_row(t, l);
                    if (a < 0 || rank >= out.fptr[a + 1] - out.fptr[a]) continue;
                    const int32_t f = out.finc[size_t(out.fptr[a] + rank)].f;
                    if (owner[size_t(f)] == t) continue;
                    owner[size_t(f)] = t;
                    where[size_t(f)] = int32_t(nl++);
                    SliceFace sf;
                    for (int i = 0; i < 3; ++i) sf.v[i] = in.faces[3 * int64_t(f) + i];
                    sf.f = f;
                    out.sface.push_back(sf);
                }
            if (out.sf_ptr[size_t(t)] + nl > INT32_MAX) return "too many faces for the slice lists";
            out.sf_ptr[size_t(t) + 1] = int32_t(out.sf_ptr[size_t(t)] + nl);
            for (int64_t l = 0; l < kSliceRows; ++l) {
                const int32_t a = slice_row(t, l);
                if (a < 0) continue;
                for (int32_t k = out.fptr[a]; k < out.fptr[a + 1]; ++k) {
                    RowFace e;
                    e.lf = uint32_t(where[size_t(out.finc[size_t(k)].f)]);
                    e.pi = out.finc[size_t(k)].pk & 3u;
                    out.rfinc[size_t(k)] = e;
                }
                std::sort(out.rfinc.begin() + out.fptr[a], out.rfinc.begin() + out.fptr[a + 1],
                          [](const RowFace &p, const RowFace &q) { return p.lf < q.lf; });
            }
        }
    }
    for (int32_t v0 = 0; v0 < nv;) {
        int32_t n = 0, blk = 0;
        while (n < kRowsPerChunk && v0 + n < nv) {
            const int32_t len = rp[v0 + n + 1] - rp[v0 + n];
            if (blk + len > kRowBaseBlocks) break;
            blk += len;
            ++n;
        }
        if (n == 0) return "vertex " + std::to_string(v0) + " has a row too long for the row path";
        PatchHdr h;
        std::memset(&h, 0, sizeof(h));
        h.v0 = v0;
        h.nown = n;
        h.blk0 = rp[v0];
        h.nblk = blk;
        h.amap_cap = kRowLdsBlocks;
        // a chunk that is exactly one spring slice and whose rows hold only
        // their diagonal and their springs' blocks reads its springs from the
        // slice (spr_off = the slice), else from its rows (-1)
        h.spr_off = -1;
        if (out.sl_rows.empty() && v0 % kSliceRows == 0 && n == std::min(kSliceRows, nv - v0)) {
            bool dense = true;
            for (int32_t a = v0; a < v0 + n && dense; ++a)
                for (int32_t k = rp[a]; k < rp[a + 1] && dense; ++k)
                    dense = ci[k] == a || out.slot_rest[size_t(k)] >= 0.0;
            if (dense) h.spr_off = v0 / kSliceRows;
        }
        out.chunk.push_back(h);
        v0 += n;
    }
    return "";
}

std::string build_insert_tiles(const std::vector<PatchHdr> &units, int32_t nv, bool align_units,
                               InsertTiles &out)
{
    out = InsertTiles();
    if (nv <= 0) return "nv must be positive";
    out.row_tile.assign(size_t(nv), 0);
    out.tile_row.push_back(0);
    out.tile_unit.push_back(0);
    if (align_units) {
        out.row_unit.assign(size_t(nv), 0);
        int32_t next = 0;
        for (size_t u = 0; u < units.size(); ++u) {
            if (units[u].v0 != next || units[u].nown <= 0)
                return "units must cover the rows in order";
            if (units[u].nown > kInsTileRows) return "a row chunk exceeds the tile row limit";
            next += units[u].nown;
        }
        if (next != nv) return "units must cover the rows in order";
        int32_t rows = 0, nu = 0;
        for (size_t u = 0; u < units.size(); ++u) {
            if (nu > 0 && (rows + units[u].nown > kInsTileRows || nu == kInsTileUnits)) {
                out.tile_row.push_back(units[u].v0);
                out.tile_unit.push_back(int32_t(u));
                rows = nu = 0;
            }
            rows += units[u].nown;
            ++nu;
            for (int32_t a = units[u].v0; a < units[u].v0 + units[u].nown; ++a)
                out.row_unit[size_t(a)] = int32_t(u);
        }
        out.tile_row.push_back(nv);
        out.tile_unit.push_back(int32_t(units.size()));
    } else {
        for (int32_t r = kInsTileRows; r < nv; r += kInsTileRows) {
            out.tile_row.push_back(r);
            out.tile_unit.push_back(0);
        }
        out.tile_row.push_back(nv);
        out.tile_unit.push_back(0);
    }
    const size_t nt = out.tile_row.size() - 1;
    if (nt > size_t(kInsMaxTiles)) return "too many rows for pair insertion";
    for (size_t t = 0; t < nt; ++t)
        for (int32_t a = out.tile_row[t]; a < out.tile_row[t + 1]; ++a)
            out.row_tile[size_t(a)] = int32_t(t);
    return "";
}

}  // namespace lad
