// Host-only checks of the two evaluation plans built by lad_patch.cpp: the
// patch plan (contiguous-row patches with ribbon vertices, per-patch element
// records, colours) and the row plan (row chunks, per-block rest lengths,
// per-row face incidence).  No GPU is touched.  Prints one line per failed
// check and exits non-zero if any failed.
#include <algorithm>
#include <cstdio>
#include <map>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "lad_internal.h"

using namespace lad;

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                                     \
    do {                                                     \
        if (!(cond)) {                                       \
            ++g_fail;                                        \
            if (g_fail < 40) {                               \
                std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                std::printf(__VA_ARGS__);                    \
                std::printf("\n");                           \
            }                                                \
        }                                                    \
    } while (0)

struct Mesh {
    int32_t nv = 0;
    std::vector<int32_t> faces, springs;
    std::vector<double> rest;
};

void add_edge_springs(Mesh &m)
{
    std::set<std::pair<int32_t, int32_t>> e;
    for (size_t f = 0; f * 3 < m.faces.size(); ++f)
        for (int i = 0; i < 3; ++i) {
            int32_t a = m.faces[3 * f + i], b = m.faces[3 * f + (i + 1) % 3];
            e.insert({std::min(a, b), std::max(a, b)});
        }
    for (auto &p : e) {
        m.springs.push_back(p.first);
        m.springs.push_back(p.second);
        m.rest.push_back(0.5 + 0.001 * double((p.first * 7 + p.second) % 100));
    }
}

Mesh grid(int n)
{
    Mesh m;
    m.nv = n * n;
    for (int j = 0; j + 1 < n; ++j)
        for (int i = 0; i + 1 < n; ++i) {
            const int v = j * n + i;
            m.faces.insert(m.faces.end(), {v, v + 1, v + n + 1, v, v + n + 1, v + n});
        }
    add_edge_springs(m);
    return m;
}

// Irregular mesh: random triangles over a shuffled vertex numbering (rows of
// very different lengths, far-apart column indices).
Mesh random_mesh(int nv, int nf, unsigned seed)
{
    std::mt19937 rng(seed);
    std::uniform_int_distribution<int> U(0, nv - 1);
    Mesh m;
    m.nv = nv;
    for (int f = 0; f < nf; ++f) {
        int a = U(rng), b = U(rng), c = U(rng);
        if (a == b || b == c || a == c) continue;
        m.faces.insert(m.faces.end(), {a, b, c});
    }
    add_edge_springs(m);
    return m;
}

void pattern(const Mesh &m, std::vector<int32_t> &rp, std::vector<int32_t> &ci)
{
    std::vector<std::set<int32_t>> rows(m.nv);
    for (int32_t v = 0; v < m.nv; ++v) rows[v].insert(v);
    for (size_t f = 0; f * 3 < m.faces.size(); ++f)
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) rows[m.faces[3 * f + i]].insert(m.faces[3 * f + j]);
    for (size_t s = 0; s * 2 < m.springs.size(); ++s) {
        rows[m.springs[2 * s]].insert(m.springs[2 * s + 1]);
        rows[m.springs[2 * s + 1]].insert(m.springs[2 * s]);
    }
    rp.assign(m.nv + 1, 0);
    ci.clear();
    for (int32_t v = 0; v < m.nv; ++v) {
        ci.insert(ci.end(), rows[v].begin(), rows[v].end());
        rp[v + 1] = int32_t(ci.size());
    }
}

int32_t slot_of(const std::vector<int32_t> &rp, const std::vector<int32_t> &ci, int32_t a, int32_t b)
{
    for (int32_t k = rp[a]; k < rp[a + 1]; ++k)
        if (ci[k] == b) return k;
    return -1;
}

PlanInput make_input(const Mesh &m, const std::vector<int32_t> &rp, const std::vector<int32_t> &ci,
                     bool faces_on, int es, int budget)
{
    PlanInput in;
    in.nv = m.nv;
    in.nf = int32_t(m.faces.size() / 3);
    in.faces = m.faces.data();
    in.ns = int32_t(m.springs.size() / 2);
    in.springs = m.springs.data();
    in.face_energy = faces_on ? 1 : 0;
    in.row_ptr = rp.data();
    in.col_idx = ci.data();
    in.elem_size = es;
    in.lds_budget = budget;
    return in;
}

void check_patch_plan(const Mesh &m, bool faces_on, int es, int budget, const char *tag)
{
    std::vector<int32_t> rp, ci;
    pattern(m, rp, ci);
    const PlanInput in = make_input(m, rp, ci, faces_on, es, budget);
    Plan plan;
    const std::string err = build_plan(in, plan);
    CHECK(err.empty(), "%s: build_plan failed: %s", tag, err.c_str());
    if (!err.empty()) return;
    const int32_t np = int32_t(plan.hdr.size());
    int32_t expect_v0 = 0;
    std::vector<int> spr_seen(in.ns, 0), fac_seen(in.nf, 0);
    for (int32_t p = 0; p < np; ++p) {
        const PatchHdr &h = plan.hdr[p];
        CHECK(h.v0 == expect_v0 && h.nown > 0, "%s: patch %d does not continue the rows", tag, p);
        expect_v0 = h.v0 + h.nown;
        CHECK(h.blk0 == rp[h.v0] && h.nblk == rp[h.v0 + h.nown] - rp[h.v0], "%s: patch %d block range", tag, p);
        CHECK(h.lds_eval <= budget, "%s: patch %d LDS %d over budget %d", tag, p, h.lds_eval, budget);
        CHECK(h.amap_cap >= h.nblk, "%s: patch %d map capacity", tag, p);
        auto owned = [&](int32_t v) { return v >= h.v0 && v < h.v0 + h.nown; };
        // ribbon = sorted non-owned columns of the owned rows
        std::set<int32_t> rib_expect;
        for (int32_t v = h.v0; v < h.v0 + h.nown; ++v)
            for (int32_t k = rp[v]; k < rp[v + 1]; ++k)
                if (!owned(ci[k])) rib_expect.insert(ci[k]);
        std::vector<int32_t> rib(plan.rib.begin() + h.rib_off, plan.rib.begin() + h.rib_off + h.nrib);
        CHECK(std::vector<int32_t>(rib_expect.begin(), rib_expect.end()) == rib, "%s: patch %d ribbon", tag, p);
        auto global_of = [&](int l) { return l < h.nown ? h.v0 + l : rib[size_t(l - h.nown)]; };
        for (int32_t v = h.v0; v < h.v0 + h.nown; ++v)
            CHECK(plan.diag_rel[v] == slot_of(rp, ci, v, v) - h.blk0, "%s: diagonal slot of %d", tag, v);
        // springs: exactly those touching an owned vertex, once each
        std::set<int32_t> expect_s;
        for (int32_t s = 0; s < in.ns; ++s)
            if (owned(m.springs[2 * s]) || owned(m.springs[2 * s + 1])) expect_s.insert(s);
        std::multiset<int32_t> got_s;
        const int32_t *cb = plan.col_bounds.data() + h.col_off;
        for (int32_t r = 0; r < h.nspr; ++r) {
            const int32_t s = plan.spr_src[h.spr_off + r];
            got_s.insert(s);
            spr_seen[s] += 1;
            const SpringRec rec = plan.spr[h.spr_off + r];
            const int la = rec.lab & 0xFFFF, lb = rec.lab >> 16;
            const int32_t a = m.springs[2 * s], b = m.springs[2 * s + 1];
            CHECK(global_of(la) == a && global_of(lb) == b, "%s: spring %d local ids", tag, s);
            const int32_t sab = owned(a) ? slot_of(rp, ci, a, b) - h.blk0 : kNone;
            const int32_t sba = owned(b) ? slot_of(rp, ci, b, a) - h.blk0 : kNone;
            CHECK(int32_t(rec.blk & 0xFFFF) == sab && int32_t(rec.blk >> 16) == sba, "%s: spring %d slots", tag, s);
        }
        CHECK(got_s.size() == expect_s.size() &&
                  std::equal(expect_s.begin(), expect_s.end(), std::set<int32_t>(got_s.begin(), got_s.end()).begin()),
              "%s: patch %d spring set", tag, p);
        // colours: bounds monotone, no two springs of a colour share an owned vertex
        for (int c = 0; c < h.nspr_col; ++c) {
            CHECK(cb[c] <= cb[c + 1], "%s: colour bounds", tag);
            std::set<int32_t> used;
            for (int32_t r = cb[c]; r < cb[c + 1]; ++r) {
                const int32_t s = plan.spr_src[h.spr_off + r];
                for (int i = 0; i < 2; ++i) {
                    const int32_t v = m.springs[2 * s + i];
                    if (!owned(v)) continue;
                    CHECK(!used.count(v), "%s: colour %d shares vertex %d", tag, c, v);
                    used.insert(v);
                }
            }
        }
        if (h.nspr > 0) CHECK(cb[0] == 0 && cb[h.nspr_col] == h.nspr, "%s: colour bounds span", tag);
        // faces
        if (faces_on) {
            const int32_t *fb = cb + (h.nspr_col ? h.nspr_col + 1 : 0);
            std::set<int32_t> expect_f;
            for (int32_t f = 0; f < in.nf; ++f)
                for (int i = 0; i < 3; ++i)
                    if (owned(m.faces[3 * f + i])) expect_f.insert(f);
            CHECK(int32_t(expect_f.size()) == h.nfac, "%s: patch %d face count", tag, p);
            for (int32_t r = 0; r < h.nfac; ++r) {
                const int32_t f = plan.fac_src[h.fac_off + r];
                fac_seen[f] += 1;
                CHECK(expect_f.count(f), "%s: face %d not incident", tag, f);
                const FaceRec &rec = plan.fac[h.fac_off + r];
                for (int i = 0; i < 3; ++i) {
                    const int32_t a = m.faces[3 * f + i];
                    CHECK(global_of(rec.l[i]) == a, "%s: face %d local id", tag, f);
                    for (int j = 0; j < 3; ++j) {
                        const int32_t want = owned(a) ? slot_of(rp, ci, a, m.faces[3 * f + j]) - h.blk0 : kNone;
                        CHECK(int32_t(rec.blk[3 * i + j]) == want, "%s: face %d block slot", tag, f);
                    }
                }
            }
            for (int c = 0; c < h.nfac_col; ++c) {
                std::set<int32_t> used;
                for (int32_t r = fb[c]; r < fb[c + 1]; ++r) {
                    const int32_t f = plan.fac_src[h.fac_off + r];
                    for (int i = 0; i < 3; ++i) {
                        const int32_t v = m.faces[3 * f + i];
                        if (!owned(v)) continue;
                        CHECK(!used.count(v), "%s: face colour %d shares vertex %d", tag, c, v);
                        used.insert(v);
                    }
                }
            }
        }
    }
    CHECK(expect_v0 == m.nv, "%s: patches do not cover the rows", tag);
    // an element is evaluated by every patch that owns one of its vertices
    for (int32_t s = 0; s < in.ns; ++s) {
        std::set<int32_t> ps = {plan.vpatch[m.springs[2 * s]], plan.vpatch[m.springs[2 * s + 1]]};
        CHECK(spr_seen[s] == int(ps.size()), "%s: spring %d evaluated %d times, owners %zu", tag, s, spr_seen[s], ps.size());
    }
    if (faces_on)
        for (int32_t f = 0; f < in.nf; ++f) {
            std::set<int32_t> ps;
            for (int i = 0; i < 3; ++i) ps.insert(plan.vpatch[m.faces[3 * f + i]]);
            CHECK(fac_seen[f] == int(ps.size()), "%s: face %d evaluated %d times", tag, f, fac_seen[f]);
        }
}

// Element-once plan: every element in exactly one patch (the owner of its
// lowest vertex id), ribbons from the patch's own elements, foreign blocks
// and flags as the kernels use them.  The kernels' data flow is replayed on
// the host with one random scalar per element written into every block it
// touches (and every gradient entry): LDS per patch, global adds for foreign
// rows into zeroed boundary slots, then the flush (flagged entries added when
// non-zero, the rest stored).  The result must equal the direct assembly.
void check_element_once_plan(const Mesh &m, bool faces_on, int es, int budget, const char *tag)
{
    std::vector<int32_t> rp, ci;
    pattern(m, rp, ci);
    PlanInput in = make_input(m, rp, ci, faces_on, es, budget);
    in.element_once = 1;
    Plan plan;
    const std::string err = build_plan(in, plan);
    CHECK(err.empty(), "%s: build_plan failed: %s", tag, err.c_str());
    if (!err.empty()) return;
    const int32_t nv = m.nv, nnzb = rp[nv], nf = faces_on ? in.nf : 0;
    CHECK(plan.spr_gblk.size() == 2 * plan.spr.size() && plan.fac_gblk.size() == 9 * plan.fac.size(),
          "%s: foreign block tables sized", tag);
    CHECK(int32_t(plan.blk_flag.size()) == nnzb && int32_t(plan.vtx_flag.size()) == nv, "%s: flag sizes", tag);
    std::mt19937 rng(7);
    std::uniform_real_distribution<double> U(0.5, 1.5);
    std::vector<double> ws(in.ns), wf(nf);
    for (auto &w : ws) w = U(rng);
    for (auto &w : wf) w = U(rng);
    // direct assembly
    std::vector<double> H(nnzb, 0.0), G(nv, 0.0);
    std::vector<int> foreign_blk(nnzb, 0), foreign_vtx(nv, 0);
    auto direct = [&](const int32_t *vs, int k, double w) {
        for (int i = 0; i < k; ++i) {
            G[vs[i]] += w;
            for (int j = 0; j < k; ++j) H[slot_of(rp, ci, vs[i], vs[j])] += w;
        }
    };
    for (int32_t s = 0; s < in.ns; ++s) direct(&m.springs[2 * s], 2, ws[s]);
    for (int32_t f = 0; f < nf; ++f) direct(&m.faces[3 * f], 3, wf[f]);
    // replay of the kernels
    std::vector<double> Hk(nnzb, -7.0), Gk(nv, -7.0);  // stale values everywhere
    for (int32_t b : plan.bnd_blk) Hk[b] = 0.0;
    for (int32_t v : plan.bnd_vtx) Gk[v] = 0.0;
    std::vector<int> spr_seen(in.ns, 0), fac_seen(nf, 0);
    std::vector<double> Hl, Gl;
    std::vector<std::pair<int32_t, double>> hadd, gadd;  // global adds (any order)
    for (size_t p = 0; p < plan.hdr.size(); ++p) {
        const PatchHdr &h = plan.hdr[p];
        auto owned = [&](int32_t v) { return v >= h.v0 && v < h.v0 + h.nown; };
        std::vector<int32_t> rib(plan.rib.begin() + h.rib_off, plan.rib.begin() + h.rib_off + h.nrib);
        std::set<int32_t> rib_expect;
        auto global_of = [&](int l) { return l < h.nown ? h.v0 + l : rib[size_t(l - h.nown)]; };
        Hl.assign(h.nblk, 0.0);
        Gl.assign(h.nown, 0.0);
        for (int32_t r = 0; r < h.nspr; ++r) {
            const int32_t s = plan.spr_src[h.spr_off + r];
            spr_seen[s] += 1;
            const int32_t a = m.springs[2 * s], b = m.springs[2 * s + 1];
            CHECK(owned(std::min(a, b)), "%s: spring %d not in its lowest vertex's patch", tag, s);
            const SpringRec rec = plan.spr[h.spr_off + r];
            const int la = rec.lab & 0xFFFF, lb = rec.lab >> 16;
            CHECK(global_of(la) == a && global_of(lb) == b, "%s: spring %d local ids", tag, s);
            for (int32_t v : {a, b})
                if (!owned(v)) rib_expect.insert(v);
            const int32_t *gb = &plan.spr_gblk[2 * size_t(h.spr_off + r)];
            const double w = ws[s];
            for (int e = 0; e < 2; ++e) {
                const int32_t v = e ? b : a, o = e ? a : b;
                const int l = e ? lb : la;
                if (owned(v)) {
                    Gl[l] += w;
                    Hl[plan.diag_rel[v]] += w;
                    Hl[(e ? rec.blk >> 16 : rec.blk & 0xFFFF)] += w;
                } else {
                    CHECK(gb[0] == slot_of(rp, ci, v, v) && gb[1] == slot_of(rp, ci, v, o),
                          "%s: spring %d foreign blocks", tag, s);
                    gadd.push_back({v, w});
                    hadd.push_back({gb[0], w});
                    hadd.push_back({gb[1], w});
                    foreign_blk[gb[0]] = foreign_blk[gb[1]] = foreign_vtx[v] = 1;
                }
            }
            if (owned(a) && owned(b)) CHECK(gb[0] == -1 && gb[1] == -1, "%s: spring %d owned, foreign blocks set", tag, s);
        }
        for (int32_t r = 0; r < h.nfac; ++r) {
            const int32_t f = plan.fac_src[h.fac_off + r];
            fac_seen[f] += 1;
            const int32_t *t = &m.faces[3 * f];
            CHECK(owned(std::min({t[0], t[1], t[2]})), "%s: face %d not in its lowest vertex's patch", tag, f);
            const FaceRec &rec = plan.fac[h.fac_off + r];
            const int32_t *gb = &plan.fac_gblk[9 * size_t(h.fac_off + r)];
            for (int i = 0; i < 3; ++i) {
                CHECK(global_of(rec.l[i]) == t[i], "%s: face %d local id", tag, f);
                if (!owned(t[i])) rib_expect.insert(t[i]);
                if (owned(t[i])) Gl[rec.l[i]] += wf[f];
                else {
                    gadd.push_back({t[i], wf[f]});
                    foreign_vtx[t[i]] = 1;
                }
                for (int j = 0; j < 3; ++j) {
                    if (owned(t[i])) {
                        CHECK(gb[3 * i + j] == -1, "%s: face %d owned row with a foreign block", tag, f);
                        Hl[rec.blk[3 * i + j]] += wf[f];
                    } else {
                        CHECK(gb[3 * i + j] == slot_of(rp, ci, t[i], t[j]), "%s: face %d foreign block", tag, f);
                        hadd.push_back({gb[3 * i + j], wf[f]});
                        foreign_blk[gb[3 * i + j]] = 1;
                    }
                }
            }
        }
        CHECK(std::vector<int32_t>(rib_expect.begin(), rib_expect.end()) == rib, "%s: patch %zu ribbon", tag, p);
        CHECK(h.lds_eval <= budget && 2 * h.amap_cap >= h.nblk + h.nown, "%s: patch %zu LDS", tag, p);
        // flush of the owned slice
        for (int32_t i = 0; i < h.nblk; ++i) {
            const int32_t b = h.blk0 + i;
            if (plan.blk_flag[b]) {
                if (Hl[i] != 0.0) hadd.push_back({b, Hl[i]});
            } else {
                Hk[b] = Hl[i];
            }
        }
        for (int32_t i = 0; i < h.nown; ++i) {
            const int32_t v = h.v0 + i;
            if (plan.vtx_flag[v]) {
                if (Gl[i] != 0.0) gadd.push_back({v, Gl[i]});
            } else {
                Gk[v] = Gl[i];
            }
        }
    }
    for (auto &a : hadd) Hk[a.first] += a.second;
    for (auto &a : gadd) Gk[a.first] += a.second;
    for (int32_t s = 0; s < in.ns; ++s) CHECK(spr_seen[s] == 1, "%s: spring %d in %d patches", tag, s, spr_seen[s]);
    for (int32_t f = 0; f < nf; ++f) CHECK(fac_seen[f] == 1, "%s: face %d in %d patches", tag, f, fac_seen[f]);
    int nbad_flag = 0, nbad_val = 0;
    for (int32_t b = 0; b < nnzb; ++b) {
        nbad_flag += int(plan.blk_flag[b]) != foreign_blk[b];
        nbad_val += std::abs(Hk[b] - H[b]) > 1e-12 * (1.0 + std::abs(H[b]));
    }
    for (int32_t v = 0; v < nv; ++v) {
        nbad_flag += int(plan.vtx_flag[v]) != foreign_vtx[v];
        nbad_val += std::abs(Gk[v] - G[v]) > 1e-12 * (1.0 + std::abs(G[v]));
    }
    CHECK(nbad_flag == 0, "%s: %d boundary flags differ from the foreign writes", tag, nbad_flag);
    CHECK(nbad_val == 0, "%s: %d replayed values differ from the direct assembly", tag, nbad_val);
    std::vector<int32_t> bb, bv;
    for (int32_t b = 0; b < nnzb; ++b)
        if (foreign_blk[b]) bb.push_back(b);
    for (int32_t v = 0; v < nv; ++v)
        if (foreign_vtx[v]) bv.push_back(v);
    CHECK(bb == plan.bnd_blk && bv == plan.bnd_vtx, "%s: boundary lists", tag);
}

bool has_spring(const Mesh &m, int32_t a, int32_t b)
{
    for (size_t s = 0; s * 2 < m.springs.size(); ++s)
        if ((m.springs[2 * s] == a && m.springs[2 * s + 1] == b) ||
            (m.springs[2 * s] == b && m.springs[2 * s + 1] == a))
            return true;
    return false;
}

void check_row_plan(const Mesh &m, bool faces_on, const char *tag)
{
    std::vector<int32_t> rp, ci;
    pattern(m, rp, ci);
    const PlanInput in = make_input(m, rp, ci, faces_on, 4, 0);
    RowPlan plan;
    const std::string err = build_row_plan(in, m.rest.data(), plan);
    CHECK(err.empty(), "%s: build_row_plan failed: %s", tag, err.c_str());
    if (!err.empty()) return;
    const int32_t nsl = (m.nv + kSliceRows - 1) / kSliceRows;
    // product slices: contiguous rows, or with the face term on a partition
    // of the rows into full slices (the last may be short) listed in
    // sl_rows, padded with -1 at the end
    CHECK(plan.sl_rows.empty() != faces_on, "%s: slice rows present %d", tag, int(!plan.sl_rows.empty()));
    if (!plan.sl_rows.empty()) {
        CHECK(plan.sl_rows.size() == size_t(nsl) * kSliceRows, "%s: slice rows size", tag);
        if (plan.sl_rows.size() != size_t(nsl) * kSliceRows) return;
        std::vector<int32_t> seen(size_t(m.nv), 0);
        for (size_t k = 0; k < plan.sl_rows.size(); ++k) {
            const int32_t a = plan.sl_rows[k];
            if (k < size_t(m.nv)) {
                CHECK(a >= 0 && a < m.nv, "%s: slice entry %zu row %d", tag, k, a);
                if (a >= 0 && a < m.nv) seen[size_t(a)] += 1;
            } else {
                CHECK(a == -1, "%s: slice padding %zu", tag, k);
            }
        }
        for (int32_t a = 0; a < m.nv; ++a) CHECK(seen[size_t(a)] == 1, "%s: row %d in %d slices", tag, a, seen[size_t(a)]);
    }
    auto row_of = [&](int32_t t, int32_t l) -> int32_t {
        if (!plan.sl_rows.empty()) return plan.sl_rows[size_t(t) * kSliceRows + size_t(l)];
        return t * kSliceRows + l < m.nv ? t * kSliceRows + l : -1;
    };
    int32_t expect_v0 = 0;
    for (const PatchHdr &h : plan.chunk) {
        CHECK(h.v0 == expect_v0 && h.nown > 0 && h.nown <= kRowsPerChunk, "%s: chunk rows", tag);
        CHECK(h.nblk == rp[h.v0 + h.nown] - rp[h.v0] && h.nblk <= kRowBaseBlocks, "%s: chunk blocks", tag);
        CHECK(h.amap_cap == kRowLdsBlocks, "%s: chunk capacity", tag);
        // slice-aligned chunks whose off-diagonal blocks all carry springs
        bool dense = plan.sl_rows.empty() && h.v0 % kSliceRows == 0 &&
                     h.nown == std::min(kSliceRows, m.nv - h.v0);
        for (int32_t a = h.v0; a < h.v0 + h.nown && dense; ++a)
            for (int32_t k = rp[a]; k < rp[a + 1]; ++k)
                if (ci[k] != a && !has_spring(m, a, ci[k])) dense = false;
        CHECK(h.spr_off == (dense ? h.v0 / kSliceRows : -1), "%s: chunk %d slice flag", tag, h.v0);
        expect_v0 = h.v0 + h.nown;
    }
    CHECK(expect_v0 == m.nv, "%s: chunks do not cover the rows", tag);
    // the face kernel's staging capacity: the largest block count of the
    // first kRowsPerChunk / 2 rows of a chunk or of the rest
    {
        int32_t most = 1;
        for (const PatchHdr &h : plan.chunk)
            for (int32_t part = 0; part < 2; ++part) {
                const int32_t a = h.v0 + std::min(h.nown, part * (kRowsPerChunk / 2));
                const int32_t b = part == 0 ? h.v0 + std::min(h.nown, kRowsPerChunk / 2) : h.v0 + h.nown;
                most = std::max(most, rp[b] - rp[a]);
            }
        CHECK(half_chunk_blocks(plan.chunk, rp.data()) == most, "%s: half-chunk staging %d, want %d",
              tag, half_chunk_blocks(plan.chunk, rp.data()), most);
    }
    std::vector<double> want(ci.size(), -1.0);
    for (size_t s = 0; s * 2 < m.springs.size(); ++s) {
        want[size_t(slot_of(rp, ci, m.springs[2 * s], m.springs[2 * s + 1]))] = m.rest[s];
        want[size_t(slot_of(rp, ci, m.springs[2 * s + 1], m.springs[2 * s]))] = m.rest[s];
    }
    CHECK(plan.slot_rest == want, "%s: per-block rest lengths", tag);
    // spring slices: every row's springs by ascending neighbour, from the
    // spring list itself; widths are the slice maxima, padding marked
    std::vector<std::vector<std::pair<int32_t, double>>> sp(m.nv);
    for (size_t s = 0; s * 2 < m.springs.size(); ++s) {
        sp[m.springs[2 * s]].push_back({m.springs[2 * s + 1], m.rest[s]});
        sp[m.springs[2 * s + 1]].push_back({m.springs[2 * s], m.rest[s]});
    }
    for (auto &l : sp) std::sort(l.begin(), l.end());
    CHECK(int32_t(plan.sl_ptr.size()) == nsl + 1 && plan.sl_ptr[0] == 0, "%s: slice offsets size", tag);
    if (int32_t(plan.sl_ptr.size()) != nsl + 1) return;
    CHECK(size_t(plan.sl_ptr[nsl]) == plan.sl_nb.size() && plan.sl_nb.size() == plan.sl_rest.size(),
          "%s: slice entry count", tag);
    for (int32_t t = 0; t < nsl; ++t) {
        const int32_t len = plan.sl_ptr[t + 1] - plan.sl_ptr[t];
        size_t wmax = 0;
        for (int32_t l = 0; l < kSliceRows; ++l)
            if (row_of(t, l) >= 0) wmax = std::max(wmax, sp[size_t(row_of(t, l))].size());
        CHECK(len >= 0 && len % kSliceRows == 0 && size_t(len / kSliceRows) == wmax,
              "%s: slice %d width", tag, t);
        if (len < 0 || size_t(plan.sl_ptr[t + 1]) > plan.sl_nb.size()) continue;
        for (int32_t l = 0; l < kSliceRows; ++l) {
            const int32_t a = row_of(t, l);
            for (int32_t j = 0; j < len / kSliceRows; ++j) {
                const size_t e = size_t(plan.sl_ptr[t] + j * kSliceRows + l);
                if (a >= 0 && size_t(j) < sp[a].size())
                    CHECK(plan.sl_nb[e] == sp[a][j].first && plan.sl_rest[e] == sp[a][j].second,
                          "%s: row %d spring %d", tag, a, j);
                else
                    CHECK(plan.sl_nb[e] == (a >= 0 ? a : m.nv - 1) && plan.sl_rest[e] == -1.0,
                          "%s: row %d padding %d", tag, a, j);
            }
        }
    }
    // 16-bit neighbour differences: present exactly when every one fits
    bool fit = true;
    for (int32_t t = 0; t < nsl; ++t)
        for (int32_t e = plan.sl_ptr[t]; e < plan.sl_ptr[t + 1]; ++e) {
            const int32_t r = row_of(t, (e - plan.sl_ptr[t]) % kSliceRows);
            const int64_t a = r >= 0 ? r : m.nv - 1;
            const int64_t d = int64_t(plan.sl_nb[size_t(e)]) - a;
            fit = fit && d >= INT16_MIN && d <= INT16_MAX;
            if (!plan.sl_d16.empty() && size_t(e) < plan.sl_d16.size())
                CHECK(a + plan.sl_d16[size_t(e)] == plan.sl_nb[size_t(e)], "%s: entry %d difference", tag, e);
        }
    CHECK(fit == (plan.sl_d16.size() == plan.sl_nb.size()) && (fit || plan.sl_d16.empty()),
          "%s: 16-bit differences present %d, fit %d", tag, int(!plan.sl_d16.empty()), int(fit));
    if (!faces_on) return;
    CHECK(int32_t(plan.fptr.size()) == m.nv + 1, "%s: face offsets size", tag);
    std::vector<std::vector<int32_t>> inc(m.nv);
    for (size_t f = 0; f * 3 < m.faces.size(); ++f)
        for (int i = 0; i < 3; ++i) inc[m.faces[3 * f + i]].push_back(int32_t(f));
    for (int32_t a = 0; a < m.nv; ++a) {
        CHECK(plan.fptr[a + 1] - plan.fptr[a] == int32_t(inc[a].size()), "%s: row %d face count", tag, a);
        for (int32_t k = plan.fptr[a]; k < plan.fptr[a + 1] && k - plan.fptr[a] < int32_t(inc[a].size()); ++k) {
            const FaceInc &e = plan.finc[k];
            const int32_t f = inc[a][size_t(k - plan.fptr[a])];
            CHECK(e.f == f, "%s: row %d faces not in id order", tag, a);
            const int i = int(e.pk & 3u);
            const int32_t *t = m.faces.data() + 3 * f;
            CHECK(i < 3 && t[i] == a && e.o1 == t[(i + 1) % 3] && e.o2 == t[(i + 2) % 3], "%s: row %d face %d vertices", tag, a, f);
            for (int u = 0; u < 3; ++u)
                CHECK(int32_t((e.pk >> (8 * u + 8)) & 255u) == slot_of(rp, ci, a, t[u]) - rp[a], "%s: row %d face %d slot", tag, a, f);
        }
    }
    // slice face lists of the product kernels: each face incident to a
    // slice's rows exactly once, ordered by (its first position in an
    // incident row's id-sorted face list, that row's lane); every row's
    // faces by their position in its slice's list, with the row's position
    // in the face
    CHECK(int32_t(plan.sf_ptr.size()) == nsl + 1 && plan.sf_ptr[0] == 0, "%s: slice face offsets", tag);
    if (int32_t(plan.sf_ptr.size()) != nsl + 1) return;
    CHECK(size_t(plan.sf_ptr[nsl]) == plan.sface.size(), "%s: slice face count", tag);
    CHECK(plan.rfinc.size() == plan.finc.size(), "%s: row face records", tag);
    for (int32_t t = 0; t < nsl; ++t) {
        std::map<int32_t, std::pair<int32_t, int32_t>> key;  // face -> (rank, lane)
        for (int32_t l = 0; l < kSliceRows; ++l) {
            const int32_t a = row_of(t, l);
            if (a < 0) continue;
            for (size_t r = 0; r < inc[a].size(); ++r) {
                const auto k = std::make_pair(int32_t(r), l);
                auto it = key.find(inc[a][r]);
                if (it == key.end() || k < it->second) key[inc[a][r]] = k;
            }
        }
        const int32_t n = plan.sf_ptr[t + 1] - plan.sf_ptr[t];
        CHECK(n == int32_t(key.size()), "%s: slice %d lists %d faces, %zu incident", tag, t, n, key.size());
        if (n != int32_t(key.size())) continue;
        std::vector<std::pair<std::pair<int32_t, int32_t>, int32_t>> order;
        for (const auto &kv : key) order.push_back({kv.second, kv.first});
        std::sort(order.begin(), order.end());
        for (int32_t k = 0; k < n; ++k) {
            const SliceFace &sf = plan.sface[size_t(plan.sf_ptr[t] + k)];
            const int32_t f = order[size_t(k)].second;
            CHECK(sf.f == f, "%s: slice %d list position %d", tag, t, k);
            for (int i = 0; i < 3; ++i) CHECK(sf.v[i] == m.faces[3 * size_t(f) + i], "%s: face %d vertices", tag, f);
        }
        for (int32_t l = 0; l < kSliceRows; ++l) {
            const int32_t a = row_of(t, l);
            if (a < 0) continue;
            std::vector<int32_t> got;
            for (int32_t k = plan.fptr[a]; k < plan.fptr[a + 1] && size_t(k) < plan.rfinc.size(); ++k) {
                const RowFace &e = plan.rfinc[size_t(k)];
                CHECK(k == plan.fptr[a] || plan.rfinc[size_t(k - 1)].lf < e.lf, "%s: row %d faces not in list order", tag, a);
                CHECK(int32_t(e.lf) < n, "%s: row %d face position", tag, a);
                if (int32_t(e.lf) >= n) continue;
                const int32_t f = plan.sface[size_t(plan.sf_ptr[t] + int32_t(e.lf))].f;
                got.push_back(f);
                CHECK(m.faces[3 * size_t(f) + (e.pi & 3u)] == a, "%s: row %d face %d position", tag, a, f);
            }
            std::sort(got.begin(), got.end());
            CHECK(got == inc[a], "%s: row %d faces", tag, a);
        }
    }
}

void check_row_plan_rejects()
{
    Mesh m = grid(6);
    std::vector<int32_t> rp, ci;
    RowPlan plan;
    Mesh dup = m;  // the same spring twice
    dup.springs.push_back(dup.springs[0]);
    dup.springs.push_back(dup.springs[1]);
    dup.rest.push_back(1.0);
    pattern(dup, rp, ci);
    CHECK(!build_row_plan(make_input(dup, rp, ci, false, 4, 0), dup.rest.data(), plan).empty(), "duplicate spring accepted");
    Mesh neg = m;
    neg.rest[3] = -0.5;
    pattern(neg, rp, ci);
    CHECK(!build_row_plan(make_input(neg, rp, ci, false, 4, 0), neg.rest.data(), plan).empty(), "negative rest length accepted");
}

// Insertion tiles: consecutive runs of whole units (row chunks) within the
// row and unit limits, or fixed row blocks; row_tile and row_unit agree.
void check_insert_tiles(const std::vector<PatchHdr> &units, int32_t nv, bool align,
                        const char *tag)
{
    InsertTiles t;
    const std::string msg = build_insert_tiles(units, nv, align, t);
    CHECK(msg.empty(), "%s: %s", tag, msg.c_str());
    if (!msg.empty()) return;
    const size_t nt = t.tile_row.size() - 1;
    CHECK(t.tile_row.front() == 0 && t.tile_row.back() == nv, "%s: tiles cover the rows", tag);
    CHECK(t.tile_unit.size() == nt + 1, "%s: tile_unit size", tag);
    CHECK(t.row_tile.size() == size_t(nv), "%s: row_tile size", tag);
    for (size_t k = 0; k < nt; ++k) {
        const int32_t r0 = t.tile_row[k], r1 = t.tile_row[k + 1];
        CHECK(r1 > r0 && r1 - r0 <= kInsTileRows, "%s: tile %zu rows %d..%d", tag, k, r0, r1);
        for (int32_t a = r0; a < r1; ++a) CHECK(t.row_tile[size_t(a)] == int32_t(k), "%s: row_tile %d", tag, a);
        if (align) {
            const int32_t u0 = t.tile_unit[k], u1 = t.tile_unit[k + 1];
            CHECK(u1 > u0 && u1 - u0 <= kInsTileUnits, "%s: tile %zu units", tag, k);
            CHECK(units[size_t(u0)].v0 == r0, "%s: tile %zu starts a unit", tag, k);
            CHECK(units[size_t(u1 - 1)].v0 + units[size_t(u1 - 1)].nown == r1, "%s: tile %zu ends a unit", tag, k);
            for (int32_t u = u0; u < u1; ++u)
                for (int32_t a = units[size_t(u)].v0; a < units[size_t(u)].v0 + units[size_t(u)].nown; ++a)
                    CHECK(t.row_unit[size_t(a)] == u, "%s: row_unit %d", tag, a);
            // greedy: the next unit would not have fitted
            if (k + 1 < nt)
                CHECK(u1 - u0 == kInsTileUnits ||
                          r1 - r0 + units[size_t(u1)].nown > kInsTileRows,
                      "%s: tile %zu closed early", tag, k);
        } else {
            CHECK(k + 1 == nt || r1 - r0 == kInsTileRows, "%s: fixed tile %zu", tag, k);
        }
    }
    // rejected inputs
    if (align && !units.empty()) {
        std::vector<PatchHdr> gap = units;
        gap.back().nown += 1;
        CHECK(!build_insert_tiles(gap, nv, true, t).empty(), "%s: units past nv accepted", tag);
    }
}

void check_insert_tiles_all()
{
    std::mt19937 rng(7);
    for (int rep = 0; rep < 4; ++rep) {
        std::vector<PatchHdr> units;
        int32_t v0 = 0;
        const int32_t nv = rep == 0 ? 9 : 1000 + 150000 * rep;
        while (v0 < nv) {
            PatchHdr h{};
            h.v0 = v0;
            h.nown = std::min<int32_t>(nv - v0, rep == 3 ? 1 + int32_t(rng() % 3) : 1 + int32_t(rng() % 64));
            units.push_back(h);
            v0 += h.nown;
        }
        char tag[64];
        std::snprintf(tag, sizeof(tag), "tiles rep %d", rep);
        check_insert_tiles(units, nv, true, tag);
        check_insert_tiles(units, nv, false, tag);
    }
}

}  // namespace

int main()
{
    const Mesh g10 = grid(10), g37 = grid(37), g64 = grid(64);
    const Mesh r1 = random_mesh(300, 700, 1), r2 = random_mesh(2000, 6000, 2);
    check_patch_plan(g10, false, 8, 40 * 1024, "grid10");
    check_patch_plan(g37, true, 4, 6144, "grid37 faces small patches");
    check_patch_plan(g37, false, 8, 6144, "grid37 fp64 small patches");
    check_patch_plan(g64, true, 4, 40 * 1024, "grid64 faces");
    check_patch_plan(r1, true, 8, 8192, "random300 faces");
    check_patch_plan(r2, true, 4, 16384, "random2000 faces");
    check_element_once_plan(g10, false, 8, 40 * 1024, "grid10 element-once");
    check_element_once_plan(g37, true, 4, 6144, "grid37 faces element-once small patches");
    check_element_once_plan(g64, true, 4, 40 * 1024, "grid64 faces element-once");
    check_element_once_plan(r1, true, 8, 8192, "random300 faces element-once");
    check_element_once_plan(r2, true, 4, 16384, "random2000 faces element-once");
    check_row_plan(g10, false, "grid10 rows");
    {
        // a chain of 40,000 vertices with one spring across it: differences
        // beyond 16 bits, so the slices keep full vertex ids
        Mesh chain;
        chain.nv = 40000;
        for (int32_t v = 0; v + 1 < chain.nv; ++v) {
            chain.springs.push_back(v);
            chain.springs.push_back(v + 1);
            chain.rest.push_back(1.0);
        }
        chain.springs.push_back(3);
        chain.springs.push_back(39990);
        chain.rest.push_back(2.0);
        auto narrow = [&](const Mesh &mm) {
            std::vector<int32_t> rp, ci;
            pattern(mm, rp, ci);
            RowPlan rplan;
            const std::string err = build_row_plan(make_input(mm, rp, ci, false, 4, 0), mm.rest.data(), rplan);
            CHECK(err.empty(), "chain: %s", err.c_str());
            return !rplan.sl_d16.empty();
        };
        check_row_plan(chain, false, "chain40000 rows wide");
        CHECK(!narrow(chain), "chain40000 with a long spring: 16-bit differences kept");
        chain.springs.resize(chain.springs.size() - 2);
        chain.rest.pop_back();
        check_row_plan(chain, false, "chain40000 rows narrow");
        CHECK(narrow(chain), "chain40000: no 16-bit differences");
    }
    check_row_plan(g64, true, "grid64 rows faces");
    check_row_plan(r1, true, "random300 rows faces");
    check_row_plan(r2, false, "random2000 rows");
    check_row_plan_rejects();
    check_insert_tiles_all();
    if (g_fail) {
        std::printf("%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("all plan checks passed\n");
    return 0;
}
