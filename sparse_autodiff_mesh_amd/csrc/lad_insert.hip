// lad_insert.hip -- double-buffered insertion of runtime contacts: vertex-
// vertex pairs and vertex-face contacts.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", key design 4: interaction elements found at run time (the
// page names vertex-vertex and vertex-face ones) add off-diagonal Hessian
// blocks; discovery is decoupled from evaluation, and a double-buffered CSR
// with reserved storage takes the new non-zeros in parallel on the GPU, then
// the buffers swap, with no CPU round trip.
//
// Pattern of a step = topology pattern U {(i,j), (j,i) : current pairs}
// U {(v,t), (t,v) : current contacts (v, face), t a vertex of the face},
// rows sorted and de-duplicated; the previous step's contacts are dropped.
//
// Elements of one insert are numbered pairs first (ids 0 .. np-1), then
// vertex-face contacts (ids np .. np+nvf-1).  Each element has one
// incidence entry per vertex (2 for a pair, 4 for a contact); a row's
// entries are kept sorted by element id, which fixes the order in which
// the row evaluates them.  A row's new partners go to pnew at three slots
// per incidence entry (a contact's vertex row gains up to three).
// Buffer 0 is the immutable topology pattern; buffers 1 and 2 alternate.
// Every kernel below picks the back buffer from the device-side state, so
// the host never needs to know which buffer is active.  The insert commits
// (flips `active`) only if every device-side check passed.
//
// An insert is three launches: count (per row and per tile), bucket (the
// entries grouped by tile), and one workgroup per tile of consecutive rows
// that builds the incidence lists and the new rows of its tile and chains
// the tiles' new-block sums into the row pointers by decoupled look-back
// (each tile publishes its own sum, then its sum including every earlier
// tile, in one status word; a tile adds up its predecessors' words back to
// the nearest inclusive one).  On the row path the last tile commits; the
// patch path merges every row, then commits, in two more launches.
//
// A row that no pair touches keeps its topology row, shifted to its new
// offset.  The row-owner kernels read such rows through the topology
// pattern, so on that path an insert writes the columns of the touched rows
// only (a few percent of the rows) and the rest of the column array is
// filled in when a caller asks for the pattern; the patch path reads every
// row and gets the complete array at once.
#include "lad_internal.h"

namespace lad {

namespace {

__device__ __forceinline__ int back_of(const DevState *st) { return st->active == 1 ? 2 : 1; }

// Rows whose topology row has at most kRegCols columns (and at most kRegNew
// new ones) are handled with their columns in registers.
constexpr int kRegCols = 16;
constexpr int kRegNew = 8;

// Workgroup barrier that orders LDS only: it does not wait for the
// workgroup's global stores to complete (which a full barrier does, at
// about a memory round trip each time).  Global data written before it is
// not made visible to other threads by it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive prefix of v over the workgroup (kThreads threads) and the
// total; wsum holds kThreads / 64 ints of LDS.
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t &total, int32_t *wsum)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    lds_barrier();
    int32_t before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
        const int32_t y = wsum[i];
        before += i < w ? y : 0;
        total += y;
    }
    lds_barrier();
    return before + incl - v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v |= __shfl_xor(v, m, 64);
    return v;
}

// Index of incidence entry k of element q: 2 per pair, then 4 per contact.
__device__ __forceinline__ int64_t entry_of(int32_t q, int k, int32_t np)
{
    return q < np ? 2 * int64_t(q) + k : 2 * int64_t(np) + 4 * int64_t(q - np) + k;
}

// First kernel of an insert, one workgroup per kThreads elements (a thread
// per element).  Records the buffer it writes and advances the insert
// counter (thread 0), copies the elements into the back buffer, validates
// them (bit 1 of err_cur if one fails), and groups the workgroup's
// incidence entries by tile: an LDS histogram over the tiles gives each
// entry its rank in its tile (arrival order); the histogram and its
// exclusive prefix go to hist / hoff (tile-major, nwg workgroups per tile)
// and the entries to the workgroup's part of seg, tile after tile.  An
// entry holds (row, element, topology row start, topology row length) and
// the row's partners in the element: a pair's other vertex; for a contact,
// the face's three vertices (row = the contact vertex) or the contact
// vertex (row = a face vertex); INT32_MAX past the last; then the row's
// vertex's place in the element (0: the pair's first vertex or the
// contact vertex).
__global__ void __launch_bounds__(kThreads)
k_ins_count(DevState *st, const int32_t *__restrict__ pairs_in, int32_t np,
            const int32_t *__restrict__ vf_in, int32_t nvf, int32_t nv, int32_t nf, int32_t nwg,
            InsertBufs b)
{
    extern __shared__ int32_t bins[];  // [ntiles]: entries per tile, then their prefix
    __shared__ int32_t wsum[kThreads / 64];
    const int tid = threadIdx.x;
    const int32_t g = blockIdx.x, nt = b.ntiles;
    const int32_t q = g * kThreads + tid;
    const int bk = back_of(st);
    if (q == 0) {
        st->ins_back = bk;
        st->ins_seq = st->ins_seq + 1u;
    }
    for (int32_t i = tid; i < nt; i += kThreads) bins[i] = 0;
    const bool live = q < np + nvf;
    int32_t vert[4] = {0, 0, 0, 0};
    int m = 0;
    if (live) {
        if (q < np) {
            const int32_t i = pairs_in[2 * q], j = pairs_in[2 * q + 1];
            b.pairs[bk][2 * q] = i;
            b.pairs[bk][2 * q + 1] = j;
            if (i >= 0 && i < nv && j >= 0 && j < nv && i != j) {
                vert[0] = i;
                vert[1] = j;
                m = 2;
            }
        } else {
            const int32_t e = q - np;
            const int32_t v = vf_in[2 * e], f = vf_in[2 * e + 1];
            b.vf[bk][2 * e] = v;
            b.vf[bk][2 * e + 1] = f;
            if (v >= 0 && v < nv && f >= 0 && f < nf) {
                vert[0] = v;
                m = 4;
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    vert[1 + k] = b.faces[3 * int64_t(f) + k];
                    if (vert[1 + k] == v) m = 0;
                }
            }
        }
        if (m == 0) atomicOr(&st->err_cur, 1);
    }
    int32_t tl[4], rb[4], re[4], rank[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        tl[k] = k < m ? b.row_tile[vert[k]] : 0;
        rb[k] = k < m ? b.rp[0][vert[k]] : 0;
        re[k] = k < m ? b.rp[0][vert[k] + 1] : 0;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 4; ++k) rank[k] = k < m ? atomicAdd(&bins[tl[k]], 1) : 0;
    lds_barrier();
    {
        const int32_t per = (nt + kThreads - 1) / kThreads;
        const int32_t i0 = min(tid * per, nt), i1 = min(i0 + per, nt);
        int32_t run = 0;
        for (int32_t i = i0; i < i1; ++i) run += bins[i];
        int32_t tot;
        run = block_excl_scan(run, tot, wsum);
        for (int32_t i = i0; i < i1; ++i) {
            const int32_t c = bins[i];
            b.hist[int64_t(i) * nwg + g] = c;
            b.hoff[int64_t(i) * nwg + g] = run;
            bins[i] = run;
            run += c;
        }
    }
    lds_barrier();
    int4 *seg = b.seg + 2 * int64_t(g) * kInsWgEnt;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (k < m) {
            const int32_t pos = bins[tl[k]] + rank[k];
            seg[2 * pos] = make_int4(vert[k], q, rb[k], re[k] - rb[k]);
            seg[2 * pos + 1] = m == 2   ? make_int4(vert[1 - k], INT32_MAX, INT32_MAX, k)
                               : k == 0 ? make_int4(vert[1], vert[2], vert[3], 0)
                                        : make_int4(vert[0], INT32_MAX, INT32_MAX, k);
        }
}

__device__ __forceinline__ int32_t lower_bound(const int32_t *c, int32_t lo, int32_t hi, int32_t x)
{
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (c[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void merge_row(const int32_t *cb, int32_t len, const int32_t *pn,
                                          int32_t nn, int32_t *out)
{
    int32_t i = 0, m = 0;
    for (int32_t o = 0; o < len + nn; ++o) {
        const bool take_new = m < nn && (i >= len || pn[m] < cb[i]);
        out[o] = take_new ? pn[m++] : cb[i++];
    }
}

// A touched row a in global memory (any number of entries p0 .. p0+d, any
// topology row rb0 .. rb0+len): its entries (in pinc, in any order) sorted
// by element id, its distinct partners that the topology row lacks,
// ascending, into pnew at three slots per entry from p0, and per entry the
// slots, from the row's start, of a pair's (row, partner) block (-1 for a
// contact) and of the diagonal block, and the pair's partner and orientation
// (see PatternBufs::pslot), into pslot; the caller adds the row's start to
// the slots.  Returns the number of new partners.
__device__ int32_t order_row_global(const InsertBufs &b, int bk, int32_t np, int32_t a,
                                    int32_t p0, int32_t d, int32_t rb0, int32_t len)
{
    int32_t *pl = b.pinc[bk];
    const int32_t *prs = b.pairs[bk];
    int32_t *pn = b.pnew[bk] + 3 * int64_t(p0);
    const int32_t p1 = p0 + d, rb1 = rb0 + len;
    for (int32_t i = p0 + 1; i < p1; ++i) {
        const int32_t key = pl[i];
        int32_t j = i - 1;
        while (j >= p0 && pl[j] > key) {
            pl[j + 1] = pl[j];
            --j;
        }
        pl[j + 1] = key;
    }
    int32_t nn = 0;
    for (int32_t k = p0; k < p1; ++k) {
        const int32_t q = pl[k];
        int32_t part[3];
        int npart = 0;
        if (q < np) {
            part[npart++] = prs[2 * q] == a ? prs[2 * q + 1] : prs[2 * q];
        } else {
            const int32_t v = b.vf[bk][2 * (q - np)], f = b.vf[bk][2 * (q - np) + 1];
            if (v == a)
                for (int t = 0; t < 3; ++t) part[npart++] = b.faces[3 * int64_t(f) + t];
            else
                part[npart++] = v;
        }
        for (int t = 0; t < npart; ++t) {
            const int32_t other = part[t];
            const int32_t pos = lower_bound(b.ci[0], rb0, rb1, other);
            if (pos < rb1 && b.ci[0][pos] == other) continue;
            bool dup = false;
            for (int32_t m = 0; m < nn; ++m) dup |= pn[m] == other;
            if (!dup) pn[nn++] = other;
        }
    }
    for (int32_t i = 1; i < nn; ++i) {
        const int32_t key = pn[i];
        int32_t j = i - 1;
        while (j >= 0 && pn[j] > key) {
            pn[j + 1] = pn[j];
            --j;
        }
        pn[j + 1] = key;
    }
    auto below = [&](int32_t col) {
        return (lower_bound(b.ci[0], rb0, rb1, col) - rb0) + lower_bound(pn, 0, nn, col);
    };
    const int32_t ds = below(a);
    for (int32_t k = p0; k < p1; ++k) {
        const int32_t q = pl[k];
        int4 ps = make_int4(-1, ds, -1, 0);
        if (q < np) {
            const bool first = prs[2 * q] == a;
            const int32_t other = first ? prs[2 * q + 1] : prs[2 * q];
            ps.x = below(other);
            ps.z = 2 * other + (first ? 1 : 0);
        }
        b.pslot[bk][k] = ps;
    }
    return nn;
}

// A touched row of at most kRegEnt entries and kRegCols topology columns,
// in registers: its topology columns c, and its partners part (three per
// entry, INT32_MAX where none) of which keep marks the new ones (neither in
// the topology row nor an earlier partner).
constexpr int kRegEnt = 4;
constexpr int kRegPart = 3 * kRegEnt;

struct RegRow {
    int32_t c[kRegCols];
    int32_t part[kRegPart];
    int32_t q[kRegEnt];  // the entries' elements, ascending (INT32_MAX past the last)
    uint32_t keep;       // bit k: part[k] is new
    uint32_t firstm;     // bit i: the row's vertex is entry i's pair's first vertex
    uint32_t place;      // bits 2i, 2i + 1: the row's vertex's place in entry i's element
};

__device__ __forceinline__ bool kept(const RegRow &w, int k) { return (w.keep >> k) & 1u; }

__device__ __forceinline__ int32_t reg_below(const RegRow &w, int32_t col)
{
    int32_t n = 0;
#pragma unroll
    for (int i = 0; i < kRegCols; ++i) n += w.c[i] < col ? 1 : 0;
#pragma unroll
    for (int k = 0; k < kRegPart; ++k) n += (kept(w, k) && w.part[k] < col) ? 1 : 0;
    return n;
}

// order_row_global for such a row in two parts: row_reg forms it in
// registers from its entries (element ids eq, partners ep, unsorted, in LDS)
// and its topology row, and returns the number of new partners;
// emit_row_reg stores it (entries from p0): trow, pinc_row, pinc, pslot,
// pnew and rins1.  The stores wait until the kernel's last global loads
// are issued, since a wait on a load also waits on older stores.
__device__ __forceinline__ void load_topo(const InsertBufs &b, int32_t rb0, int32_t len,
                                          int32_t c[kRegCols])
{
#pragma unroll
    for (int i = 0; i < kRegCols; ++i) c[i] = i < len ? b.ci[0][rb0 + i] : INT32_MAX;
}

// ctop: the row's topology columns (load_topo)
__device__ __forceinline__ int32_t row_reg(const int32_t ctop[kRegCols], int32_t d,
                                           const int32_t *eq, const int4 *ep, RegRow &w)
{
#pragma unroll
    for (int i = 0; i < kRegCols; ++i) w.c[i] = ctop[i];
    int4 pp[kRegEnt];
#pragma unroll
    for (int i = 0; i < kRegEnt; ++i) {
        w.q[i] = i < d ? eq[i] : INT32_MAX;
        pp[i] = i < d ? ep[i] : make_int4(INT32_MAX, INT32_MAX, INT32_MAX, 0);
    }
    // sort the entries by element id (odd-even transposition)
#pragma unroll
    for (int r = 0; r < kRegEnt; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < kRegEnt; i += 2) {
            const bool sw = w.q[i] > w.q[i + 1];
            const int32_t qa = sw ? w.q[i + 1] : w.q[i], qb = sw ? w.q[i] : w.q[i + 1];
            const int4 pa = sw ? pp[i + 1] : pp[i], pb = sw ? pp[i] : pp[i + 1];
            w.q[i] = qa;
            w.q[i + 1] = qb;
            pp[i] = pa;
            pp[i + 1] = pb;
        }
    w.firstm = 0;
    w.place = 0;
#pragma unroll
    for (int i = 0; i < kRegEnt; ++i) {
        w.part[3 * i] = pp[i].x;
        w.part[3 * i + 1] = pp[i].y;
        w.part[3 * i + 2] = pp[i].z;
        w.firstm |= pp[i].w == 0 ? (1u << i) : 0u;
        w.place |= uint32_t(pp[i].w & 3) << (2 * i);
    }
    int32_t nn = 0;
    w.keep = 0;
#pragma unroll
    for (int k = 0; k < kRegPart; ++k) {
        bool drop = w.part[k] == INT32_MAX;
#pragma unroll
        for (int i = 0; i < kRegCols; ++i) drop |= w.c[i] == w.part[k];
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) drop |= w.part[k2] == w.part[k];
        w.keep |= drop ? 0u : (1u << k);
        nn += drop ? 0 : 1;
    }
    return nn;
}

__device__ __forceinline__ void emit_row_reg(const InsertBufs &b, int bk, int32_t np, int32_t a,
                                             int32_t p0, int32_t d, int32_t s0, const RegRow &w)
{
    int32_t *pn = b.pnew[bk] + 3 * int64_t(p0);
    int32_t first = INT32_MAX;
#pragma unroll
    for (int k = 0; k < kRegPart; ++k)
        if (kept(w, k)) {
            int32_t rk = 0;
#pragma unroll
            for (int k2 = 0; k2 < kRegPart; ++k2)
                rk += (kept(w, k2) && w.part[k2] < w.part[k]) ? 1 : 0;
            pn[rk] = w.part[k];
            first = min(first, w.part[k]);
        }
    b.rins1[bk][a] = first;
    const int32_t ds = s0 + reg_below(w, a);
    const int32_t sw = __popc(w.keep) > kMaxIns ? -1 - s0 : s0;
#pragma unroll
    for (int i = 0; i < kRegEnt; ++i)
        if (i < d) {
            b.trow[bk][p0 + i] = i == 0 ? a : -1;
            b.pinc_row[bk][p0 + i] = a;
            b.pinc[bk][p0 + i] = w.q[i];
            const bool pair = w.q[i] < np;
            b.pslot[bk][p0 + i] =
                make_int4(pair ? s0 + reg_below(w, w.part[3 * i]) : -1, ds,
                          pair ? 2 * w.part[3 * i] + int32_t((w.firstm >> i) & 1u)
                               : -2 - int32_t((w.place >> (2 * i)) & 3u),
                          sw);
        }
}

// The active columns of a touched row, from slot o0: its topology columns
// merged with its new partners, each at its index in its own list plus the
// number of smaller columns in the other (the lists are disjoint).
__device__ __forceinline__ void merge_reg(const RegRow &w, int32_t len, int32_t *out)
{
#pragma unroll
    for (int i = 0; i < kRegCols; ++i) {
        int32_t before = 0;
#pragma unroll
        for (int k = 0; k < kRegPart; ++k) before += (kept(w, k) && w.part[k] < w.c[i]) ? 1 : 0;
        if (i < len) out[i + before] = w.c[i];
    }
#pragma unroll
    for (int k = 0; k < kRegPart; ++k)
        if (kept(w, k)) out[reg_below(w, w.part[k])] = w.part[k];
}

// The same from global memory (topology row rb0 .. rb0+len, nn new
// partners in pnew from 3 p0); short rows in registers, long ones by a
// sequential merge.
__device__ __forceinline__ void merge_touched(const InsertBufs &b, int bk, int32_t rb0,
                                              int32_t len, int32_t p0, int32_t o0, int32_t nn)
{
    const int32_t *cb = b.ci[0] + rb0;
    const int32_t *pn = b.pnew[bk] + 3 * int64_t(p0);
    int32_t *out = b.ci[bk] + o0;
    if (len <= kRegCols && nn <= kRegNew) {
        int32_t c[kRegCols], p[kRegNew];
#pragma unroll
        for (int i = 0; i < kRegCols; ++i) c[i] = i < len ? cb[i] : INT32_MAX;
#pragma unroll
        for (int m = 0; m < kRegNew; ++m) p[m] = m < nn ? pn[m] : INT32_MAX;
#pragma unroll
        for (int i = 0; i < kRegCols; ++i) {
            int32_t before = 0;
#pragma unroll
            for (int m = 0; m < kRegNew; ++m) before += p[m] < c[i] ? 1 : 0;
            if (i < len) out[i + before] = c[i];
        }
#pragma unroll
        for (int m = 0; m < kRegNew; ++m) {
            int32_t before = 0;
#pragma unroll
            for (int i = 0; i < kRegCols; ++i) before += c[i] < p[m] ? 1 : 0;
            if (m < nn) out[m + before] = p[m];
        }
    } else {
        merge_row(cb, len, pn, nn, out);
    }
}

// Look-back status of a tile: its new-block sum (the tile's alone, flag 1,
// or inclusive of every earlier tile, flag 2), the error bits seen so far
// and the insert's tag (a word of another insert reads as not yet written).
constexpr uint32_t kTagMask = (1u << 26) - 1u;

__device__ __forceinline__ unsigned long long tile_word(uint32_t tag, uint32_t flag, uint32_t err,
                                                        uint32_t val)
{
    return (static_cast<unsigned long long>(tag & kTagMask) << 38) |
           (static_cast<unsigned long long>(err & 15u) << 34) |
           (static_cast<unsigned long long>(flag & 3u) << 32) | val;
}

// Bound on the look-back's polls (well over a second): a chain that does
// not complete reports error 4 instead of waiting for ever.
constexpr int32_t kSpinLimit = 1 << 20;

constexpr int kTileSeg = kInsTileRows / kThreads;  // rows per thread in the row passes
static_assert(kInsTileRows % kThreads == 0, "tile rows per thread");
constexpr int kTileEnt = 512;  // incidence entries of a tile kept in LDS, at most

// Second kernel, one workgroup per tile (workgroup t = tile t).  A tile
// waits only on tiles of lower index; workgroups are dispatched in index
// order, so those already run (and a bounded wait turns a broken chain into
// error 4 rather than a hang).  For the tile's rows [r0, r1):
//   A. the tile's entries, gathered from the count kernel's workgroups
//      (their counts and offsets for this tile: one read each), each
//      entry's rank in its row counted in LDS; the tile's first incidence
//      entry e0 is the sum of those offsets;
//   B. the exclusive prefix of the row counts, the entries put at their
//      row positions (LDS when they fit, else pinc);
//   C. each touched row's new partners counted (row_reg, else
//      order_row_global) by the row's owner: the thread that read the row's
//      entry of rank 0, which started loading the row's topology columns
//      in A;
//   D. the exclusive prefix of the new blocks over the tile, the chunk
//      capacity checks (row path), then the prefix over all earlier tiles
//      by decoupled look-back;
//   E. the stores: incidence offsets, first inserted columns, the touched
//      rows (emit_row_reg), the active row pointers and on the row path the
//      touched rows' columns; the last tile commits.
// On CDNA a wait on a global load also waits on every older global store,
// so the tile's stores are issued after its last loads, and barriers that
// only order LDS do not wait for global stores at all.
__global__ void __launch_bounds__(kThreads)
k_ins_tiles(DevState *st, int32_t np, int32_t nvf, int32_t nv, int32_t nwg,
            const PatchHdr *__restrict__ hdr, InsertBufs b, int row_path)
{
    __shared__ int32_t s_cnt[kInsTileRows];      // entries per row, then their offsets
    __shared__ int32_t s_nn[kInsTileRows];       // new blocks per row, then their prefix
    __shared__ int32_t s_rb[kInsTileRows];       // topology row start of touched rows
    __shared__ int32_t s_len[kInsTileRows];      // ... and length
    __shared__ int32_t s_gp[kInsMaxWg + 1];      // per count workgroup: prefix of its entries here,
    __shared__ int32_t s_go[kInsMaxWg];          // and their offset in its part of seg
    __shared__ int32_t s_eq[kTileEnt];           // entries at their row positions: element,
    __shared__ int4 s_ep[kTileEnt];              // partners
    __shared__ int32_t s_ugrow[kInsTileUnits];
    __shared__ int32_t wsum[kThreads / 64];
    __shared__ uint32_t s_vs[kThreads / 64], s_es[kThreads / 64];
    __shared__ int32_t s_ok[kThreads / 64];
    __shared__ int32_t s_err, s_first, s_gap;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int32_t nt = b.ntiles;
    const int32_t t = int32_t(blockIdx.x);
    const int bk = st->ins_back;
    const uint32_t tag = st->ins_seq;
    const int32_t r0 = b.tile_row[t], r1 = b.tile_row[t + 1], nr = r1 - r0;
    const int32_t u0 = row_path ? b.tile_unit[t] : 0, u1 = row_path ? b.tile_unit[t + 1] : 0;
    // the count workgroups' entries for this tile; topology row pointers
    // (used in E); all read before anything waits
    constexpr int kWgPer = kInsMaxWg / kThreads;
    int32_t hc[kWgPer], ho[kWgPer];
#pragma unroll
    for (int j = 0; j < kWgPer; ++j) {
        const int32_t gg = tid * kWgPer + j;
        hc[j] = gg < nwg ? b.hist[int64_t(t) * nwg + gg] : 0;
        ho[j] = gg < nwg ? b.hoff[int64_t(t) * nwg + gg] : 0;
    }
    int32_t rp0v[kTileSeg];  // rows tid + kThreads j (coalesced)
#pragma unroll
    for (int j = 0; j < kTileSeg; ++j) {
        const int32_t i = tid + kThreads * j;
        rp0v[j] = i < nr ? b.rp[0][r0 + i] : 0;
    }
    for (int32_t i = tid; i < nr; i += kThreads) s_cnt[i] = 0;
    for (int32_t i = tid; i < u1 - u0; i += kThreads) s_ugrow[i] = 0;
    if (tid == 0) s_err = 0;
    int32_t tcnt, e0;
    {
        int32_t sc = 0, so = 0;
#pragma unroll
        for (int j = 0; j < kWgPer; ++j) {
            sc += hc[j];
            so += ho[j];
        }
        int32_t run = block_excl_scan(sc, tcnt, wsum);  // its barriers order the set-up above
#pragma unroll
        for (int j = 0; j < kWgPer; ++j) {
            const int32_t gg = tid * kWgPer + j;
            if (gg < nwg) {
                s_gp[gg] = run;
                s_go[gg] = ho[j];
            }
            run += hc[j];
        }
        if (tid == 0) s_gp[nwg] = tcnt;
        block_excl_scan(so, e0, wsum);  // e0 = the sum of the offsets
    }
    const int32_t e1 = e0 + tcnt;
    const bool ent_lds = tcnt <= kTileEnt;
    // entry k of the tile: workgroup gg (s_gp[gg] <= k < s_gp[gg+1]), at
    // s_go[gg] + k - s_gp[gg] in its part of seg
    auto seg_index = [&](int32_t k) __attribute__((always_inline)) {
        int32_t lo = 0, hi = nwg - 1;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (s_gp[mid] <= k) lo = mid;
            else hi = mid - 1;
        }
        return int64_t(lo) * kInsWgEnt + s_go[lo] + (k - s_gp[lo]);
    };

    // A. ranks of the entries in their rows (a thread's first entry kept in
    // registers, later ones' ranks in erank).  The entry of rank 0 in its
    // row makes its thread the row's owner in C and E; the owner of a
    // short row starts loading its topology columns now.
    int4 my_h = make_int4(0, 0, 0, 0), my_p = my_h;
    int32_t my_rank = 1;
    int32_t ctop[kRegCols];
    for (int32_t k = tid; k < tcnt; k += kThreads) {
        const int64_t si = seg_index(k);
        const int4 h = b.seg[2 * si];
        const int32_t i = h.x - r0;
        const int32_t rk = atomicAdd(&s_cnt[i], 1);
        if (rk == 0) {
            s_rb[i] = h.z;
            s_len[i] = h.w;
        }
        if (k == tid) {
            my_h = h;
            my_p = b.seg[2 * si + 1];
            my_rank = rk;
        } else {
            b.erank[si] = rk;
        }
    }
    const bool own = tid < tcnt && my_rank == 0;
    if (own && my_h.w <= kRegCols) load_topo(b, my_h.z, my_h.w, ctop);
    lds_barrier();

    // B. row offsets; entries at their positions (LDS when the tile's
    // entries fit, else pinc)
    {
        int32_t rc[kTileSeg], sum = 0;
#pragma unroll
        for (int j = 0; j < kTileSeg; ++j) {
            const int32_t i = tid * kTileSeg + j;
            rc[j] = i < nr ? s_cnt[i] : 0;
            sum += rc[j];
        }
        int32_t tot;
        int32_t run = block_excl_scan(sum, tot, wsum);
#pragma unroll
        for (int j = 0; j < kTileSeg; ++j) {
            const int32_t i = tid * kTileSeg + j;
            if (i < nr) {
                s_cnt[i] = run;
                s_nn[i] = 0;
            }
            run += rc[j];
        }
    }
    lds_barrier();
    if (ent_lds) {
        if (tid < tcnt) {
            const int32_t lp = s_cnt[my_h.x - r0] + my_rank;
            s_eq[lp] = my_h.y;
            s_ep[lp] = my_p;
        }
        for (int32_t k = tid + kThreads; k < tcnt; k += kThreads) {
            const int64_t si = seg_index(k);
            const int32_t lp = s_cnt[b.seg[2 * si].x - r0] + b.erank[si];
            s_eq[lp] = b.seg[2 * si].y;
            s_ep[lp] = b.seg[2 * si + 1];
        }
        lds_barrier();
    } else {
        if (tid < tcnt) b.pinc[bk][e0 + s_cnt[my_h.x - r0] + my_rank] = my_h.y;
        for (int32_t k = tid + kThreads; k < tcnt; k += kThreads) {
            const int64_t si = seg_index(k);
            b.pinc[bk][e0 + s_cnt[b.seg[2 * si].x - r0] + b.erank[si]] = b.seg[2 * si].y;
        }
        __syncthreads();  // the entries went through global memory
    }

    // C. each touched row's new partners counted by its owner: a thread's
    // own row formed in registers and stored in E; further rows (a tile of
    // more than kThreads entries) and long rows stored here
    auto row_span = [&](int32_t i, int32_t &off, int32_t &d) __attribute__((always_inline)) {
        off = s_cnt[i];
        d = (i + 1 < nr ? s_cnt[i + 1] : tcnt) - off;
    };
    auto slow_row = [&](int32_t i, int32_t off, int32_t d) __attribute__((always_inline)) {
        const int32_t a = r0 + i, p0 = e0 + off;
        for (int32_t k = 0; k < d; ++k) {
            b.trow[bk][p0 + k] = k == 0 ? a : -1;
            b.pinc_row[bk][p0 + k] = a;
            if (ent_lds) b.pinc[bk][p0 + k] = s_eq[off + k];
        }
        const int32_t nn = order_row_global(b, bk, np, a, p0, d, s_rb[i], s_len[i]);
        b.rins1[bk][a] = nn > 0 ? b.pnew[bk][3 * int64_t(p0)] : INT32_MAX;
        return nn;
    };
    auto count_row = [&](int32_t i, int32_t nn) __attribute__((always_inline)) {
        s_nn[i] = nn;
        if (row_path && nn > 0) atomicAdd(&s_ugrow[b.row_unit[r0 + i] - u0], nn);
    };
    RegRow w;
    bool w_ok = false;
    if (own) {
        const int32_t i = my_h.x - r0;
        int32_t off, d;
        row_span(i, off, d);
        if (ent_lds && d <= kRegEnt && my_h.w <= kRegCols) {
            count_row(i, row_reg(ctop, d, s_eq + off, s_ep + off, w));
            w_ok = true;
        } else {
            count_row(i, slow_row(i, off, d));
        }
    }
    for (int32_t k = tid + kThreads; k < tcnt; k += kThreads) {
        const int64_t si = seg_index(k);
        if (b.erank[si] != 0) continue;
        const int32_t i = b.seg[2 * si].x - r0;
        int32_t off, d;
        row_span(i, off, d);
        count_row(i, slow_row(i, off, d));
    }
    lds_barrier();

    // D. prefix of the new blocks within the tile, capacity checks
    int32_t agg;
    {
        int32_t c[kTileSeg], sum = 0;
#pragma unroll
        for (int j = 0; j < kTileSeg; ++j) {
            const int32_t i = tid * kTileSeg + j;
            c[j] = i < nr ? s_nn[i] : 0;
            sum += c[j];
        }
        int32_t run = block_excl_scan(sum, agg, wsum);
#pragma unroll
        for (int j = 0; j < kTileSeg; ++j) {
            const int32_t i = tid * kTileSeg + j;
            if (i < nr) s_nn[i] = run;
            run += c[j];
        }
    }
    for (int32_t u = u0 + tid; u < u1; u += kThreads)
        if (hdr[u].nblk + s_ugrow[u - u0] > hdr[u].amap_cap) atomicOr(&s_err, 2);
    lds_barrier();
    const uint32_t err = uint32_t(s_err);
    // ... and over the earlier tiles: the status words of up to kLook
    // preceding tiles are read at once (their loads issued before this
    // tile's own word is stored); the walk ends at the nearest inclusive
    // word once every word before it has arrived (words that arrived are
    // not read again), else the block moves kLook tiles back
    // The stores that do not depend on the earlier tiles (incidence
    // offsets, the first inserted column of untouched rows, the owned
    // register rows).  They go out after the look-back: a load issued
    // after them would wait for them too.
    auto late_stores = [&](int32_t X) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kTileSeg; ++j) {
            const int32_t i = tid + kThreads * j;
            if (i < nr) {
                const int32_t off = s_cnt[i];
                b.pinc_ptr[bk][r0 + i] = e0 + off;
                if ((i + 1 < nr ? s_cnt[i + 1] : tcnt) == off) b.rins1[bk][r0 + i] = INT32_MAX;
            }
        }
        if (tid == 0 && t == nt - 1) b.pinc_ptr[bk][nv] = e1;
        if (w_ok) {
            const int32_t i = my_h.x - r0;
            int32_t off, d;
            row_span(i, off, d);
            emit_row_reg(b, bk, np, r0 + i, e0 + off, d, my_h.z + X + s_nn[i], w);
        }
    };
    constexpr int kLookPer = 4, kLook = kLookPer * kThreads;
    uint32_t excl = 0, eacc = 0;
    if (t == 0) {
        if (tid == 0)
            __hip_atomic_store(&b.tstat[0], tile_word(tag, 2, err, uint32_t(agg)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        int32_t j = t - 1, spins = 0;
        unsigned long long wd[kLookPer];
        bool got[kLookPer];
        auto poll = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < kLookPer; ++k) {
                const int32_t idx = j - (tid * kLookPer + k);
                if (!got[k])
                    wd[k] = idx >= 0 ? __hip_atomic_load(&b.tstat[int64_t(idx) * kStatStride],
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                     : tile_word(tag, 2, 0, 0);
            }
        };
#pragma unroll
        for (int k = 0; k < kLookPer; ++k) got[k] = false;
        poll();  // the first window's loads go out before this tile's word
        if (tid == 0)
            __hip_atomic_store(&b.tstat[int64_t(t) * kStatStride],
                               tile_word(tag, 1, err, uint32_t(agg)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        bool fresh = true;  // wd holds loads of the current window not yet examined
        for (;;) {
            int first = kLook;
            bool timed_out = false;
            for (;;) {
                if (!fresh) poll();
                fresh = false;
                if (tid == 0) {
                    s_first = kLook;
                    s_gap = kLook;
                }
                lds_barrier();
#pragma unroll
                for (int k = 0; k < kLookPer; ++k) {
                    got[k] = uint32_t(wd[k] >> 38) == (tag & kTagMask) && ((wd[k] >> 32) & 3u) != 0;
                    if (!got[k]) atomicMin(&s_gap, tid * kLookPer + k);
                    else if (((wd[k] >> 32) & 3u) == 2u) atomicMin(&s_first, tid * kLookPer + k);
                }
                lds_barrier();
                first = s_first;
                const int gap = s_gap;
                lds_barrier();
                if (first < gap || gap == kLook) break;  // block-uniform
                if (++spins >= kSpinLimit) {
                    timed_out = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            if (timed_out) {
                eacc |= 4u;
                break;
            }
            uint32_t v = 0, ev = 0;
#pragma unroll
            for (int k = 0; k < kLookPer; ++k)
                if (tid * kLookPer + k <= first) {
                    v += uint32_t(wd[k]);
                    ev |= uint32_t(wd[k] >> 34) & 15u;
                }
            v = wave_sum(v);
            ev = wave_or(ev);
            if (lane == 0) {
                s_vs[wid] = v;
                s_es[wid] = ev;
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < kThreads / 64; ++i) {
                excl += s_vs[i];
                eacc |= s_es[i];
            }
            lds_barrier();
            if (first < kLook) break;
            j -= kLook;
#pragma unroll
            for (int k = 0; k < kLookPer; ++k) got[k] = false;
        }
    }
    const uint32_t eincl = eacc | err;
    if (tid == 0 && t > 0)
        __hip_atomic_store(&b.tstat[int64_t(t) * kStatStride], tile_word(tag, 2, eincl, excl + uint32_t(agg)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t X = int32_t(excl);

    // E. the stores: those above, then the active row pointers and the
    // touched rows' columns; the commit (last tile)
    late_stores(X);
#pragma unroll
    for (int j = 0; j < kTileSeg; ++j) {
        const int32_t i = tid + kThreads * j;
        if (i < nr) b.rp[bk][r0 + i] = rp0v[j] + X + s_nn[i];
    }
    if (tid == 0 && t == nt - 1) {
        const int32_t nnzb = b.rp[0][nv] + X + agg;
        b.rp[bk][nv] = nnzb;
        if (row_path) {
            const int32_t e = st->err_cur | int32_t(eincl);
            if (e == 0) {
                st->np[bk] = np;
                st->nvf[bk] = nvf;
                st->nnzb[bk] = nnzb;
                st->active = bk;
            } else {
                st->err_latched |= e;
                st->err_cur = 0;
            }
        } else if (eincl != 0) {
            st->err_cur |= int32_t(eincl);  // the patch path's commit kernel reads it
        }
    }
    // rows ordered in global memory: their columns, and their slots made
    // absolute
    auto finish_slow = [&](int32_t i) __attribute__((always_inline)) {
        const int32_t nn = (i + 1 < nr ? s_nn[i + 1] : agg) - s_nn[i];
        const int32_t s0 = s_rb[i] + X + s_nn[i];
        if (row_path) merge_touched(b, bk, s_rb[i], s_len[i], e0 + s_cnt[i], s0, nn);
        int32_t off, d;
        row_span(i, off, d);
        for (int32_t k = e0 + off; k < e0 + off + d; ++k) {
            int4 ps = b.pslot[bk][k];
            ps.x = ps.x >= 0 ? s0 + ps.x : -1;
            ps.y += s0;
            ps.w = nn > kMaxIns ? -1 - s0 : s0;
            b.pslot[bk][k] = ps;
        }
    };
    if (own) {
        const int32_t i = my_h.x - r0;
        if (!w_ok) finish_slow(i);
        else if (row_path) merge_reg(w, my_h.w, b.ci[bk] + my_h.z + X + s_nn[i]);
    }
    for (int32_t k = tid + kThreads; k < tcnt; k += kThreads) {
        const int64_t si = seg_index(k);
        if (b.erank[si] == 0) finish_slow(b.seg[2 * si].x - r0);
    }
}

constexpr int kMergeThreads = 64;
constexpr int kMergeStage = 512;   // ints per staging buffer

// One 64-thread workgroup (one wave) per row chunk or patch, walking its
// rows 64 at a time.  For each group of rows the wave loads the topology
// columns of the group into LDS with coalesced loads, every lane builds its
// row of the new pattern in a second LDS buffer (a copy, or a merge with the
// row's new partners), and the wave stores the
// group's new columns with coalesced stores.  A group whose rows exceed the
// staging buffers is merged row by row straight from and to global memory.
// Finally the chunk's new block count is checked against its reserved
// staging capacity.  With use_active set it completes the active buffer of
// a row-path insert instead (every row rewritten with the same result, no
// check; nothing to do while the topology pattern is active).
__global__ void __launch_bounds__(kMergeThreads)
k_ins_merge(DevState *st, const PatchHdr *__restrict__ hdr, InsertBufs b, int use_active)
{
    __shared__ int32_t inb[kMergeStage], outb[kMergeStage];
    const int bk = use_active ? st->active : back_of(st);
    if (bk == 0) return;
    const PatchHdr h = hdr[blockIdx.x];
    const int32_t *cb = b.ci[0];
    const int32_t *rp0 = b.rp[0], *rpn = b.rp[bk];
    int32_t *out = b.ci[bk];
    const int lane = threadIdx.x;
    for (int32_t g0 = h.v0; g0 < h.v0 + h.nown; g0 += kMergeThreads) {
        const int32_t g1 = min(g0 + kMergeThreads, h.v0 + h.nown);
        const int32_t sb = rp0[g0], se = rp0[g1], ob = rpn[g0], oe = rpn[g1];
        const int32_t a = g0 + lane;
        const bool mine = a < g1;
        const int32_t rb0 = mine ? rp0[a] : 0, rb1 = mine ? rp0[a + 1] : 0;
        const int32_t o0 = mine ? rpn[a] : 0, o1 = mine ? rpn[a + 1] : 0;
        const int32_t len = rb1 - rb0, nn = (o1 - o0) - len;
        const int32_t *pn =
            (mine && nn > 0) ? b.pnew[bk] + 3 * int64_t(b.pinc_ptr[bk][a]) : nullptr;
        if (se - sb <= kMergeStage && oe - ob <= kMergeStage) {  // wave-uniform
            for (int32_t k = lane; k < se - sb; k += kMergeThreads) inb[k] = cb[sb + k];
            __syncthreads();
            if (mine) {
                if (nn == 0)
                    for (int32_t k = 0; k < len; ++k) outb[o0 - ob + k] = inb[rb0 - sb + k];
                else
                    merge_row(inb + (rb0 - sb), len, pn, nn, outb + (o0 - ob));
            }
            __syncthreads();
            for (int32_t k = lane; k < oe - ob; k += kMergeThreads) out[ob + k] = outb[k];
            __syncthreads();
        } else if (mine) {
            if (nn == 0)
                for (int32_t k = 0; k < len; ++k) out[o0 + k] = cb[rb0 + k];
            else
                merge_row(cb + rb0, len, pn, nn, out + o0);
        }
    }
    if (!use_active && lane == 0 && rpn[h.v0 + h.nown] - rpn[h.v0] > h.amap_cap)
        atomicOr(&st->err_cur, 2);
}

// Flip the active buffer if every check of this insert passed, else latch
// the error; either way re-arm err_cur for the next insert.  The kernels of
// the next call run after this one on the same stream.
__global__ void k_ins_commit(DevState *st, int32_t np, int32_t nvf, int32_t nv, InsertBufs b)
{
    const int bk = back_of(st);
    if (st->err_cur == 0) {
        st->np[bk] = np;
        st->nvf[bk] = nvf;
        st->nnzb[bk] = b.rp[bk][nv];
        st->active = bk;
    } else {
        st->err_latched |= st->err_cur;
        st->err_cur = 0;
    }
}

__global__ void k_restore_topology(DevState *st) { st->active = 0; }

inline unsigned blocks_for(int64_t n) { return unsigned((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_insert(DevState *st, const int32_t *d_pairs, int32_t np, const int32_t *d_vf,
                         int32_t nvf, int32_t nv, int32_t nf, InsertBufs b, const PatchHdr *hdr,
                         int32_t npatch, int complete_cols, hipStream_t s)
{
    // every array a kernel below dereferences must exist
    for (int k = 1; k <= 2; ++k)
        if (!b.rp[k] || !b.ci[k] || !b.pinc_ptr[k] || !b.pinc[k] || !b.pinc_row[k] ||
            !b.pnew[k] || !b.trow[k] || !b.pslot[k] || !b.rins1[k] ||
            (np > 0 && !b.pairs[k]) || (nvf > 0 && !b.vf[k]))
            return hipErrorInvalidValue;
    const int64_t nel = int64_t(np) + nvf;
    const int32_t nwg = int32_t((nel + kThreads - 1) / kThreads);
    if (!b.rp[0] || !b.ci[0] || !hdr || b.ntiles <= 0 || b.ntiles > kInsMaxTiles ||
        !b.tile_row || !b.row_tile || !b.tstat || !b.hist || !b.hoff || !b.seg || !b.erank ||
        nwg > b.max_wg || nwg > kInsMaxWg || (!complete_cols && (!b.tile_unit || !b.row_unit)) ||
        (nvf > 0 && (!b.faces || !d_vf)) || (np > 0 && !d_pairs))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_ins_count, dim3(nwg), dim3(kThreads), size_t(b.ntiles) * sizeof(int32_t),
                       s, st, d_pairs, np, d_vf, nvf, nv, nf, nwg, b);
    hipLaunchKernelGGL(k_ins_tiles, dim3(b.ntiles), dim3(kThreads), 0, s, st, np, nvf, nv, nwg, hdr,
                       b, complete_cols ? 0 : 1);
    if (complete_cols) {
        // patch path: every row's columns (and the capacity check per
        // patch), then the commit
        hipLaunchKernelGGL(k_ins_merge, dim3(npatch), dim3(kMergeThreads), 0, s, st, hdr, b, 0);
        hipLaunchKernelGGL(k_ins_commit, dim3(1), dim3(1), 0, s, st, np, nvf, nv, b);
    }
    return hipGetLastError();
}

hipError_t launch_complete_cols(DevState *st, InsertBufs b, const PatchHdr *hdr, int32_t npatch,
                                hipStream_t s)
{
    hipLaunchKernelGGL(k_ins_merge, dim3(npatch), dim3(kMergeThreads), 0, s, st, hdr, b, 1);
    return hipGetLastError();
}

hipError_t launch_restore_topology(DevState *st, hipStream_t s)
{
    hipLaunchKernelGGL(k_restore_topology, dim3(1), dim3(1), 0, s, st);
    return hipGetLastError();
}

}  // namespace lad
