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
// the host never needs to know which buffer is active.  The last kernel
// commits (flips `active`) only if every device-side check passed.
//
// A row that no pair touches keeps its topology row, shifted to its new
// offset.  The row-owner kernels read such rows through the topology
// pattern, so on that path an insert writes the columns of the touched rows
// only (a few percent of the rows) and the rest of the column array is
// filled in when a caller asks for the pattern; the patch path reads every
// row and gets the complete array at once.
#include "lad_internal.h"

namespace lad {

hipError_t launch_scan_back(const int32_t *in, int32_t *const out[3], const int32_t *add,
                            const DevState *st, int32_t n, int32_t *tmp, hipStream_t s);

namespace {

__device__ __forceinline__ int back_of(const DevState *st) { return st->active == 1 ? 2 : 1; }

// Rows whose topology row has at most kRegCols columns (and at most kRegNew
// new ones) are handled with their columns in registers.
constexpr int kRegCols = 16;
constexpr int kRegNew = 8;

// The vertices of element q of the back buffer (2 for a pair, 4 for a
// contact: the vertex, then its face's three); 0 if the element fails the
// device-side check (an index out of range, a pair with i == j, a contact
// whose vertex belongs to its face).
__device__ __forceinline__ int element_vertices(const InsertBufs &b, int bk, int32_t q,
                                                int32_t np, int32_t nv, int32_t nf,
                                                int32_t vert[4])
{
    if (q < np) {
        const int32_t i = b.pairs[bk][2 * q], j = b.pairs[bk][2 * q + 1];
        if (!(i >= 0 && i < nv && j >= 0 && j < nv && i != j)) return 0;
        vert[0] = i;
        vert[1] = j;
        return 2;
    }
    const int32_t e = q - np;
    const int32_t v = b.vf[bk][2 * e], f = b.vf[bk][2 * e + 1];
    if (!(v >= 0 && v < nv && f >= 0 && f < nf)) return 0;
    vert[0] = v;
    for (int k = 0; k < 3; ++k) {
        vert[1 + k] = b.faces[3 * int64_t(f) + k];
        if (vert[1 + k] == v) return 0;
    }
    return 4;
}

// Copy the elements into the back buffer, validate them and count the
// incidence entries per row.
__global__ void __launch_bounds__(kThreads)
k_ins_count(DevState *st, const int32_t *__restrict__ pairs_in, int32_t np,
            const int32_t *__restrict__ vf_in, int32_t nvf, int32_t nv, int32_t nf, InsertBufs b)
{
    const int32_t q = blockIdx.x * kThreads + threadIdx.x;
    if (q >= np + nvf) return;
    const int bk = back_of(st);
    if (q < np) {
        b.pairs[bk][2 * q] = pairs_in[2 * q];
        b.pairs[bk][2 * q + 1] = pairs_in[2 * q + 1];
    } else {
        b.vf[bk][2 * (q - np)] = vf_in[2 * (q - np)];
        b.vf[bk][2 * (q - np) + 1] = vf_in[2 * (q - np) + 1];
    }
    int32_t vert[4];
    const int m = element_vertices(b, bk, q, np, nv, nf, vert);
    if (m == 0) {
        atomicOr(&st->err_cur, 1);
        return;
    }
    for (int k = 0; k < m; ++k) atomicAdd(&b.cnt[vert[k]], 1);
}

// Scatter element ids into the per-row incidence lists; cnt returns to zero.
__global__ void __launch_bounds__(kThreads)
k_ins_fill(const DevState *st, int32_t np, int32_t nvf, int32_t nv, int32_t nf, InsertBufs b)
{
    const int32_t q = blockIdx.x * kThreads + threadIdx.x;
    if (q >= np + nvf) return;
    const int bk = back_of(st);
    int32_t vert[4];
    const int m = element_vertices(b, bk, q, np, nv, nf, vert);
    for (int k = 0; k < m; ++k) {
        const int32_t r = vert[k];
        const int32_t pos = b.pinc_ptr[bk][r] + atomicSub(&b.cnt[r], 1) - 1;
        b.pinc[bk][pos] = q;
        b.pinc_row[bk][pos] = r;
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

// Per row that contacts touch (one thread per incidence entry; the row's
// first entry does the work): order the row's entries by element id (fixed
// evaluation order), collect the distinct partners that are not already in
// the topology row (sorted, into pnew at three slots per entry from the
// row's offset) and store their number in nnew[row].  nnew is zero for
// every other row.  Every entry also records in trow whether it is its
// row's first (the row) or not (-1): the later kernels find the touched
// rows there in one load.  Only the first pinc_ptr[nv] entries were filled
// (elements that failed the device check have none), so threads past that
// read nothing else.
__global__ void __launch_bounds__(kThreads)
k_ins_rows(const DevState *st, int32_t nent, int32_t np, int32_t nv, InsertBufs b)
{
    const int32_t k = blockIdx.x * kThreads + threadIdx.x;
    if (k >= nent) return;
    const int bk = back_of(st);
    int32_t a = -1;
    if (k < b.pinc_ptr[bk][nv]) {
        const int32_t r = b.pinc_row[bk][k];
        if (r >= 0 && r < nv && k == b.pinc_ptr[bk][r]) a = r;
    }
    b.trow[bk][k] = a;
    if (a < 0) return;
    const int32_t p0 = k, p1 = b.pinc_ptr[bk][a + 1];
    const int32_t rb0 = b.rp[0][a], rb1 = b.rp[0][a + 1];
    int32_t *pl = b.pinc[bk];
    for (int32_t i = p0 + 1; i < p1; ++i) {
        const int32_t key = pl[i];
        int32_t j = i - 1;
        while (j >= p0 && pl[j] > key) {
            pl[j + 1] = pl[j];
            --j;
        }
        pl[j + 1] = key;
    }
    const int32_t *prs = b.pairs[bk];
    int32_t *pn = b.pnew[bk] + 3 * int64_t(p0);
    int32_t nn = 0;
    // the topology row in registers when it is short (membership tests
    // then take no dependent loads), else binary search
    const bool reg = rb1 - rb0 <= kRegCols;
    int32_t topo[kRegCols];
#pragma unroll
    for (int i = 0; i < kRegCols; ++i) topo[i] = (reg && rb0 + i < rb1) ? b.ci[0][rb0 + i] : -1;
    for (int32_t q0 = p0; q0 < p1; ++q0) {
        const int32_t q = pl[q0];
        // this row's partners in element q: a pair's other vertex; for a
        // contact, the face's vertices (row = the contact vertex) or the
        // contact vertex (row = a face vertex)
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
            bool in_topo = false;
            if (reg) {
#pragma unroll
                for (int i = 0; i < kRegCols; ++i) in_topo |= topo[i] == other;
            } else {
                const int32_t pos = lower_bound(b.ci[0], rb0, rb1, other);
                in_topo = pos < rb1 && b.ci[0][pos] == other;
            }
            if (in_topo) continue;
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
    b.nnew[a] = nn;
}

constexpr int kMergeThreads = 64;
constexpr int kMergeStage = 512;   // ints per staging buffer

__device__ __forceinline__ void merge_row(const int32_t *cb, int32_t len, const int32_t *pn,
                                          int32_t nn, int32_t *out)
{
    int32_t i = 0, m = 0;
    for (int32_t o = 0; o < len + nn; ++o) {
        const bool take_new = m < nn && (i >= len || pn[m] < cb[i]);
        out[o] = take_new ? pn[m++] : cb[i++];
    }
}

// Columns of the rows that pairs touch (one thread per incidence entry; the
// thread of the row's first entry does the work): the topology row merged
// with the row's new partners.  Each such row also checks the staging
// capacity of the chunk that holds it (the only chunks whose size changed),
// and re-zeroes its new-block count.
// Rows of at most kRegCols topology columns and kRegNew new ones are merged
// in registers: both lists are loaded at once and each column goes to its
// index in its own list plus the number of smaller columns in the other
// (the lists are sorted and disjoint).  Longer rows take the loop.
__global__ void __launch_bounds__(kThreads)
k_ins_merge_rows(DevState *st, int32_t nent, InsertBufs b, const PatchHdr *__restrict__ hdr)
{
    const int32_t k = blockIdx.x * kThreads + threadIdx.x;
    if (k >= nent) return;
    const int bk = back_of(st);
    const int32_t a = b.trow[bk][k];
    if (a < 0) return;
    const PatchHdr h = hdr[b.row_chunk[a]];
    const int32_t rb0 = b.rp[0][a], len = b.rp[0][a + 1] - rb0;
    const int32_t o0 = b.rp[bk][a], nn = (b.rp[bk][a + 1] - o0) - len;
    const int32_t *cb = b.ci[0] + rb0;
    const int32_t *pn = b.pnew[bk] + 3 * int64_t(k);
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
    if (nn > 0) b.nnew[a] = 0;
    if (b.rp[bk][h.v0 + h.nown] - b.rp[bk][h.v0] > h.amap_cap) atomicOr(&st->err_cur, 2);
}

// One 64-thread workgroup (one wave) per row chunk or patch, walking its
// rows 64 at a time.  For each group of rows the wave loads the topology
// columns of the group into LDS with coalesced loads, every lane builds its
// row of the new pattern in a second LDS buffer (a copy, or a merge with the
// row's new partners, which also re-zeroes nnew), and the wave stores the
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
        if (mine && nn > 0) b.nnew[a] = 0;
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
            !b.pnew[k] || !b.trow[k] || (np > 0 && !b.pairs[k]) || (nvf > 0 && !b.vf[k]))
            return hipErrorInvalidValue;
    if (!b.rp[0] || !b.ci[0] || !b.cnt || !b.nnew || !b.tmp || !hdr ||
        (!complete_cols && !b.row_chunk) || (nvf > 0 && (!b.faces || !d_vf)) ||
        (np > 0 && !d_pairs))
        return hipErrorInvalidValue;
    const int64_t nel = int64_t(np) + nvf, nent = 2 * int64_t(np) + 4 * int64_t(nvf);
    hipLaunchKernelGGL(k_ins_count, dim3(blocks_for(nel)), dim3(kThreads), 0, s, st, d_pairs, np,
                       d_vf, nvf, nv, nf, b);
    hipError_t e = launch_scan_back(b.cnt, b.pinc_ptr, nullptr, st, nv, b.tmp, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ins_fill, dim3(blocks_for(nel)), dim3(kThreads), 0, s, st, np, nvf, nv,
                       nf, b);
    hipLaunchKernelGGL(k_ins_rows, dim3(blocks_for(nent)), dim3(kThreads), 0, s, st,
                       int32_t(nent), np, nv, b);
    // new row_ptr = topology row_ptr + prefix of the new blocks per row
    e = launch_scan_back(b.nnew, b.rp, b.rp[0], st, nv, b.tmp, s);
    if (e != hipSuccess) return e;
    if (complete_cols)
        hipLaunchKernelGGL(k_ins_merge, dim3(npatch), dim3(kMergeThreads), 0, s, st, hdr, b, 0);
    else
        hipLaunchKernelGGL(k_ins_merge_rows, dim3(blocks_for(nent)), dim3(kThreads), 0, s, st,
                           int32_t(nent), b, hdr);
    hipLaunchKernelGGL(k_ins_commit, dim3(1), dim3(1), 0, s, st, np, nvf, nv, b);
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
