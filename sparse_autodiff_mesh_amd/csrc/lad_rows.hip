// lad_rows.hip -- row-owner evaluation of two-vertex radial terms (springs,
// runtime vertex-vertex pairs) and vertex terms (inertia) on gfx950.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations":
//   * section "Method": F(x) = sum_j f_j(x_j), g = sum_j S_j^T g_j,
//     H = sum_j S_j^T H_j S_j, and the matrix-free Hessian-vector product;
//   * key design 1: every local term is differentiated in forward mode with
//     all intermediates on chip, and global traffic is one read of the mesh
//     data and one write of the final sparse derivatives;
//   * key design 4: runtime pairs add off-diagonal blocks to the pattern.
//
// Parallel decomposition (differs from the page's one-block-per-patch with
// atomic scatter-add): one lane owns one block row a of H.  It evaluates
// every spring incident to a with second-order dual numbers in registers
// (each spring is thus evaluated once from each end; with the difference
// z = x_a - x_b as seed variables the local Hessian is the same 3x3 block K
// both times, bit for bit), writes the off-diagonal block -K of every slot
// of its row exactly once, and accumulates the diagonal block and g_a in
// registers.  Spring blocks are written once, there are no atomics, and
// every sum is taken in a fixed order: the result is bitwise reproducible.
// A wave's 64 consecutive rows form one contiguous slice of the value array;
// it is staged in LDS and streamed to HBM with 16-byte nontemporal stores.
// Workgroups are persistent: the explicit kernels take row chunks round
// robin in an XCD-grouped numbering, the product kernels contiguous slice
// ranges grouped by XCD, so that vertex positions shared by neighbouring
// rows stay in one L2.
#include "dual2.h"
#include "energies.h"
#include "lad_device.h"
#include "cg_device.h"
#include "lad_internal.h"
#include "lad_jacobian.h"
#include "residuals.h"

namespace lad {

namespace {

constexpr int kBatch = 8;  // slots whose loads a lane issues together
static_assert(kRowThreads == 64, "one wave per workgroup: LDS hand-off needs no barrier");

// LDS hand-off between the lanes of one wave.  A wave's LDS instructions
// execute in issue order, so a read issued after another lane's write sees
// it; the wavefront-scope fences only keep the compiler from moving memory
// operations across this point.  Unlike a workgroup barrier this does not
// wait for outstanding global loads and stores, so a chunk's HBM stores
// drain while the next chunk is being computed.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Position of column b in the sorted active row [lo, hi); the caller knows
// it is present.
__device__ __forceinline__ int32_t find_slot(const int32_t *ci, int32_t lo, int32_t hi, int32_t b)
{
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (ci[mid] < b) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <typename T>
struct Row {
    int32_t a, s0, s1;        // vertex, active slot range
    int32_t kb0, kb1;         // topology slot range
    int32_t f0, f1;           // incident-face range (when the face term is on)
    int32_t p0, p1;           // pair-incidence range (when pairs are active)
    int32_t nn;               // columns the active row has beyond its topology row
    T xa[3];
    T xt[3];                  // inertial target (when the inertia term is on)
};

// Row header loads, all independent of each other.
// With WITH_XT = false the inertial target is not loaded (the HVP needs
// only the inertia term's Hessian, which does not depend on it).
template <typename T, bool WITH_XT = true, bool PINC = true>
__device__ __forceinline__ Row<T> load_row(const RowArgs<T> &A, int act, const int32_t *rpa,
                                           int32_t a, const T *__restrict__ x)
{
    Row<T> r;
    r.p0 = (PINC && act != 0) ? A.pat.pinc_ptr[act][a] : 0;
    r.p1 = (PINC && act != 0) ? A.pat.pinc_ptr[act][a + 1] : 0;
    r.a = a;
    r.s0 = rpa[a];
    r.s1 = rpa[a + 1];
    r.kb0 = A.rp0[a];
    r.kb1 = A.rp0[a + 1];
    r.f0 = A.faces_on ? A.fptr[a] : 0;
    r.f1 = A.faces_on ? A.fptr[a + 1] : 0;
    r.nn = act != 0 ? (r.s1 - r.s0) - (r.kb1 - r.kb0) : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        r.xa[k] = x[int64_t(a) * 3 + k];
        r.xt[k] = (WITH_XT && A.inertia_on) ? A.x_tilde[int64_t(a) * 3 + k] : r.xa[k];
    }
    return r;
}

// Operands of up to kBatch consecutive slots of one row.  kb is the slot's
// index in the topology pattern (-1 past the row end or for a block inserted
// by pairs), b its column, L the rest length of the spring behind the block
// (negative: none) and xb the column vertex's position.
template <typename T>
struct SlotBatch {
    int32_t kb[kBatch], b[kBatch];
    T L[kBatch];
    T xb[kBatch][3];
};

// Load one batch starting at active slot `base`.  Every load uses an index
// that is valid whatever the slot (the row's first topology slot, or the
// row's own vertex), so all loads of the batch are issued back to back and
// only the arithmetic that consumes them is predicated.
//
// Topology pattern active (act == 0), or a row that no current pair
// touches (its active row is its topology row): active slot s is topology
// slot kb0 + (s - s0).  Otherwise the active row is the topology row with
// the pairs' new columns merged in, both sorted, so a slot is inserted
// exactly when its column is not in the topology row.  The batch then loads
// the active columns and a window of kBatch topology columns starting at
// the cursor `jb` (the active slots of the batch can only match topology
// slots in that window) and matches them in registers; `jb` advances past
// the matched slots.
template <typename T>
__device__ __forceinline__ void load_batch(const RowArgs<T> &A, const Row<T> &r, int act,
                                           const int32_t *cia, int32_t base, int32_t &jb,
                                           const T *__restrict__ x, SlotBatch<T> &q)
{
    if (act == 0 || r.p1 == r.p0) {  // uniform in a wave with no pair rows
#pragma unroll
        for (int j = 0; j < kBatch; ++j) q.kb[j] = base + j < r.s1 ? r.kb0 + (base + j - r.s0) : -1;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int32_t kl = q.kb[j] >= 0 ? q.kb[j] : r.kb0;
            q.b[j] = A.ci0[kl];
            q.L[j] = A.springs_on ? A.slot_rest[kl] : T(-1);
        }
    } else {
        int32_t ca[kBatch], cb[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            ca[j] = cia[min(base + j, r.s1 - 1)];
            cb[j] = A.ci0[min(jb + j, r.kb1 - 1)];
        }
        int32_t nmatch = 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            int32_t kb = -1;
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                kb = (jb + k < r.kb1 && cb[k] == ca[j]) ? jb + k : kb;
            q.kb[j] = base + j < r.s1 ? kb : -1;
            q.b[j] = ca[j];
            nmatch += q.kb[j] >= 0 ? 1 : 0;
        }
        jb += nmatch;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            q.L[j] = A.springs_on ? A.slot_rest[q.kb[j] >= 0 ? q.kb[j] : r.kb0] : T(-1);
    }
    // neighbour positions only for the spring term (uniform)
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int32_t bl = (base + j < r.s1) ? q.b[j] : r.a;
#pragma unroll
        for (int c = 0; c < 3; ++c) q.xb[j][c] = A.springs_on ? x[int64_t(bl) * 3 + c] : T(0);
        if (q.kb[j] < 0 || !A.springs_on) q.L[j] = T(-1);
    }
}

// ---------------------------------------------------------------------------
// Runtime pairs of one row.  The first kRowPairs of them (in pair order) are
// loaded before the slot loop, so their chain of dependent loads (pair id ->
// endpoints -> partner position) overlaps the slot loads, and the slot loop
// finds each partner's block by comparing columns in registers.  Further
// pairs of the same row are handled one by one afterwards.
// ---------------------------------------------------------------------------
constexpr int kRowPairs = 2;

template <typename T>
struct PairPre {
    int32_t n;                 // prefetched pairs of this row (<= kRowPairs)
    int32_t b[kRowPairs];      // partner vertex
    int32_t first[kRowPairs];  // 1 if this row is the pair's first vertex
    int32_t slot[kRowPairs];   // partner's block in the active row
    T xb[kRowPairs][3];
};

// Every field is set whatever the row: with no (or fewer) pairs the unused
// entries name the row's own vertex, so loads indexed by pp.b stay in range.
// A row's incidence entries are sorted by element id, pairs (ids < npa)
// before vertex-face contacts, so the prefetched pairs are the leading ones.
template <typename T>
__device__ __forceinline__ void prefetch_pairs(const RowArgs<T> &A, int act, int32_t npa,
                                               const Row<T> &r, const T *__restrict__ x,
                                               PairPre<T> &pp)
{
    pp.n = 0;
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k) {
        pp.b[k] = r.a;
        pp.first[k] = 0;
        pp.slot[k] = r.s0;
#pragma unroll
        for (int c = 0; c < 3; ++c) pp.xb[k][c] = r.xa[c];
    }
    if (act == 0 || r.p1 == r.p0) return;
    const int32_t *pl = A.pat.pinc[act];
    const int32_t *prs = A.pat.pairs[act];
    int32_t q[kRowPairs];
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k) q[k] = pl[min(r.p0 + k, r.p1 - 1)];
    int32_t n = 0;
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k) n += (n == k && k < r.p1 - r.p0 && q[k] < npa) ? 1 : 0;
    pp.n = n;
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k)
        if (k < n) {
            const int32_t i0 = prs[2 * q[k]], i1 = prs[2 * q[k] + 1];
            pp.first[k] = i0 == r.a ? 1 : 0;
            pp.b[k] = i0 == r.a ? i1 : i0;
        }
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k)
#pragma unroll
        for (int c = 0; c < 3; ++c) pp.xb[k][c] = x[int64_t(pp.b[k]) * 3 + c];
}

// ---------------------------------------------------------------------------
// Face terms.  The symmetric-Dirichlet energy is differentiated in its
// natural variables F = [p1 - p0, p2 - p0] M (M = Dm^-1, F stored row-major
// F[2s + c]), a constant linear image of the face's vertex positions:
// dF[s][c] / dp_u[s] = w[u][c] with w1 = M row 0, w2 = M row 1,
// w0 = -(w1 + w2).  The row of the face's vertex at position i then gets
//   g_a[s]        += sum_c w[i][c] dE/dF[s][c]
//   H_(a,u)[s][t] += sum_{c,c'} w[i][c] w[u][c'] d2E/dF[s][c] dF[t][c'].
// The explicit kernel has every row evaluate its own faces (each face
// three times, once per vertex row: the evaluation stays in registers and
// the kernel keeps its occupancy); the product kernel evaluates every face
// of a slice's list once per slice, one face per lane, and keeps its
// per-vertex results in LDS for the rows of the slice to gather (fields of
// one face are kFaceRound apart, so the lanes of a wave touch distinct
// banks).
// ---------------------------------------------------------------------------
constexpr int kFaceHvpFields = 9;   // product kernel: w_u^T (d2E/dF2 dF) for u = 0, 1, 2
constexpr int kRowFaceRegs = 8;     // a row's first faces, held in registers
constexpr int kFaceBatch = 3;       // incident faces whose loads a lane issues together
constexpr int kHalfFaceBatch = 2;   // the same for a lane that shares its row

// Face positions (in face order), Dm^-1 and area of one face.
template <typename T>
struct FaceIn {
    T p[3][3];
    T m[4];
    T area;
};

// One face of a slice's list, loaded by the lane that evaluates it.
template <typename T>
__device__ __forceinline__ void load_face(const RowArgs<T> &A, const SliceFace &sf,
                                          const T *__restrict__ x, FaceIn<T> &q)
{
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int c = 0; c < 3; ++c) q.p[u][c] = x[int64_t(sf.v[u]) * 3 + c];
#pragma unroll
    for (int c = 0; c < 4; ++c) q.m[c] = A.face_dm[int64_t(sf.f) * 4 + c];
    q.area = A.face_area[sf.f];
}

// The incident faces [base, base + kFaceBatch) of row r (explicit kernel),
// with indices clamped into the row's range so that every load is valid:
// each face's record, the positions of its other two vertices, Dm^-1 and
// area, all issued together.
template <typename T, int NB = kFaceBatch>
struct FaceBatch {
    static constexpr int n = NB;
    FaceInc e[NB];
    T xo[NB][2][3];    // positions of o1, o2
    T m[NB][4];        // Dm^-1
    T area[NB];
};

// STRIDE: every STRIDE-th face from base (a row shared by a pair of lanes).
template <typename T, int STRIDE = 1, int NB = kFaceBatch>
__device__ __forceinline__ void load_faces(const RowArgs<T> &A, const Row<T> &r, int32_t base,
                                           const T *__restrict__ x, FaceBatch<T, NB> &q)
{
#pragma unroll
    for (int j = 0; j < NB; ++j) q.e[j] = A.finc[min(base + STRIDE * j, r.f1 - 1)];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            q.xo[j][0][c] = x[int64_t(q.e[j].o1) * 3 + c];
            q.xo[j][1][c] = x[int64_t(q.e[j].o2) * 3 + c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) q.m[j][c] = A.face_dm[int64_t(q.e[j].f) * 4 + c];
        q.area[j] = A.face_area[q.e[j].f];
    }
}

// Face j of a batch in face order: p_i = x_a, p_(i+1)%3 = o1, p_(i+2)%3 = o2.
template <typename T, int NB>
__device__ __forceinline__ void batch_face(const Row<T> &r, const FaceBatch<T, NB> &q, int j, int i,
                                           FaceIn<T> &f)
{
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const T *o1 = q.xo[j][0], *o2 = q.xo[j][1];
        f.p[0][c] = i == 0 ? r.xa[c] : (i == 1 ? o2[c] : o1[c]);
        f.p[1][c] = i == 1 ? r.xa[c] : (i == 2 ? o2[c] : o1[c]);
        f.p[2][c] = i == 2 ? r.xa[c] : (i == 0 ? o2[c] : o1[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) f.m[c] = q.m[j][c];
    f.area = q.area[j];
}

// F = [p1 - p0, p2 - p0] M.
template <typename T>
__device__ __forceinline__ void face_F(const FaceIn<T> &q, T Fv[6])
{
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const T d0 = q.p[1][s] - q.p[0][s], d1 = q.p[2][s] - q.p[0][s];
        Fv[2 * s + 0] = d0 * q.m[0] + d1 * q.m[2];
        Fv[2 * s + 1] = d0 * q.m[1] + d1 * q.m[3];
    }
}

// The weights w[u][c] = dF[.][c] / dp_u from M.
template <typename T>
__device__ __forceinline__ void face_w(const T m[4], T w[3][2])
{
    w[1][0] = m[0];
    w[1][1] = m[1];
    w[2][0] = m[2];
    w[2][1] = m[3];
    w[0][0] = -(m[0] + m[2]);
    w[0][1] = -(m[1] + m[3]);
}

// The row's part of one face from its F-space derivatives gE (6) and the
// packed d2E/dF2 h (21), the row vertex at face position i: the gradient
// into G, the row's own block into D, and the blocks of the face vertices
// at positions (i+1)%3 and (i+2)%3 into B1 and B2.  The row's material
// weights are contracted first,
//   P[s][t][c'] = sum_c w[i][c] d2E/dF[s][c] dF[t][c'],
// then each block is P against the column vertex's weights.  (The weights
// are picked by selects, not by indexing with i, which would put them in
// scratch memory.)
template <typename T>
__device__ __forceinline__ void face_row_blocks(const T gE[6], const T h[21], const T m[4], int i,
                                                T D[9], T G[3], T B1[9], T B2[9])
{
    // w[u][c] from M: w1 = M row 0, w2 = M row 1, w0 = -(w1 + w2)
    auto pick = [&](int u, int c) __attribute__((always_inline)) {
        const T a = m[c], b = m[2 + c];
        return u == 1 ? a : (u == 2 ? b : -(a + b));
    };
    const int i1 = i == 2 ? 0 : i + 1;
    const T wa[2] = {pick(i, 0), pick(i, 1)};
    const T wb[2] = {pick(i1, 0), pick(i1, 1)};
#pragma unroll
    for (int s = 0; s < 3; ++s) G[s] += wa[0] * gE[2 * s] + wa[1] * gE[2 * s + 1];
    auto H = [&](int p, int q) __attribute__((always_inline)) {
        return p <= q ? h[Tri<6>::idx(p, q)] : h[Tri<6>::idx(q, p)];
    };
    T P[3][3][2];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                P[s][t][c] = wa[0] * H(2 * s, 2 * t + c) + wa[1] * H(2 * s + 1, 2 * t + c);
    // the three weights sum to zero, so the three blocks do too
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const T own = P[s][t][0] * wa[0] + P[s][t][1] * wa[1];
            D[3 * s + t] += own;
            B1[3 * s + t] = P[s][t][0] * wb[0] + P[s][t][1] * wb[1];
            B2[3 * s + t] = -(own + B1[3 * s + t]);
        }
}

// The same, with the two blocks handed to blk(position, block).
template <typename T, typename BlockAdd>
__device__ __forceinline__ void face_row(const T gE[6], const T h[21], const T m[4], int i,
                                         T D[9], T G[3], BlockAdd blk)
{
    T B1[9], B2[9];
    face_row_blocks(gE, h, m, i, D, G, B1, B2);
    blk(i == 2 ? 0 : i + 1, B1);
    blk(i == 0 ? 2 : i - 1, B2);
}

// ---------------------------------------------------------------------------
// Energy, gradient and Hessian rows.
// ---------------------------------------------------------------------------

// Inserted columns of a touched row (ascending; INT32_MAX past the count).
// The first is stored per row (rins1, read with the row's header); the
// others, for the few rows that gain more than one column, come from pnew
// at the row's incidence offset.
template <typename T>
__device__ __forceinline__ void load_inserted(const RowArgs<T> &A, int act, const Row<T> &r,
                                              int32_t first, int32_t ins[kMaxIns])
{
    ins[0] = r.nn > 0 ? first : INT32_MAX;
#pragma unroll
    for (int m = 1; m < kMaxIns; ++m) ins[m] = INT32_MAX;
    if (r.nn > 1) {
        const int32_t *pn = A.pat.pnew[act] + 3 * int64_t(A.pat.pinc_ptr[act][r.a]);
#pragma unroll
        for (int m = 1; m < kMaxIns; ++m)
            if (m < r.nn) ins[m] = pn[m];
    }
}

// Inserted columns before column b: topology slot kb0 + i of the row sits at
// active slot s0 + i + shift_of(ins, its column).
__device__ __forceinline__ int32_t shift_of(const int32_t ins[kMaxIns], int32_t b)
{
    int32_t n = 0;
#pragma unroll
    for (int m = 0; m < kMaxIns; ++m) n += ins[m] < b ? 1 : 0;
    return n;
}


// Runtime pair (a, b) seen from row a: -K into block `slot` (a
// read-modify-write), +K into the diagonal D, the gradient into G; the
// energy counted by the pair's first vertex.
template <typename T>
__device__ __forceinline__ void pair_add(const RowArgs<T> &A, const T xa[3], const T xb[3],
                                         T *B, bool first, T D[9], T G[3], double &E)
{
    T dz[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) dz[c] = xa[c] - xb[c];
    const T l2 = dz[0] * dz[0] + dz[1] * dz[1] + dz[2] * dz[2];
    if (!(l2 < A.dhat * A.dhat)) return;  // outside the barrier's support
    Dual2<T, 3> d[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(dz[c], c);
    const Dual2<T, 3> e = barrier_energy(d, A.kappa, A.dhat);
    if (first) E += double(e.v);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        G[i] += e.g[i];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const T h = e.hess(i, j);
            B[3 * i + j] -= h;
            D[3 * i + j] += h;
        }
    }
}

// Vertex-face contact e of the active buffer seen from row a: k_vf_eval
// stored, for each of its four vertices, that row's strip (energy in the
// contact vertex's strip only, the gradient part, 3 Hessian rows over the
// contact's 12 variables) and the four blocks' offsets in that row.  The
// row's own block goes to D; the other three are added into the staged row
// Hrow (block offsets from the row's first slot).
template <typename T>
__device__ __forceinline__ void vf_add(const RowArgs<T> &A, int32_t a, int32_t e, T *Hrow, T D[9],
                                       T G[3], double &E, int li = -1)
{
    if (li < 0) {  // the row's vertex's place in the contact, when not given
        const int4 w = *reinterpret_cast<const int4 *>(A.vf_ids + 4 * int64_t(e));
        li = w.x == a ? 0 : (w.y == a ? 1 : (w.z == a ? 2 : 3));
    }
    const int64_t strip = 4 * int64_t(e) + li;
    const int4 so = *reinterpret_cast<const int4 *>(A.vf_slots + strip * 4);
    const T *L = A.vf_eval + strip * kVfStrip;
    T v[kVfStrip];
#pragma unroll
    for (int k = 0; k < kVfStrip; ++k) v[k] = L[k];
    E += double(v[0]);
#pragma unroll
    for (int c = 0; c < 3; ++c) G[c] += v[1 + c];
    const int32_t off[4] = {so.x, so.y, so.z, so.w};
    // The four blocks are distinct (distinct columns), so every load is
    // issued before any store; block li is the diagonal, kept in D.
    T cur[4][9];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int k = 0; k < 9; ++k) cur[m][k] = Hrow[9 * off[m] + k];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int rr = 0; rr < 3; ++rr)
#pragma unroll
            for (int cc = 0; cc < 3; ++cc) {
                // D is updated unconditionally (a select between D and a
                // block would take D's address and move it to scratch)
                const T h = v[kVfHessOff + 12 * rr + 3 * m + cc];
                D[3 * rr + cc] += m == li ? h : T(0);
                cur[m][3 * rr + cc] += h;
            }
#pragma unroll
    for (int m = 0; m < 4; ++m)
        if (m != li)
#pragma unroll
            for (int k = 0; k < 9; ++k) Hrow[9 * off[m] + k] = cur[m][k];
}

// What a row accumulates in registers: its diagonal block, its gradient,
// its part of the energy, and the active slot of its diagonal block.
template <typename T>
struct RowAcc {
    T D[9];
    T G[3];
    double E;
    int32_t dslot;
};

template <typename T>
__device__ __forceinline__ void acc_init(RowAcc<T> &acc, int32_t s0)
{
#pragma unroll
    for (int i = 0; i < 9; ++i) acc.D[i] = T(0);
#pragma unroll
    for (int i = 0; i < 3; ++i) acc.G[i] = T(0);
    acc.E = 0.0;
    acc.dslot = s0;
}

// The slot loop of one row over the active slots [rt.s0, rt.s1): every
// slot gets its spring's block -K (+K into D), or zeros (no spring behind
// it, or a block inserted by contacts); the diagonal slot is recorded.
// PAIRS: slots found through the active row (column matching), and the
// prefetched pairs' slots recorded in pp.  SHIFT: the topology slots in
// order, each moved past the inserted columns before it.  Each spring's
// energy is counted by its lower-numbered endpoint's row.
template <typename T, bool PAIRS, bool SHIFT>
__device__ __forceinline__ void row_slots(const RowArgs<T> &A, int act, const int32_t *cia,
                                          const Row<T> &r, const Row<T> &rt,
                                          const int32_t ins[kMaxIns], int32_t sb, T *Hs,
                                          const T *__restrict__ x, RowAcc<T> &acc,
                                          PairPre<T> &pp)
{
    int32_t jb = r.kb0;
    for (int32_t base = rt.s0; base < rt.s1; base += kBatch) {
        SlotBatch<T> q;
        load_batch(A, rt, act, cia, base, jb, x, q);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            int32_t s = base + j;
            if (s >= rt.s1) break;
            if constexpr (SHIFT) s += shift_of(ins, q.b[j]);
            if constexpr (PAIRS)
#pragma unroll
                for (int k = 0; k < kRowPairs; ++k) pp.slot[k] = q.b[j] == pp.b[k] ? s : pp.slot[k];
            T *B = Hs + 9 * (s - sb);
            if (q.kb[j] >= 0 && q.b[j] == r.a) {
                acc.dslot = s;
                continue;
            }
            if (!(q.L[j] >= T(0))) {  // inserted by a contact, or no spring behind the block
#pragma unroll
                for (int i = 0; i < 9; ++i) B[i] = T(0);
                continue;
            }
            Dual2<T, 3> d[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(r.xa[c] - q.xb[j][c], c);
            const Dual2<T, 3> e = spring_energy(d, q.L[j], A.k);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                acc.G[i] += e.g[i];
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const T h = e.hess(i, k);
                    B[3 * i + k] = -h;
                    acc.D[3 * i + k] += h;
                }
            }
            if (r.a < q.b[j]) acc.E += double(e.v);
        }
    }
}

// The spring blocks of a row of a chunk that is exactly spring slice t and
// whose rows hold only their diagonal and their springs' blocks (lane
// `lane`, row r.a): spring j (its j-th neighbour in ascending column
// order) comes from the slice with one coalesced load per j for the whole
// wave and sits at slot s0 + j, moved one on past the diagonal when its
// column is above the row; the diagonal's slot follows from the number of
// neighbours below.  SHIFT: every slot also moves past the row's inserted
// columns below it.  The same blocks, in the same order, as row_slots.
constexpr int kDenseBatch = 6;  // springs whose loads a lane issues together

// Neighbour vertices of N spring slice entries e[j] of row a (clamped to
// the last row): from their 16-bit differences when the slices store those,
// else the stored vertex ids.  The test is uniform over the launch and taken
// once for all N loads, which are issued before any of them is used.
template <int N, typename T>
__device__ __forceinline__ void slice_nbs(const RowArgs<T> &A, const int64_t (&e)[N], int32_t a,
                                          int32_t (&nb)[N])
{
    int32_t raw[N];
    const bool d16 = A.sl_d16 != nullptr;
    if (d16) {
#pragma unroll
        for (int j = 0; j < N; ++j) raw[j] = A.sl_d16[e[j]];
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) raw[j] = A.sl_nb[e[j]];
    }
#pragma unroll
    for (int j = 0; j < N; ++j) nb[j] = d16 ? a + raw[j] : raw[j];
}

template <typename T, bool SHIFT>
__device__ __forceinline__ void row_slice_springs(const RowArgs<T> &A, int32_t t, int lane,
                                                  const Row<T> &r, const int32_t ins[kMaxIns],
                                                  int32_t sb, T *Hs, const T *__restrict__ x,
                                                  RowAcc<T> &acc)
{
    const int32_t p = A.sl_ptr[t];
    const int32_t ns = (A.sl_ptr[t + 1] - p) / kSliceRows;  // wave-uniform
    int32_t below = 0;
    int32_t ins_below[kMaxIns] = {};  // SHIFT: topology columns below each inserted one
    for (int32_t j0 = 0; j0 < ns; j0 += kDenseBatch) {
        int32_t nb[kDenseBatch];
        T L[kDenseBatch], xb[kDenseBatch][3];
        int64_t e[kDenseBatch];
#pragma unroll
        for (int j = 0; j < kDenseBatch; ++j)
            e[j] = p + int64_t(min(j0 + j, ns - 1)) * kSliceRows + lane;
        slice_nbs(A, e, r.a, nb);
#pragma unroll
        for (int j = 0; j < kDenseBatch; ++j) L[j] = j0 + j < ns ? A.sl_rest[e[j]] : T(-1);
#pragma unroll
        for (int j = 0; j < kDenseBatch; ++j)
#pragma unroll
            for (int c = 0; c < 3; ++c) xb[j][c] = x[int64_t(nb[j]) * 3 + c];
#pragma unroll
        for (int j = 0; j < kDenseBatch; ++j) {
            if (!(L[j] >= T(0))) continue;  // padding: the row has fewer springs
            const bool above = nb[j] > r.a;
            below += above ? 0 : 1;
            int32_t sl = r.s0 + j0 + j + (above ? 1 : 0);
            if constexpr (SHIFT) {
                sl += shift_of(ins, nb[j]);
#pragma unroll
                for (int m = 0; m < kMaxIns; ++m) ins_below[m] += nb[j] < ins[m] ? 1 : 0;
            }
            T *B = Hs + 9 * (sl - sb);
            Dual2<T, 3> d[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(r.xa[c] - xb[j][c], c);
            const Dual2<T, 3> e = spring_energy(d, L[j], A.k);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                acc.G[i] += e.g[i];
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const T h = e.hess(i, k);
                    B[3 * i + k] = -h;
                    acc.D[3 * i + k] += h;
                }
            }
            if (above) acc.E += double(e.v);
        }
    }
    acc.dslot = r.s0 + below;
    if constexpr (SHIFT) {
        acc.dslot += shift_of(ins, r.a);
        // the inserted columns' blocks get contact terms only (added by
        // k_eval_pair_rows): zero them.  An inserted column follows the
        // inserted columns and the topology columns (the diagonal, the
        // springs) below it.
#pragma unroll
        for (int m = 0; m < kMaxIns; ++m)
            if (ins[m] != INT32_MAX) {
                const int32_t sl = r.s0 + shift_of(ins, ins[m]) + ins_below[m] + (r.a < ins[m] ? 1 : 0);
                T *B = Hs + 9 * (sl - sb);
#pragma unroll
                for (int i = 0; i < 9; ++i) B[i] = T(0);
            }
    }
}

template <typename T>
__device__ __forceinline__ void row_inertia(const RowArgs<T> &A, const Row<T> &r, RowAcc<T> &acc)
{
    if (!A.inertia_on) return;
    Dual2<T, 3> z[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) z[c] = Dual2<T, 3>::var(r.xa[c] - r.xt[c], c);
    const Dual2<T, 3> e = inertia_energy(z, A.c);
    acc.E += double(e.v);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        acc.G[i] += e.g[i];
#pragma unroll
        for (int j = 0; j < 3; ++j) acc.D[3 * i + j] += e.hess(i, j);
    }
}

// The diagonal block into its slot, the gradient into g.
template <typename T>
__device__ __forceinline__ void row_store(const Row<T> &r, int32_t sb, T *Hs, T *__restrict__ g,
                                          const RowAcc<T> &acc)
{
    T *B = Hs + 9 * (acc.dslot - sb);
#pragma unroll
    for (int i = 0; i < 9; ++i) B[i] = acc.D[i];
#pragma unroll
    for (int c = 0; c < 3; ++c) g[int64_t(r.a) * 3 + c] = acc.G[c];
}

// The faces of one row, evaluated by the row itself in face-id order,
// kFaceBatch at a time with all their loads issued together: the gradient
// part and the diagonal block into acc, the blocks of the face's other two
// vertices added into the staged row (block s - sb holds active slot s).
// Block placement: the topology pattern active (act == 0) or a row no
// contact touches, at the topology offset (SHIFT: moved past the inserted
// columns before it); else at the column's position in the active row.
// The energy of a face is counted by the row of its first vertex.
template <typename T, bool SHIFT>
__device__ __forceinline__ void row_faces(const RowArgs<T> &A, int act, const int32_t *cia,
                                          const Row<T> &r, const int32_t ins[kMaxIns], int32_t sb,
                                          T *Hs, const T *__restrict__ x, RowAcc<T> &acc)
{
    for (int32_t base = r.f0; base < r.f1; base += kFaceBatch) {
        FaceBatch<T> q;
        load_faces(A, r, base, x, q);
#pragma unroll
        for (int j = 0; j < kFaceBatch; ++j) {
            if (base + j >= r.f1) break;
            const FaceInc fe = q.e[j];
            const int i = int(fe.pk & 3u);
            FaceIn<T> f;
            batch_face(r, q, j, i, f);
            T Fv[6];
            face_F(f, Fv);
            Dual2<T, 6> F[6];
#pragma unroll
            for (int c = 0; c < 6; ++c) F[c] = Dual2<T, 6>::var(Fv[c], c);
            const Dual2<T, 6> en = face_energy(F, f.area);
            if (i == 0) acc.E += double(en.v);
            face_row(en.g, en.h, f.m, i, acc.D, acc.G,
                     [&](int u, const T B[9]) __attribute__((always_inline)) {
                         // u is the face position (i+1)%3 or (i+2)%3: o1 or o2
                         const int32_t vu = u == (i == 2 ? 0 : i + 1) ? fe.o1 : fe.o2;
                         int32_t sl;
                         if (act == 0 || r.p1 == r.p0) {
                             const int32_t off = int32_t((fe.pk >> (8 * u + 8)) & 255u);
                             sl = r.s0 + off;
                             if constexpr (SHIFT) sl += shift_of(ins, vu);
                         } else {
                             sl = find_slot(cia, r.s0, r.s1, vu);
                         }
                         T *Bp = Hs + 9 * (sl - sb);
#pragma unroll
                         for (int k2 = 0; k2 < 9; ++k2) Bp[k2] += B[k2];
                     });
        }
    }
}

// The full evaluation of a row whose active row differs from its topology
// row by more than kMaxIns columns (k_eval_pair_rows): column matching,
// topology terms, its faces, inertia, then its
// pairs and vertex-face contacts in element order; every block written
// into Hs (block s - sb holds active slot s), g_a into g.
template <typename T, bool FACES>
__device__ __forceinline__ double eval_row_full(const RowArgs<T> &A, int act, const int32_t *cia,
                                                const Row<T> &r, int32_t sb, T *Hs,
                                                const T *__restrict__ x, T *__restrict__ g)
{
    RowAcc<T> acc;
    acc_init(acc, r.s0);
    int32_t ins[kMaxIns];
#pragma unroll
    for (int m = 0; m < kMaxIns; ++m) ins[m] = INT32_MAX;
    const int32_t npa = act != 0 ? A.state->np[act] : 0;
    PairPre<T> pp;
    prefetch_pairs(A, act, npa, r, x, pp);
    row_slots<T, true, false>(A, act, cia, r, r, ins, sb, Hs, x, acc, pp);
    if constexpr (FACES) row_faces<T, false>(A, act, cia, r, ins, sb, Hs, x, acc);
    row_inertia(A, r, acc);
    // runtime pairs of this row, in pair order: -K into the (a, b) block,
    // +K into the diagonal; then further pairs and contacts
#pragma unroll
    for (int k = 0; k < kRowPairs; ++k)
        if (k < pp.n)
            pair_add(A, r.xa, pp.xb[k], Hs + 9 * (pp.slot[k] - sb), pp.first[k] != 0, acc.D, acc.G,
                     acc.E);
    if (r.p1 - r.p0 > pp.n) {
        const int32_t *pl = A.pat.pinc[act];
        const int32_t *prs = A.pat.pairs[act];
        for (int32_t k = r.p0 + pp.n; k < r.p1; ++k) {
            const int32_t q = pl[k];
            if (q >= npa) {
                vf_add(A, r.a, q - npa, Hs + 9 * (r.s0 - sb), acc.D, acc.G, acc.E);
                continue;
            }
            const int32_t i0 = prs[2 * q], i1 = prs[2 * q + 1];
            const int32_t b = i0 == r.a ? i1 : i0;
            T xb[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) xb[c] = x[int64_t(b) * 3 + c];
            pair_add(A, r.xa, xb, Hs + 9 * (find_slot(cia, r.s0, r.s1, b) - sb), i0 == r.a, acc.D,
                     acc.G, acc.E);
        }
    }
    row_store(r, sb, Hs, g, acc);
    return acc.E;
}

// The contact terms of touched row a (incidence entries k0 .. k1; pi0 the
// first entry's slots) whose topology terms the main kernel evaluated
// (SHIFT mode): pairs and vertex-face contacts in element order, added into
// the row's blocks, its diagonal block and its gradient in HBM.  The
// insertion stored each entry's block slots, partner and orientation; the
// main kernel zeroed the row's inserted blocks.  The first entry's loads
// all go out at once.
template <typename T>
__device__ __forceinline__ double eval_row_contacts(const RowArgs<T> &A, int act, int32_t a,
                                                    int32_t k0, const int4 &pi0, int32_t q0,
                                                    const T *__restrict__ x, T *__restrict__ hv,
                                                    T *__restrict__ g)
{
    const int32_t npa = A.state->np[act];
    const int32_t k1 = A.pat.pinc_ptr[act][a + 1];
    T xa[3], D[9], G[3];
    T *Bd = hv + 9 * int64_t(pi0.y);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        xa[c] = x[int64_t(a) * 3 + c];
        G[c] = g[int64_t(a) * 3 + c];
    }
#pragma unroll
    for (int i = 0; i < 9; ++i) D[i] = Bd[i];
    double E = 0.0;
    for (int32_t k = k0; k < k1; ++k) {
        const int4 pi = k == k0 ? pi0 : A.pat.pslot[act][k];
        if (pi.z < 0) {  // vertex-face contact
            const int32_t q = k == k0 ? q0 : A.pat.pinc[act][k];
            vf_add(A, a, q - npa, hv + 9 * int64_t(pi.w), D, G, E, pi.z <= -2 ? -2 - pi.z : -1);
            continue;
        }
        const int32_t b = pi.z >> 1;
        T xb[3];
#pragma unroll
        for (int c = 0; c < 3; ++c) xb[c] = x[int64_t(b) * 3 + c];
        pair_add(A, xa, xb, hv + 9 * int64_t(pi.x), (pi.z & 1) != 0, D, G, E);
    }
#pragma unroll
    for (int i = 0; i < 9; ++i) Bd[i] = D[i];
#pragma unroll
    for (int c = 0; c < 3; ++c) g[int64_t(a) * 3 + c] = G[c];
    return E;
}

template <typename T, bool FACES, bool PAIRS>
__global__ void __launch_bounds__(kRowThreads)
k_eval_rows(RowArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
            EnergySink esink)
{
    extern __shared__ __align__(16) unsigned char smem[];
    T *stage = reinterpret_cast<T *>(smem);
    // without pair capacity the topology pattern is always the active one
    const int act = PAIRS ? A.state->active : 0;
    const int32_t *rpa = A.pat.rp[act];
    const int32_t *cia = A.pat.ci[act];
    double eacc = 0.0;
    for (int c = first_chunk(); c < A.nchunk; c += int(gridDim.x)) {  // round robin
        const int32_t v0 = A.chunk[c].v0, nrows = A.chunk[c].nown;
        const int32_t dense_t = A.chunk[c].spr_off;  // its spring slice, or -1
        const int32_t sb = rpa[v0];
        const int32_t nblk = rpa[v0 + nrows] - sb;
        // The insertion check keeps every chunk within the staging capacity;
        // a chunk that does not fit is never written.
        const bool fits = nblk <= A.lds_blocks;
        const int pad = stage_pad<T>(int64_t(sb) * 9);
        T *Hs = stage + pad;
        // Every row's topology terms, through the topology pattern (act =
        // 0, no pair code); with contact capacity each block is moved to its
        // active slot and the contact terms of touched rows follow in
        // k_eval_pair_rows.  A row with more than kMaxIns inserted columns
        // is left to that kernel whole (its slice of the staging area is
        // streamed out unwritten and overwritten there).
        Row<T> r{};
        bool own = false;
        int32_t first_ins = INT32_MAX;
        if (fits && int(threadIdx.x) < nrows) {
            r = load_row<T, true, false>(A, act, rpa, v0 + int32_t(threadIdx.x), x);
            if constexpr (PAIRS)
                if (act != 0) first_ins = A.pat.rins1[act][r.a];
            own = !PAIRS || r.nn <= kMaxIns;
        }
        RowAcc<T> acc;
        acc_init(acc, r.s0);
        int32_t ins[kMaxIns];
#pragma unroll
        for (int m = 0; m < kMaxIns; ++m) ins[m] = INT32_MAX;
        if (own) {
            Row<T> rt = r;  // the row as the slot loop walks it
            if constexpr (PAIRS) {
                load_inserted(A, act, r, first_ins, ins);
                rt.s1 = r.s0 + (r.kb1 - r.kb0);  // topology slots, in order
                rt.p0 = rt.p1 = 0;
                // the blocks of inserted columns get contact terms only
                // (k_eval_pair_rows adds them): zero the row first (the
                // spring-slice path zeroes just those blocks itself)
                if (r.nn > 0 && !(A.springs_on && dense_t >= 0))
                    for (int32_t i = 9 * (r.s0 - sb); i < 9 * (r.s1 - sb); ++i) Hs[i] = T(0);
            }
            PairPre<T> pp;
            prefetch_pairs(A, 0, 0, r, x, pp);
            if (A.springs_on && dense_t >= 0)  // wave-uniform
                row_slice_springs<T, PAIRS>(A, dense_t, int(threadIdx.x), r, ins, sb, Hs, x, acc);
            else
                row_slots<T, false, PAIRS>(A, 0, cia, r, rt, ins, sb, Hs, x, acc, pp);
            if constexpr (FACES) row_faces<T, PAIRS>(A, 0, cia, r, ins, sb, Hs, x, acc);
        }
        if (own) {
            row_inertia(A, r, acc);
            row_store(r, sb, Hs, g, acc);
            eacc += acc.E;
        }
        wave_lds_sync();
        if (fits) stream_out<kRowThreads>(hv + int64_t(sb) * 9, Hs, nblk * 9, pad);
        wave_lds_sync();
    }
    store_energy(esink, block_sum<kRowThreads>(eacc, nullptr));
}

// The faces of row r taken by one lane of the pair that shares the row
// (k_eval_face_rows): faces f0 + half, f0 + half + 2, ... in face-id order,
// kFaceBatch at a time with all their loads issued together; the gradient
// part and the diagonal block into acc.  The pair's two lanes add into the
// same staged blocks (a neighbour's block gets a term from each face on
// their shared edge), so every face step adds in two phases, first the
// lanes of even half, then those of odd half, with a wave-level LDS
// hand-off between them: no block is ever read and written by both lanes
// of a pair in one instruction, and every block sums its terms in a fixed
// order.  Topology pattern only.
template <typename T>
__device__ __forceinline__ void row_faces_half(const RowArgs<T> &A, const Row<T> &r, int half,
                                               int32_t sb, T *Hs, const T *__restrict__ x,
                                               RowAcc<T> &acc)
{
    for (int32_t base = r.f0 + half; base < r.f1; base += 2 * kHalfFaceBatch) {
        FaceBatch<T, kHalfFaceBatch> q;
        load_faces<T, 2, kHalfFaceBatch>(A, r, base, x, q);
#pragma unroll
        for (int j = 0; j < kHalfFaceBatch; ++j) {
            if (base + 2 * j >= r.f1) break;
            const FaceInc fe = q.e[j];
            const int i = int(fe.pk & 3u);
            // the row's own block (every face of the row names it)
            acc.dslot = r.s0 + int32_t((fe.pk >> (8 * i + 8)) & 255u);
            FaceIn<T> f;
            batch_face(r, q, j, i, f);
            T Fv[6];
            face_F(f, Fv);
            Dual2<T, 6> F[6];
#pragma unroll
            for (int c = 0; c < 6; ++c) F[c] = Dual2<T, 6>::var(Fv[c], c);
            const Dual2<T, 6> en = face_energy(F, f.area);
            if (i == 0) acc.E += double(en.v);
            T B1[9], B2[9];
            face_row_blocks(en.g, en.h, f.m, i, acc.D, acc.G, B1, B2);
            // B1 belongs to the vertex at face position (i+1)%3, which is
            // o1; B2 to o2 (batch_face's order)
            const int u1 = i == 2 ? 0 : i + 1, u2 = i == 0 ? 2 : i - 1;
            T *P1 = Hs + 9 * (r.s0 + int32_t((fe.pk >> (8 * u1 + 8)) & 255u) - sb);
            T *P2 = Hs + 9 * (r.s0 + int32_t((fe.pk >> (8 * u2 + 8)) & 255u) - sb);
            if (half == 0) {
#pragma unroll
                for (int k = 0; k < 9; ++k) P1[k] += B1[k];
#pragma unroll
                for (int k = 0; k < 9; ++k) P2[k] += B2[k];
            }
            wave_lds_sync();
            if (half == 1) {
#pragma unroll
                for (int k = 0; k < 9; ++k) P1[k] += B1[k];
#pragma unroll
                for (int k = 0; k < 9; ++k) P2[k] += B2[k];
            }
            wave_lds_sync();
        }
    }
}

// Explicit evaluation with the face term and no contact capacity.  The face
// work (about 540 VALU instructions per face and row) makes this kernel
// VALU-bound, and a wave's 64-row staging slice would hold it to two
// resident waves per SIMD, too few to hide its loads.  So each row is shared
// by a pair of lanes (lanes 2l and 2l + 1 own row l of 32), each taking
// every other face of the row; a wave walks its 64-row chunk as two halves
// of 32 rows and stages one half at a time (A.lds_blocks, set on the host
// to the largest half's block count), which leaves registers, not LDS, to
// limit the resident waves.  With springs, the lane of even half runs the
// row's slot loop (spring blocks, zero blocks) first; without, the wave
// zeroes the staged half chunk.  The pair's diagonal and gradient parts are
// summed across the two lanes before the lane of even half stores them.  The results
// are bitwise reproducible, as every sum keeps a fixed order.
template <typename T>
__global__ void __launch_bounds__(kRowThreads)
k_eval_face_rows(RowArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
                 EnergySink esink)
{
    constexpr int kHalfRows = kRowThreads / 2;
    extern __shared__ __align__(16) unsigned char smem[];
    T *stage = reinterpret_cast<T *>(smem);
    const int32_t *rpa = A.pat.rp[0];
    const int32_t *cia = A.pat.ci[0];
    const int half = int(threadIdx.x) & 1;
    const int rl = int(threadIdx.x) >> 1;  // the lane pair's row in the half chunk
    double eacc = 0.0;
    for (int c = first_chunk(); c < A.nchunk; c += int(gridDim.x)) {  // round robin
        const int32_t cv0 = A.chunk[c].v0, cn = A.chunk[c].nown;
        const int32_t dense_t = A.chunk[c].spr_off;  // its spring slice, or -1
        for (int32_t h0 = 0; h0 < cn; h0 += kHalfRows) {
            const int32_t v0 = cv0 + h0, nrows = min(kHalfRows, cn - h0);
            const int32_t sb = rpa[v0];
            const int32_t nblk = rpa[v0 + nrows] - sb;
            // the host sizes the staging area for the largest half chunk
            const bool fits = nblk <= A.lds_blocks;
            const int pad = stage_pad<T>(int64_t(sb) * 9);
            T *Hs = stage + pad;
            const bool own = fits && rl < nrows;
            Row<T> r{};
            if (own) r = load_row<T, true, false>(A, 0, rpa, v0 + rl, x);
            RowAcc<T> acc;
            acc_init(acc, r.s0);
            if (!A.springs_on) {  // uniform
                // a row's blocks are then its diagonal (slot s0 for a row
                // without faces; else named by each face record) and its
                // face neighbours', which the faces add into: zero the half
                // chunk's staging with the whole wave
                if (fits) zero_lds<kRowThreads>(stage, pad + 9 * nblk);
            } else if (own && half == 0) {
                const int32_t ins[kMaxIns] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX};
                static_assert(kMaxIns == 4, "ins initialiser");
                PairPre<T> pp;
                prefetch_pairs(A, 0, 0, r, x, pp);
                if (dense_t >= 0)  // wave-uniform
                    row_slice_springs<T, false>(A, dense_t, h0 + rl, r, ins, sb, Hs, x, acc);
                else
                    row_slots<T, false, false>(A, 0, cia, r, r, ins, sb, Hs, x, acc, pp);
            }
            wave_lds_sync();  // every block is written before the faces add into it
            if (own) row_faces_half(A, r, half, sb, Hs, x, acc);
            // the pair's parts of the diagonal block and the gradient (the
            // same sum in both lanes: addition is commutative)
#pragma unroll
            for (int i = 0; i < 9; ++i) acc.D[i] += __shfl_xor(acc.D[i], 1);
#pragma unroll
            for (int i = 0; i < 3; ++i) acc.G[i] += __shfl_xor(acc.G[i], 1);
            if (own && half == 0) {
                row_inertia(A, r, acc);
                row_store(r, sb, Hs, g, acc);
            }
            if (own) eacc += acc.E;
            wave_lds_sync();
            if (fits) stream_out<kRowThreads>(hv + int64_t(sb) * 9, Hs, nblk * 9, pad);
            wave_lds_sync();
        }
    }
    store_energy(esink, block_sum<kRowThreads>(eacc, nullptr));
}

// Rows that current contacts touch: one thread per row (the thread of the
// row's first incidence entry, a fixed choice, so the energy sums keep their
// order).  It runs after k_eval_rows on the same stream, which evaluated the
// topology terms of every row with at most kMaxIns inserted columns; for
// those the thread adds the row's contact terms (pairs, vertex-face
// contacts) into its blocks, diagonal and gradient in HBM.  A row with more
// inserted columns gets the full row evaluation here -- column matching,
// topology and contact terms -- written straight to HBM.  Only a few
// percent of the rows are touched, but nearly every 64-row wave holds one,
// so handling them apart keeps the divergent contact code out of the main
// kernel.  Every workgroup stores a partial energy (zero when the topology
// pattern is active).
template <typename T, bool FACES>
__global__ void __launch_bounds__(kThreads)
k_eval_pair_rows(RowArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
                 EnergySink esink)
{
    __shared__ double red[kThreads / 64];
    const int act = A.state->active;
    const int32_t k = int32_t(blockIdx.x) * kThreads + int32_t(threadIdx.x);
    double e = 0.0;
    if (act != 0 && k < A.pat.pinc_ptr[act][A.nv]) {
        const int32_t a = A.pat.trow[act][k];
        const int4 pi = A.pat.pslot[act][k];
        const int32_t q = A.pat.pinc[act][k];
        if (a >= 0) {
            if (pi.w >= 0) {
                e = eval_row_contacts(A, act, a, k, pi, q, x, hv, g);
            } else {  // more than kMaxIns new columns: the whole row here
                const Row<T> r = load_row(A, act, A.pat.rp[act], a, x);
                e = eval_row_full<T, FACES>(A, act, A.pat.ci[act], r, 0, hv, x, g);
            }
        }
    }
    store_energy(esink, block_sum<kThreads>(e, red));
}

// ---------------------------------------------------------------------------
// Matrix-free Hessian-vector product, y_a = sum over the row's terms of
// H_ab v_b, with the local Hessians formed in registers and never stored.
// ---------------------------------------------------------------------------
// Component of the Newton-CG direction -r + beta d_prev.
__device__ __forceinline__ float cg_dir_comp(float r, float d, float beta)
{
    return __builtin_fmaf(beta, d, -r);
}
__device__ __forceinline__ double cg_dir_comp(double r, double d, double beta)
{
    return __builtin_fma(beta, d, -r);
}

// Spring neighbours a lane loads together in the product kernels.
constexpr int kSliceBatch = 6;

// What a lane of the product kernels loads for its row before the gathers:
// the row (kSliceRows * t + lane, or the slice's listed row; the last row
// for lanes past the rows, which store nothing), its position, its operand (v, or r and the previous direction for
// Newton-CG), its first kSliceBatch spring neighbours with their rest
// lengths (without the face term only) or its face range.  Every load
// depends only on the slice index, so the next slice's are issued while
// the current slice is processed.
template <typename T>
struct SliceRow {
    int32_t a;
    int32_t live;
    T xa[3], o0[3], o1[3];
    int32_t nb[kSliceBatch];
    T L[kSliceBatch];
    int32_t f0, f1;
};

// Issue the loads of slice t's head for lane `lane` (every index in bounds:
// rows past the last are clamped to it, padding names a valid vertex).
template <typename T, bool FACES, bool CG>
__device__ __forceinline__ void slice_head(const RowArgs<T> &A, int32_t t, int lane,
                                           const T *__restrict__ x, const T *__restrict__ v,
                                           const CgDir<T> &cg, SliceRow<T> &h)
{
    int32_t a;
    if (A.sl_rows) {  // patches of the mesh (face term on)
        const int32_t r = A.sl_rows[int64_t(t) * kSliceRows + lane];
        h.live = r >= 0 ? 1 : 0;
        a = r >= 0 ? r : A.nv - 1;
    } else {
        h.live = t * kSliceRows + lane < A.nv ? 1 : 0;
        a = min(t * kSliceRows + lane, A.nv - 1);
    }
    h.a = a;
    const int32_t p = A.sl_ptr[t];
    const int32_t ns = A.springs_on ? (A.sl_ptr[t + 1] - p) / kSliceRows : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        h.xa[k] = x[int64_t(a) * 3 + k];
        if constexpr (CG) {
            h.o0[k] = cg.r[int64_t(a) * 3 + k];
            h.o1[k] = cg.d_old[int64_t(a) * 3 + k];
        } else {
            h.o0[k] = v[int64_t(a) * 3 + k];
        }
    }
#pragma unroll
    for (int j = 0; j < kSliceBatch; ++j) {
        h.nb[j] = a;
        h.L[j] = T(-1);
    }
    if (!FACES && ns > 0) {  // wave-uniform; with faces the registers go to them
        // entries past the widest row's springs re-read its last one and
        // are dropped
        int64_t e[kSliceBatch];
        int32_t nb[kSliceBatch];
#pragma unroll
        for (int j = 0; j < kSliceBatch; ++j) e[j] = p + int64_t(min(j, ns - 1)) * kSliceRows + lane;
        slice_nbs(A, e, a, nb);
#pragma unroll
        for (int j = 0; j < kSliceBatch; ++j) {
            const T L = A.sl_rest[e[j]];
            if (j < ns) {
                h.nb[j] = nb[j];
                h.L[j] = L;
            }
        }
    }
    h.f0 = FACES ? A.fptr[a] : 0;
    h.f1 = FACES ? A.fptr[a + 1] : 0;
}

// Spring neighbours j0 .. j0 + kSliceBatch - 1 of the lane's row (slice
// entries starting at p; ns springs in the slice's widest row): the first
// batch from the prefetched head, later ones loaded here.
template <typename T, bool FACES>
__device__ __forceinline__ void slice_batch(const RowArgs<T> &A, const SliceRow<T> &h, int32_t p,
                                            int32_t ns, int32_t j0, int lane, int32_t self,
                                            int32_t nb[kSliceBatch], T L[kSliceBatch])
{
    if (!FACES && j0 == 0) {
#pragma unroll
        for (int j = 0; j < kSliceBatch; ++j) {
            nb[j] = h.nb[j];
            L[j] = h.L[j];
        }
        return;
    }
    // j0 < ns: entries past the widest row's springs re-read its last one
    // and are dropped
    int64_t e[kSliceBatch];
    int32_t nbv[kSliceBatch];
#pragma unroll
    for (int j = 0; j < kSliceBatch; ++j) e[j] = p + int64_t(min(j0 + j, ns - 1)) * kSliceRows + lane;
    slice_nbs(A, e, self, nbv);
#pragma unroll
    for (int j = 0; j < kSliceBatch; ++j) {
        const T Lj = A.sl_rest[e[j]];
        const bool in = j0 + j < ns;
        nb[j] = in ? nbv[j] : self;
        L[j] = in ? Lj : T(-1);
    }
}

// This workgroup's slices [t0, t1) (contiguous ranges grouped by XCD) and
// its wave's first slice; the waves walk the range kSliceWaves slices
// apart.
constexpr int32_t kSliceWaves = kHvpThreads / kSliceRows;
__device__ __forceinline__ void slice_range(int32_t nv, int32_t &t0, int32_t &t1, int32_t &first)
{
    const int32_t wv = __builtin_amdgcn_readfirstlane(int32_t(threadIdx.x) / kSliceRows);
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int32_t nsl = (nv + kSliceRows - 1) / kSliceRows;
    t0 = int32_t(int64_t(nsl) * w / gridDim.x);
    t1 = int32_t(int64_t(nsl) * (w + 1) / gridDim.x);
    first = t0 + wv;
}

// The face terms of one slice (product kernel), all lanes of the wave
// together: in rounds of kFaceRound listed faces, every lane evaluates one
// face in numbers that carry the value, the gradient and the Hessian's
// action on the face's direction dF = (dF/dp) u_face, and stores, for each
// face vertex u, w_u^T (d2E/dF2 dF) in this wave's LDS records; every row
// then adds the part of its position in the round's faces it belongs to,
// in list order.  dir(i) gives component i of the direction.
template <typename T, typename Dir>
__device__ __forceinline__ void slice_faces(const RowArgs<T> &A, int32_t t, const SliceRow<T> &h,
                                            T *rec, const T *__restrict__ x, Dir dir, T Y[3])
{
    const int lane = int(threadIdx.x) & (kSliceRows - 1);
    const int32_t cf0 = A.sf_ptr[t], ncf = A.sf_ptr[t + 1] - cf0;
    if (ncf == 0) return;  // wave-uniform: no faces in this slice
    const int32_t nrf = h.live ? h.f1 - h.f0 : 0;
    RowFace rf[kRowFaceRegs];
#pragma unroll
    for (int j = 0; j < kRowFaceRegs; ++j) rf[j] = A.rfinc[nrf > 0 ? h.f0 + min(j, nrf - 1) : 0];
    auto gather = [&](const RowFace e, int32_t base) __attribute__((always_inline)) {
        const int kk = int(e.lf) - base;
        const int i = int(e.pi & 3u);
#pragma unroll
        for (int s = 0; s < 3; ++s) Y[s] += rec[(3 * i + s) * kFaceRound + kk];
    };
    // face inputs and the direction at its vertices, the next round's
    // loaded while this round is evaluated (lanes past the list take its
    // last face and store nothing)
    struct In {
        FaceIn<T> q;
        T du[3][3];
    };
    auto load_in = [&](const SliceFace &cf, In &in) __attribute__((always_inline)) {
        load_face(A, cf, x, in.q);
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int c = 0; c < 3; ++c) in.du[u][c] = dir(int64_t(cf.v[u]) * 3 + c);
    };
    auto face_at = [&](int32_t k) __attribute__((always_inline)) {
        return A.sface[cf0 + min(k, ncf - 1)];
    };
    In cur;
    load_in(face_at(lane), cur);
    SliceFace cfn = face_at(kFaceRound + lane);
    for (int32_t base = 0; base < ncf; base += kFaceRound) {  // wave-uniform
        In nxt;
        if (base + kFaceRound < ncf) load_in(cfn, nxt);  // wave-uniform
        const SliceFace cfn2 = face_at(base + 2 * kFaceRound + lane);
        T Fv[6], w[3][2];
        face_F(cur.q, Fv);
        face_w(cur.q.m, w);
        DualHv<T, 6> F[6];
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                F[2 * sp + c] = DualHv<T, 6>::var(
                    Fv[2 * sp + c], 2 * sp + c,
                    w[0][c] * cur.du[0][sp] + w[1][c] * cur.du[1][sp] + w[2][c] * cur.du[2][sp]);
        const DualHv<T, 6> en = face_energy(F, cur.q.area);
        if (base + lane < ncf)
#pragma unroll
            for (int u = 0; u < 3; ++u)
#pragma unroll
                for (int sp = 0; sp < 3; ++sp)
                    rec[(3 * u + sp) * kFaceRound + lane] =
                        w[u][0] * en.gt[2 * sp] + w[u][1] * en.gt[2 * sp + 1];
        wave_lds_sync();
        // this round's faces of the row: each register copy checked in turn
        const uint32_t lo = uint32_t(base), hi = uint32_t(base + kFaceRound);
#pragma unroll
        for (int j = 0; j < kRowFaceRegs; ++j)
            if (j < nrf && rf[j].lf >= lo && rf[j].lf < hi) gather(rf[j], base);
        for (int32_t kk = h.f0 + kRowFaceRegs; kk < h.f0 + nrf; ++kk) {  // long rows only
            const RowFace e = A.rfinc[kk];
            if (e.lf >= lo && e.lf < hi) gather(e, base);
        }
        wave_lds_sync();
        cur = nxt;
        cfn = cfn2;
    }
}

// Every row's topology terms (springs, faces, inertia); the runtime
// contacts of the rows they touch are added afterwards by k_hvp_pair_rows.
template <typename T, bool FACES, bool CG>
__global__ void __launch_bounds__(kHvpThreads)
k_hvp_rows(RowArgs<T> A, const T *__restrict__ x, const T *__restrict__ v, T *__restrict__ y,
           CgDir<T> cg)
{
    __shared__ double red[kHvpThreads / 64];
    __shared__ double sum_bc;
    __shared__ int32_t stop_bc;
    // per wave: one round of face records (face term only)
    __shared__ T frec[FACES ? kSliceWaves * kFaceHvpFields * kFaceRound : 1];
    double beta = 0.0;
    T beta_t = T(0);  // beta in the working precision
    // operand component i: v[i], or the next Newton-CG direction -r + beta d,
    // one fused multiply-add in the working precision (the same formula for
    // a row's own direction, which it stores, and for its neighbours')
    auto dir = [&](int64_t i) __attribute__((always_inline)) -> T {
        if constexpr (CG) return cg_dir_comp(cg.r[i], cg.d_old[i], beta_t);
        else return v[i];
    };
    // Rows go in slices of kSliceRows, one wave per slice: lane l takes row
    // kSliceRows * t + l, and spring j of the slice's rows is one coalesced
    // load.  A workgroup takes a contiguous slice range (ranges grouped by
    // XCD) and its waves walk it four slices apart.
    const int lane = int(threadIdx.x) & (kSliceRows - 1);
    T *rec = frec + (FACES ? (int(threadIdx.x) / kSliceRows) * kFaceHvpFields * kFaceRound : 0);
    int32_t t0, t1, tn;
    slice_range(A.nv, t0, t1, tn);
    SliceRow<T> hn;
    double vy = 0.0;  // this lane's part of v.y
    // A plain product inside a Newton-CG solve (cg.st set) does nothing once
    // the solve has ended.
    if constexpr (!CG)
        if (cg.st && cg_stop<kHvpThreads>(cg.st, &stop_bc)) return;  // workgroup-uniform
    // The first slice's loads are issued before the Newton-CG step below, so
    // that their latency overlaps its sum.
    if (tn < t1) slice_head<T, FACES, CG>(A, tn, lane, x, v, cg, hn);
    if constexpr (CG) {
        // Every workgroup takes the step that closes the previous update
        // (convergence or beta) from the partial sums of r.r, the same way;
        // none runs once the solve has ended.
        int32_t stop = cg_stop<kHvpThreads>(cg.st, &stop_bc);
        if (!stop && cg.iter > 0)
            beta = cg_beta_step<kHvpThreads>(cg.st, cg.rr_parts, cg.n_rr, cg.iter, blockIdx.x == 0,
                                             stop, red, &sum_bc);
        if (stop) return;  // workgroup-uniform
        beta_t = T(beta);
    }
    for (; tn < t1;) {  // wave-uniform
        const int32_t t = tn;
        const SliceRow<T> h = hn;
        tn += kSliceWaves;
        if (tn < t1) slice_head<T, FACES, CG>(A, tn, lane, x, v, cg, hn);
        const int32_t a = h.a;
        const bool live = h.live != 0;
        const int32_t p = A.sl_ptr[t];
        const int32_t ns = A.springs_on ? (A.sl_ptr[t + 1] - p) / kSliceRows : 0;
        T va[3], Y[3] = {T(0), T(0), T(0)};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if constexpr (CG) va[k] = cg_dir_comp(h.o0[k], h.o1[k], beta_t);
            else va[k] = h.o0[k];
            if (CG && live) cg.d_new[int64_t(a) * 3 + k] = va[k];
        }
        // Every term is evaluated once in DualHv numbers seeded with the
        // term's variables and the matching components of v; the gradient's
        // directional derivative gt is the term's Hessian applied to v.
        // Springs in the row's column order, kSliceBatch at a time.
        for (int32_t j0 = 0; j0 < ns; j0 += kSliceBatch) {  // wave-uniform
            int32_t nb[kSliceBatch];
            T L[kSliceBatch];
            slice_batch<T, FACES>(A, h, p, ns, j0, lane, a, nb, L);
            T xb[kSliceBatch][3], vb[kSliceBatch][3];
#pragma unroll
            for (int j = 0; j < kSliceBatch; ++j)
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    xb[j][k] = x[int64_t(nb[j]) * 3 + k];
                    vb[j][k] = dir(int64_t(nb[j]) * 3 + k);
                }
#pragma unroll
            for (int j = 0; j < kSliceBatch; ++j) {
                if (j0 + j >= ns) break;
                if (!(L[j] >= T(0))) continue;
                DualHv<T, 3> d[3];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    d[k] = DualHv<T, 3>::var(h.xa[k] - xb[j][k], k, va[k] - vb[j][k]);
                const DualHv<T, 3> e = spring_energy(d, L[j], A.k);
#pragma unroll
                for (int k = 0; k < 3; ++k) Y[k] += e.gt[k];
            }
        }
        if constexpr (FACES) slice_faces(A, t, h, rec, x, dir, Y);
        if (A.inertia_on) {
            // seeded at z = 0 (x_tilde not loaded): the Hessian c I is the same
            DualHv<T, 3> z[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) z[k] = DualHv<T, 3>::var(T(0), k, va[k]);
            const DualHv<T, 3> e = inertia_energy(z, A.c);
#pragma unroll
            for (int k = 0; k < 3; ++k) Y[k] += e.gt[k];
        }
        if (live)
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                // non-temporal: y is not read again here, and its lines
                // would evict neighbours' x and v from L2
                __builtin_nontemporal_store(Y[k], y + int64_t(a) * 3 + k);
                vy += double(va[k]) * double(Y[k]);
            }
    }
    if (A.hvp_dot) {
        const double sum = block_sum<kHvpThreads>(vy, red);
        if (threadIdx.x == 0) A.hvp_dot[blockIdx.x] = sum;
    }
}

// The runtime contacts' part of y for the rows they touch, after
// k_hvp_rows (topology terms of every row) and k_vf_hvp (the contacts'
// H_e u_e strips): the grid strides over the incidence entries and the
// thread at a row's first entry adds the row's pair terms, evaluated here
// in DualHv numbers, and its contact strips, in element order.  With dot
// set each workgroup stores its partial sum of v_a . (the added part),
// which completes the Newton-CG d.Hd sums of k_hvp_rows; nothing is added
// once the solve has ended.
template <typename T>
__global__ void __launch_bounds__(kThreads)
k_hvp_pair_rows(RowArgs<T> A, const T *__restrict__ x, const T *__restrict__ v,
                T *__restrict__ y, double *__restrict__ dot, const CgState *st)
{
    __shared__ double red[kThreads / 64];
    const int act = A.state->active;
    const bool live = !(st && st->stop) && act != 0;
    const int32_t ninc = live ? A.pat.pinc_ptr[act][A.nv] : 0;
    double part = 0.0;
    for (int32_t k = int32_t(blockIdx.x) * kThreads + int32_t(threadIdx.x); k < ninc;
         k += int32_t(gridDim.x) * kThreads) {
        const int32_t a = A.pat.trow[act][k];
        if (a >= 0) {
            const int32_t p0 = A.pat.pinc_ptr[act][a], p1 = A.pat.pinc_ptr[act][a + 1];
            const int32_t npa = A.state->np[act];
            const int32_t *pl = A.pat.pinc[act];
            const int32_t *prs = A.pat.pairs[act];
            T xa[3], va[3], Y[3] = {T(0), T(0), T(0)};
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                xa[c] = x[int64_t(a) * 3 + c];
                va[c] = v[int64_t(a) * 3 + c];
            }
            for (int32_t q0 = p0; q0 < p1; ++q0) {
                // the entry's stored partner (pairs) or place in the contact
                const int4 ps = A.pat.pslot[act][q0];
                const int32_t q = pl[q0];
                if (q >= npa) {  // vertex-face contact: the row's strip of H_e u_e
                    const int32_t e = q - npa;
                    int li = ps.z <= -2 ? -2 - ps.z : -1;
                    if (li < 0) {
                        const int4 w = *reinterpret_cast<const int4 *>(A.vf_ids + 4 * int64_t(e));
                        li = w.x == a ? 0 : (w.y == a ? 1 : (w.z == a ? 2 : 3));
                    }
                    const T *L = A.vf_hvp + (4 * int64_t(e) + li) * kVfHvpStrip;
#pragma unroll
                    for (int c = 0; c < 3; ++c) Y[c] += L[c];
                    continue;
                }
                int32_t b = ps.z >> 1;
                if (ps.z < 0) {  // not recorded: from the pair
                    const int32_t i0 = prs[2 * q], i1 = prs[2 * q + 1];
                    b = i0 == a ? i1 : i0;
                }
                T dz[3], dv[3];
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    dz[c] = xa[c] - x[int64_t(b) * 3 + c];
                    dv[c] = va[c] - v[int64_t(b) * 3 + c];
                }
                const T l2 = dz[0] * dz[0] + dz[1] * dz[1] + dz[2] * dz[2];
                if (!(l2 < A.dhat * A.dhat)) continue;  // outside the barrier's support
                DualHv<T, 3> d[3];
#pragma unroll
                for (int c = 0; c < 3; ++c) d[c] = DualHv<T, 3>::var(dz[c], c, dv[c]);
                const DualHv<T, 3> en = barrier_energy(d, A.kappa, A.dhat);
#pragma unroll
                for (int c = 0; c < 3; ++c) Y[c] += en.gt[c];
            }
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                y[int64_t(a) * 3 + c] += Y[c];
                part += double(va[c]) * double(Y[c]);
            }
        }
    }
    if (dot) {
        const double sum = block_sum<kThreads>(part, red);
        if (threadIdx.x == 0) dot[blockIdx.x] = sum;
    }
}

// ---------------------------------------------------------------------------
// Gauss-Newton product of the vector objective, y = J^T (J v), H's
// positive semi-definite counterpart.  Row owner as above: each spring's
// local Jacobian row w = dR/dz (z = x_a - x_b, from a first-order dual
// evaluation) is formed in registers, and the row gets w (w . (v_a - v_b));
// the inertia rows contribute sqrt(c) (sqrt(c) v_a).  J is never stored.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kHvpThreads)
k_gn_rows(RowArgs<T> A, T sqrt_k, T sqrt_c, const T *__restrict__ x, const T *__restrict__ v,
          T *__restrict__ y)
{
    // the walk of k_hvp_rows: slices of rows, the next slice's head loaded
    // while the current one is processed
    const int lane = int(threadIdx.x) & (kSliceRows - 1);
    int32_t t0, t1, tn;
    slice_range(A.nv, t0, t1, tn);
    const CgDir<T> none{};
    SliceRow<T> hn;
    if (tn < t1) slice_head<T, false, false>(A, tn, lane, x, v, none, hn);
    for (; tn < t1;) {  // wave-uniform
        const int32_t t = tn;
        const SliceRow<T> h = hn;
        tn += kSliceWaves;
        if (tn < t1) slice_head<T, false, false>(A, tn, lane, x, v, none, hn);
        const int32_t a = h.a;
        const bool live = h.live != 0;
        const int32_t p = A.sl_ptr[t];
        const int32_t ns = A.springs_on ? (A.sl_ptr[t + 1] - p) / kSliceRows : 0;
        T Y[3] = {T(0), T(0), T(0)};
        const T *va = h.o0;
        for (int32_t j0 = 0; j0 < ns; j0 += kSliceBatch) {  // wave-uniform
            int32_t nb[kSliceBatch];
            T L[kSliceBatch];
            slice_batch<T, false>(A, h, p, ns, j0, lane, a, nb, L);
            T xb[kSliceBatch][3], vb[kSliceBatch][3];
#pragma unroll
            for (int j = 0; j < kSliceBatch; ++j)
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    xb[j][k] = x[int64_t(nb[j]) * 3 + k];
                    vb[j][k] = v[int64_t(nb[j]) * 3 + k];
                }
#pragma unroll
            for (int j = 0; j < kSliceBatch; ++j) {
                if (j0 + j >= ns) break;
                if (!(L[j] >= T(0))) continue;
                Dual1<T, 3> z[3];
#pragma unroll
                for (int k = 0; k < 3; ++k) z[k] = Dual1<T, 3>::var(h.xa[k] - xb[j][k], k);
                const Dual1<T, 3> e = spring_residual(z, L[j], sqrt_k);
                const T u = e.g[0] * (va[0] - vb[j][0]) + e.g[1] * (va[1] - vb[j][1]) +
                            e.g[2] * (va[2] - vb[j][2]);
#pragma unroll
                for (int k = 0; k < 3; ++k) Y[k] += e.g[k] * u;
            }
        }
        if (A.inertia_on)
#pragma unroll
            for (int k = 0; k < 3; ++k) Y[k] += sqrt_c * (sqrt_c * va[k]);
        if (live)
#pragma unroll
            for (int k = 0; k < 3; ++k) y[int64_t(a) * 3 + k] = Y[k];
    }
}

}  // namespace

template <typename T>
hipError_t launch_gauss_newton_rows(const RowArgs<T> &a, T sqrt_k, T sqrt_c, const T *x,
                                    const T *v, T *y, int grid, hipStream_t s)
{
    hipLaunchKernelGGL(k_gn_rows<T>, dim3(grid), dim3(kHvpThreads), 0, s, a, sqrt_k, sqrt_c, x, v,
                       y);
    return hipGetLastError();
}
template hipError_t launch_gauss_newton_rows<float>(const RowArgs<float> &, float, float,
                                                    const float *, const float *, float *, int,
                                                    hipStream_t);
template hipError_t launch_gauss_newton_rows<double>(const RowArgs<double> &, double, double,
                                                     const double *, const double *, double *, int,
                                                     hipStream_t);

template <typename T>
int rows_lds_bytes(int lds_blocks)
{
    // the staging slice plus up to 16 bytes of alignment padding in front
    return int(((int64_t(lds_blocks) * 9 * int64_t(sizeof(T)) + 16) + 15) & ~int64_t(15));
}

template <typename T, bool F, bool P>
static hipError_t rows_occupancy(int lds, int *occ_e, int *occ_h)
{
    hipError_t e;
    if constexpr (F && !P)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(occ_e, k_eval_face_rows<T>, kRowThreads,
                                                         lds);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(occ_e, k_eval_rows<T, F, P>, kRowThreads,
                                                         lds);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(occ_h, k_hvp_rows<T, F, false>,
                                                         kHvpThreads, 0);
    return e;
}

template <typename T>
hipError_t rows_grid(int lds_blocks, int nchunk, int faces, int pairs, int *grid_eval,
                     int *grid_hvp)
{
    int dev = 0, cus = 0, occ_e = 0, occ_h = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int lds = rows_lds_bytes<T>(lds_blocks);
    if (e == hipSuccess) {
        if (faces)
            e = pairs ? rows_occupancy<T, true, true>(lds, &occ_e, &occ_h)
                      : rows_occupancy<T, true, false>(lds, &occ_e, &occ_h);
        else
            e = pairs ? rows_occupancy<T, false, true>(lds, &occ_e, &occ_h)
                      : rows_occupancy<T, false, false>(lds, &occ_e, &occ_h);
    }
    if (e != hipSuccess) return e;
    // The fewest workgroups that still need the same number of rounds
    // k = ceil(units / resident): every workgroup then takes k or k - 1
    // units, where a full resident grid would leave most of them idle
    // while a few take one more round (1000 x 1000 cloth eval: 15,625
    // chunks over 2048 resident workgroups, 7.6 rounds; 1954 workgroups of
    // 8 chunks ran 60.2 against 62.8 us).
    auto clamp = [&](int occ, int64_t units) {
        const int64_t full = int64_t(cus > 0 ? cus : 1) * (occ > 0 ? occ : 1);
        if (units <= full) return int(units < 1 ? 1 : units);
        const int64_t rounds = (units + full - 1) / full;
        return int((units + rounds - 1) / rounds);
    };
    // single-wave workgroups: a resident count per CU that is a multiple of
    // its four SIMDs gives every SIMD the same number of waves
    if (occ_e > 4) occ_e -= occ_e % 4;
    *grid_eval = clamp(occ_e, nchunk);
    // the product kernels walk rows kHvpThreads at a time (chunks hold at
    // most kRowsPerChunk rows) on a full resident grid: their latency-bound
    // slice walk gains more from the resident waves than from even rounds
    // (1000 x 1000 cloth HVP: 0.2-0.3 us faster than the balanced grid)
    {
        const int64_t units = (int64_t(nchunk) * kRowsPerChunk + kHvpThreads - 1) / kHvpThreads;
        const int64_t full = int64_t(cus > 0 ? cus : 1) * (occ_h > 0 ? occ_h : 1);
        *grid_hvp = int(units < full ? (units < 1 ? 1 : units) : full);
    }
    return hipSuccess;
}

template <typename T, bool F, bool P>
static void launch_eval_rows_as(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                                int grid, int lds, hipStream_t s)
{
    if constexpr (F && !P)
        hipLaunchKernelGGL((k_eval_face_rows<T>), dim3(grid), dim3(kRowThreads), lds, s, a, x, g,
                           hv, es);
    else
        hipLaunchKernelGGL((k_eval_rows<T, F, P>), dim3(grid), dim3(kRowThreads), lds, s, a, x, g,
                           hv, es);
}

// The face tables the row kernels read when the face term is on.
template <typename T>
static bool face_tables_ok(const RowArgs<T> &a)
{
    return !a.faces_on ||
           (a.fptr && a.finc && a.rfinc && a.sf_ptr && a.sface && a.face_dm && a.face_area);
}

template <typename T>
hipError_t launch_eval_pair_rows(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                                 int grid, hipStream_t s)
{
    if (!face_tables_ok(a)) return hipErrorInvalidValue;
    for (int k = 1; k <= 2; ++k)  // the contact buffers the kernel may read
        if (!a.pat.rp[k] || !a.pat.ci[k] || !a.pat.pairs[k] || !a.pat.pinc_ptr[k] ||
            !a.pat.pinc[k] || !a.pat.trow[k] || !a.pat.pslot[k])
            return hipErrorInvalidValue;
    if (a.vf_stride > 0 && (!a.vf_eval || !a.vf_ids || !a.vf_slots)) return hipErrorInvalidValue;
    if (a.faces_on)
        hipLaunchKernelGGL((k_eval_pair_rows<T, true>), dim3(grid), dim3(kThreads), 0, s, a, x, g,
                           hv, es);
    else
        hipLaunchKernelGGL((k_eval_pair_rows<T, false>), dim3(grid), dim3(kThreads), 0, s, a, x, g,
                           hv, es);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_eval_rows(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                            int grid, hipStream_t s)
{
    const int lds = rows_lds_bytes<T>(a.lds_blocks);
    if (!face_tables_ok(a)) return hipErrorInvalidValue;
    if (a.pairs_on)  // the buffers the contact-capacity variant reads
        for (int k = 1; k <= 2; ++k)
            if (!a.pat.rp[k] || !a.pat.ci[k] || !a.pat.pinc_ptr[k] || !a.pat.pnew[k] ||
                !a.pat.rins1[k])
                return hipErrorInvalidValue;
    if (a.faces_on)
        a.pairs_on ? launch_eval_rows_as<T, true, true>(a, x, g, hv, es, grid, lds, s)
                   : launch_eval_rows_as<T, true, false>(a, x, g, hv, es, grid, lds, s);
    else
        a.pairs_on ? launch_eval_rows_as<T, false, true>(a, x, g, hv, es, grid, lds, s)
                   : launch_eval_rows_as<T, false, false>(a, x, g, hv, es, grid, lds, s);
    return hipGetLastError();
}

template <typename T, bool F>
static void launch_hvp_rows_as(const RowArgs<T> &a, const T *x, const T *v, T *y, int grid,
                               hipStream_t s, const CgDir<T> &cg)
{
    if (cg.r)
        hipLaunchKernelGGL((k_hvp_rows<T, F, true>), dim3(grid), dim3(kHvpThreads), 0, s, a, x, v,
                           y, cg);
    else
        hipLaunchKernelGGL((k_hvp_rows<T, F, false>), dim3(grid), dim3(kHvpThreads), 0, s, a, x, v,
                           y, cg);
}

template <typename T>
hipError_t launch_hvp_rows(const RowArgs<T> &a, const T *x, const T *v, T *y, int grid,
                           hipStream_t s, const CgDir<T> &cg)
{
    if (!face_tables_ok(a) || !a.sl_ptr) return hipErrorInvalidValue;
    if (a.faces_on)
        launch_hvp_rows_as<T, true>(a, x, v, y, grid, s, cg);
    else
        launch_hvp_rows_as<T, false>(a, x, v, y, grid, s, cg);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hvp_pair_rows(const RowArgs<T> &a, const T *x, const T *v, T *y, double *dot,
                                int grid, const CgState *st, hipStream_t s)
{
    for (int k = 1; k <= 2; ++k)  // the contact buffers the kernel may read
        if (!a.pat.pairs[k] || !a.pat.pinc_ptr[k] || !a.pat.pinc[k] || !a.pat.trow[k] ||
            !a.pat.pslot[k])
            return hipErrorInvalidValue;
    if (a.vf_stride > 0 && (!a.vf_ids || !a.vf_hvp)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_hvp_pair_rows<T>, dim3(grid), dim3(kThreads), 0, s, a, x, v, y, dot, st);
    return hipGetLastError();
}

#define LAD_ROWS_INST(T)                                                                          \
    template int rows_lds_bytes<T>(int);                                                          \
    template hipError_t rows_grid<T>(int, int, int, int, int *, int *);                           \
    template hipError_t launch_eval_rows<T>(const RowArgs<T> &, const T *, T *, T *, EnergySink,  \
                                            int, hipStream_t);                                    \
    template hipError_t launch_eval_pair_rows<T>(const RowArgs<T> &, const T *, T *, T *,         \
                                                 EnergySink, int, hipStream_t);                   \
    template hipError_t launch_hvp_rows<T>(const RowArgs<T> &, const T *, const T *, T *, int,    \
                                           hipStream_t, const CgDir<T> &);                        \
    template hipError_t launch_hvp_pair_rows<T>(const RowArgs<T> &, const T *, const T *, T *,    \
                                                double *, int, const CgState *, hipStream_t);
LAD_ROWS_INST(float)
LAD_ROWS_INST(double)

}  // namespace lad
