// terms_engine.h -- the term front end's kernels: explicit gradient and
// block-CSR Hessian, and the matrix-free Hessian-vector product, for any
// compile-time list of user terms (user_terms.h), all of them fused into one
// pass over the rows.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", section "Method": from a user's local energy terms the
// system analyses the stencil and derivative needs, preallocates the CSR
// pattern from the topology, evaluates every term in forward mode with its
// intermediates in registers, and assembles g = sum_j S_j^T g_j and
// H = sum_j S_j^T H_j S_j.  Its stated limitation is one kernel per term
// with no fusion across terms; here one launch evaluates every term of the
// list (the unfused mode runs one launch per term and accumulates, for
// comparison).
//
// Decomposition: row owner, as the fixed-function row kernels.  One lane
// owns one block row; for each element incident to its vertex a (at
// position i in the element) it evaluates the term on numbers that carry
// only the Hessian rows of a's three variables (StripDual), seeding a's
// coordinates as variables 0..2 and the element's vertex (i + b) % K as
// variables 3b..3b+2.  The strip's block b is then exactly the row's block
// for that vertex, at a column offset the incidence record holds, so a row
// is written by one lane, in a fixed order, without atomics.  The energy of
// an element is counted by the row of its vertex 0.  The product seeds
// every variable with the direction's component and tracks derivatives in
// a's three variables only (DualHv<T, 3>): every rule of those numbers acts
// on one gradient component at a time, so this gives exactly a's part of
// H_j v_j.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "dual2.h"
#include "lad_device.h"
#include "lad_internal.h"
#include "lad_terms_internal.h"
#include "strip_dual.h"

namespace lad {
namespace terms {

// Incident elements whose loads a lane issues together: more for small
// stencils, whose per-element operands take few registers.
template <int K>
constexpr int term_batch()
{
    return K <= 2 ? 4 : 2;
}

// The same for the explicit evaluation, whose occupancy is set by its LDS
// staging (about two waves per SIMD), not by its registers: wider batches
// put more of a row's loads in flight at once (a cloth row's springs in one).
template <int K>
constexpr int term_batch_eval()
{
    return K <= 2 ? 8 : (K == 3 ? 4 : 2);
}

// LDS hand-off between the lanes of one wave: a wave's LDS operations run in
// issue order, so only the compiler must be kept from moving memory
// operations across this point (no workgroup barrier, which would also wait
// for the chunk's outstanding HBM stores).
__device__ __forceinline__ void terms_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The reverse of stream_out: n elements from global src into LDS dst, which
// sits `pad` elements after a 16-byte boundary exactly where src is
// misaligned, so the body moves in aligned 16-byte loads.
template <int NT, typename T>
__device__ __forceinline__ void stream_in(T *dst, const T *__restrict__ src, int n, int pad)
{
    constexpr int V = Vec<T>::n;
    using VT = typename Vec<T>::type;
    const int head = min(n, (V - pad) % V);
    for (int i = threadIdx.x; i < head; i += NT) dst[i] = src[i];
    const int nvec = (n - head) / V;
    VT *dv = reinterpret_cast<VT *>(dst + head);
    const VT *sv = reinterpret_cast<const VT *>(src + head);
    for (int i = threadIdx.x; i < nvec; i += NT) dv[i] = __builtin_nontemporal_load(sv + i);
    for (int i = head + nvec * V + threadIdx.x; i < n; i += NT) dst[i] = src[i];
}

// The incidence records [base, base + B) of row a (indices clamped into the
// row's range, so every load is valid): position and block offsets (pk),
// vertex ids in element order and constants.  Small stencils read them from
// the row's own records: rows in order, or (SLICED, the product kernel,
// whose waves walk whole slices) the copy transposed per slice, where a
// wave reads record j of its 64 rows with one coalesced load; larger ones
// gather the element's vertex ids and constants by element id.
template <typename Term, bool SLICED, typename T, int B>
__device__ __forceinline__ void load_records(const TermData<T> &td, int32_t a, int32_t p0,
                                             int32_t base, int32_t p1, TermInc (&rec)[B],
                                             int32_t (&vid)[B][Term::kVerts],
                                             T (&cc)[B][Term::kConsts > 0 ? Term::kConsts : 1])
{
    constexpr int K = Term::kVerts, NC = Term::kConsts;
    if constexpr (K <= kInlineVerts) {
        using R = InlineRec<T, NC>;
        R q[B];
        if constexpr (SLICED) {
            // the row's records in its slice, kTermSliceRows apart
            const R *ir = static_cast<const R *>(td.inl_sl) + td.sl_ptr[a / kTermSliceRows] +
                          a % kTermSliceRows;
#pragma unroll
            for (int j = 0; j < B; ++j)
                q[j] = ir[int64_t(min(base + j, p1 - 1) - p0) * kTermSliceRows];
        } else {
            const R *ir = static_cast<const R *>(td.inl);
#pragma unroll
            for (int j = 0; j < B; ++j) q[j] = ir[min(base + j, p1 - 1)];
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            rec[j].e = 0;  // not needed: the record holds the element's data
            rec[j].pk = q[j].pk;
            const int i = int(q[j].pk & 3u);
#pragma unroll
            for (int u = 0; u < K; ++u) vid[j][u] = u == i ? a : q[j].other;
#pragma unroll
            for (int k = 0; k < NC; ++k) cc[j][k] = q[j].c[k];
        }
    } else {
#pragma unroll
        for (int j = 0; j < B; ++j) rec[j] = td.inc[min(base + j, p1 - 1)];
#pragma unroll
        for (int j = 0; j < B; ++j) {
#pragma unroll
            for (int u = 0; u < K; ++u) vid[j][u] = td.elems[int64_t(rec[j].e) * K + u];
#pragma unroll
            for (int k = 0; k < NC; ++k) cc[j][k] = td.consts[int64_t(rec[j].e) * NC + k];
        }
    }
}

// Terms that depend only on differences of their vertices' positions say so
// (kTranslationInvariant); the engine then differentiates them in the
// positions of vertices 1 .. K-1 with vertex 0 held fixed, on one full
// second-order number of 3(K-1) variables, and rebuilds the row's blocks
// from the zero block-row sums of a translation-invariant Hessian:
//   g_0 = -sum_j g_j,   H_jk as computed (j, k >= 1),
//   H_0k = H_k0^T = -sum_j H_jk,   H_00 = sum_jk H_jk.
// For K <= 3 that is fewer numbers per value than the strip (10 against 25
// for two vertices, 28 against 37 for three).
template <typename Term>
constexpr bool use_relative()
{
    return Term::kTranslationInvariant && Term::kVerts >= 2 && Term::kVerts <= 3;
}

// A block's part into the staged row: stored by the block's first writer
// (FW: the fused pass, which starts from unwritten staging), else added.
template <bool FW, typename T>
__device__ __forceinline__ void put_block(T *B, uint32_t pk, int b, const T (&h)[9])
{
    const bool first = FW && ((pk >> (1 + b)) & 1u);
#pragma unroll
    for (int k = 0; k < 9; ++k) B[k] = first ? h[k] : B[k] + h[k];
}

// Row i's blocks of element (e, vertices vid) by relative seeding; adds
// into D (the row's diagonal), G and the row's blocks at the offsets in pk.
template <typename Term, bool FW, typename T>
__device__ __forceinline__ void row_elem_relative(const T (&xv)[Term::kVerts][3], const T *cc,
                                                  int i, uint32_t pk, T *Hrow, T D[9], T G[3],
                                                  double &E)
{
    constexpr int K = Term::kVerts, NZ = 3 * (K - 1);
    Dual2<T, NZ> z[K][3];
#pragma unroll
    for (int c = 0; c < 3; ++c) z[0][c] = Dual2<T, NZ>::constant(xv[0][c]);
#pragma unroll
    for (int v = 1; v < K; ++v)
#pragma unroll
        for (int c = 0; c < 3; ++c) z[v][c] = Dual2<T, NZ>::var(xv[v][c], 3 * (v - 1) + c);
    const Dual2<T, NZ> en = Term::energy(z, cc);
    if (i == 0) E += double(en.v);
    // Hessian block (a, b) of the full element, a, b = 0 .. K-1, entry (r, c)
    auto hb = [&](int a, int b, int r, int c) -> T {
        T s = T(0);
#pragma unroll
        for (int j = 1; j < K; ++j)
#pragma unroll
            for (int k = 1; k < K; ++k) {
                const T h = en.hess(3 * (j - 1) + r, 3 * (k - 1) + c);
                const T wa = a == 0 ? T(-1) : (a == j ? T(1) : T(0));
                const T wb = b == 0 ? T(-1) : (b == k ? T(1) : T(0));
                s += (wa * wb) * h;
            }
        return s;
    };
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        T gi = T(0);
#pragma unroll
        for (int j = 1; j < K; ++j) gi += (i == 0 ? T(-1) : (i == j ? T(1) : T(0))) * en.g[3 * (j - 1) + r];
        G[r] += gi;
#pragma unroll
        for (int c = 0; c < 3; ++c) D[3 * r + c] += hb(i, i, r, c);
    }
#pragma unroll
    for (int b = 1; b < K; ++b) {
        const int v = (i + b) % K;
        T h[9];
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int c = 0; c < 3; ++c) h[3 * r + c] = hb(i, v, r, c);
        put_block<FW>(Hrow + 9 * int32_t((pk >> (8 * b)) & 255u), pk, b, h);
    }
}

// The row's contributions from one term type: for each batch of incident
// elements, every load first (records, vertex ids, positions, constants),
// then the evaluations.  D is the row's diagonal block, G its gradient,
// Hrow its slice of the staged blocks.
template <typename Term, bool FW, typename T>
__device__ __forceinline__ void row_term_eval(const TermData<T> &td, int32_t a,
                                             const T *__restrict__ x, T *Hrow, T D[9],
                                             T G[3], double &E)
{
    constexpr int K = Term::kVerts, N = 3 * K, NC = Term::kConsts;
    constexpr int kTermBatch = term_batch_eval<K>();
    static_assert(K >= 1 && K <= kMaxVerts, "stencil of 1 to 4 vertices");
    const int32_t p0 = td.inc_ptr[a], p1 = td.inc_ptr[a + 1];
    for (int32_t base = p0; base < p1; base += kTermBatch) {
        TermInc rec[kTermBatch];
        int32_t vid[kTermBatch][K];
        T xv[kTermBatch][K][3];
        T cc[kTermBatch][NC > 0 ? NC : 1];
        load_records<Term, false>(td, a, p0, base, p1, rec, vid, cc);
#pragma unroll
        for (int j = 0; j < kTermBatch; ++j)
#pragma unroll
            for (int v = 0; v < K; ++v)
#pragma unroll
                for (int c = 0; c < 3; ++c) xv[j][v][c] = x[int64_t(vid[j][v]) * 3 + c];
#pragma unroll
        for (int j = 0; j < kTermBatch; ++j) {
            if (base + j >= p1) break;
            const int i = int(rec[j].pk & 3u);
            if constexpr (use_relative<Term>()) {
                row_elem_relative<Term, FW>(xv[j], cc[j], i, rec[j].pk, Hrow, D, G, E);
                continue;
            }
            StripDual<T, N> z[K][3];
#pragma unroll
            for (int v = 0; v < K; ++v) {
                const int b = (v - i + K) % K;  // the vertex's block in the strip
#pragma unroll
                for (int c = 0; c < 3; ++c) z[v][c] = StripDual<T, N>::var(xv[j][v][c], 3 * b + c);
            }
            const StripDual<T, N> en = Term::energy(z, cc[j]);
            if (i == 0) E += double(en.v);
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                G[r] += en.g[r];
#pragma unroll
                for (int c = 0; c < 3; ++c) D[3 * r + c] += en.h[r][c];
            }
#pragma unroll
            for (int b = 1; b < K; ++b) {
                T h[9];
#pragma unroll
                for (int r = 0; r < 3; ++r)
#pragma unroll
                    for (int c = 0; c < 3; ++c) h[3 * r + c] = en.h[r][3 * b + c];
                put_block<FW>(Hrow + 9 * int32_t((rec[j].pk >> (8 * b)) & 255u), rec[j].pk, b, h);
            }
        }
    }
}

template <typename T, bool FW, typename... Terms, size_t... I>
__device__ __forceinline__ void row_eval_all(const TermsArgs<T> &A, int32_t a,
                                             const T *__restrict__ x, T *Hrow, T D[9], T G[3],
                                             double &E, std::index_sequence<I...>)
{
    (row_term_eval<Terms, FW>(A.t[I], a, x, Hrow, D, G, E), ...);
}

// Energy, gradient and Hessian rows of the term list.  With ACC set the
// launch adds into g and H as they are (the unfused mode's later terms);
// otherwise it overwrites them.  FW (the fused launch of the whole list):
// every block's first writer stores it and the diagonal is stored, so the
// staging is not zeroed first; else it is zeroed (or read back, ACC) and
// every part added.  Chunks of 64 rows are staged in LDS (a single-wave
// workgroup, so the hand-off needs no barrier) and streamed out with
// 16-byte non-temporal stores.
template <typename T, bool ACC, bool FW, typename... Terms>
__global__ void __launch_bounds__(kRowThreads)
k_terms_eval(TermsArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
             EnergySink esink)
{
    extern __shared__ __align__(16) unsigned char smem[];
    T *stage = reinterpret_cast<T *>(smem);
    double eacc = 0.0;
    for (int ch = first_chunk(); ch < A.nchunk; ch += int(gridDim.x)) {  // round robin
        const int32_t v0 = A.chunk[ch].v0, nrows = A.chunk[ch].nown;
        const int32_t sb = A.rp[v0];
        const int32_t nblk = A.rp[v0 + nrows] - sb;
        const bool fits = nblk <= A.lds_blocks;  // checked at build; never false
        const int pad = stage_pad<T>(int64_t(sb) * 9);
        T *Hs = stage + pad;
        if (fits) {
            if constexpr (ACC)
                stream_in<kRowThreads>(Hs, hv + int64_t(sb) * 9, nblk * 9, pad);
            else if constexpr (!FW)
                for (int k = int(threadIdx.x); k < nblk * 9; k += kRowThreads) Hs[k] = T(0);
        }
        terms_lds_sync();
        if (fits && int(threadIdx.x) < nrows) {
            const int32_t a = v0 + int32_t(threadIdx.x);
            T *Hrow = Hs + 9 * (A.rp[a] - sb);
            T D[9], G[3];
#pragma unroll
            for (int k = 0; k < 9; ++k) D[k] = T(0);
#pragma unroll
            for (int k = 0; k < 3; ++k) G[k] = ACC ? g[int64_t(a) * 3 + k] : T(0);
            row_eval_all<T, FW, Terms...>(A, a, x, Hrow, D, G, eacc,
                                          std::index_sequence_for<Terms...>{});
            T *B = Hrow + 9 * A.diag[a];
#pragma unroll
            for (int k = 0; k < 9; ++k) B[k] = FW ? D[k] : B[k] + D[k];
#pragma unroll
            for (int k = 0; k < 3; ++k) g[int64_t(a) * 3 + k] = G[k];
        }
        terms_lds_sync();
        if (fits) stream_out<kRowThreads>(hv + int64_t(sb) * 9, Hs, nblk * 9, pad);
        terms_lds_sync();
    }
    store_energy(esink, block_sum<kRowThreads>(eacc, nullptr));
}

// The row's part of sum_j H_j v_j over one term type.
template <typename Term, typename T>
__device__ __forceinline__ void row_term_hvp(const TermData<T> &td, int32_t a,
                                             const T *__restrict__ x, const T *__restrict__ v,
                                             T Y[3])
{
    constexpr int K = Term::kVerts, NC = Term::kConsts;
    constexpr int kTermBatch = term_batch<K>();
    const int32_t p0 = td.inc_ptr[a], p1 = td.inc_ptr[a + 1];
    for (int32_t base = p0; base < p1; base += kTermBatch) {
        TermInc rec[kTermBatch];
        int32_t vid[kTermBatch][K];
        T xv[kTermBatch][K][3], vv[kTermBatch][K][3];
        T cc[kTermBatch][NC > 0 ? NC : 1];
        load_records<Term, true>(td, a, p0, base, p1, rec, vid, cc);
#pragma unroll
        for (int j = 0; j < kTermBatch; ++j)
#pragma unroll
            for (int u = 0; u < K; ++u)
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    xv[j][u][c] = x[int64_t(vid[j][u]) * 3 + c];
                    vv[j][u][c] = v[int64_t(vid[j][u]) * 3 + c];
                }
#pragma unroll
        for (int j = 0; j < kTermBatch; ++j) {
            if (base + j >= p1) break;
            const int i = int(rec[j].pk & 3u);
            DualHv<T, 3> z[K][3];
#pragma unroll
            for (int u = 0; u < K; ++u)
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    z[u][c] = DualHv<T, 3>::var(xv[j][u][c], u == i ? c : -1, vv[j][u][c]);
            const DualHv<T, 3> en = Term::energy(z, cc[j]);
#pragma unroll
            for (int c = 0; c < 3; ++c) Y[c] += en.gt[c];
        }
    }
}

template <typename T, typename... Terms, size_t... I>
__device__ __forceinline__ void row_hvp_all(const TermsArgs<T> &A, int32_t a,
                                            const T *__restrict__ x, const T *__restrict__ v,
                                            T Y[3], std::index_sequence<I...>)
{
    (row_term_hvp<Terms>(A.t[I], a, x, v, Y), ...);
}

// y = H v over the term list; with ACC set the launch adds into y.  Each
// workgroup walks a contiguous range of rows (ranges grouped by XCD).  The
// kernel shares nothing between lanes, so its workgroups are four waves:
// the per-CU cap on workgroups would otherwise hold single-wave groups to
// 4 waves per SIMD, though its registers allow 8.
template <typename T, bool ACC, typename... Terms>
__global__ void __launch_bounds__(kTermsHvpThreads)
k_terms_hvp(TermsArgs<T> A, const T *__restrict__ x, const T *__restrict__ v, T *__restrict__ y)
{
    // ranges start on a slice boundary, so each wave's 64 rows read one
    // slice of the small-stencil records
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t nsl = (int64_t(A.nv) + kTermSliceRows - 1) / kTermSliceRows;
    const int32_t r0 = int32_t(nsl * w / gridDim.x * kTermSliceRows);
    const int32_t r1 = int32_t(min(int64_t(A.nv), nsl * (w + 1) / gridDim.x * kTermSliceRows));
    for (int32_t a = r0 + int32_t(threadIdx.x); a < r1; a += kTermsHvpThreads) {
        T Y[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) Y[k] = ACC ? y[int64_t(a) * 3 + k] : T(0);
        row_hvp_all<T, Terms...>(A, a, x, v, Y, std::index_sequence_for<Terms...>{});
#pragma unroll
        for (int k = 0; k < 3; ++k) y[int64_t(a) * 3 + k] = Y[k];
    }
}

}  // namespace terms
}  // namespace lad
