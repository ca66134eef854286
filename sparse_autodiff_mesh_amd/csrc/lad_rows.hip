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
// registers.  No block is written twice, nothing is zero-filled, there are no
// atomics, and every sum is taken in a fixed order: the result is bitwise
// reproducible.  A wave's 64 consecutive rows form one contiguous slice of
// the value array; it is staged in LDS and streamed to HBM with 16-byte
// nontemporal stores.  Workgroups are persistent: each walks a contiguous
// range of row chunks, and the ranges are grouped by XCD so that vertex
// positions shared by neighbouring rows stay in one L2.
#include "dual2.h"
#include "energies.h"
#include "lad_device.h"
#include "lad_internal.h"

namespace lad {

namespace {

constexpr int kBatch = 8;  // slots whose loads a lane issues together

// This workgroup's contiguous range [c0, c1) of the n chunks.
__device__ __forceinline__ void chunk_range(int n, int &c0, int &c1)
{
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    c0 = int(int64_t(n) * w / gridDim.x);
    c1 = int(int64_t(n) * (w + 1) / gridDim.x);
}

__device__ __forceinline__ bool slot_inserted(const uint32_t *ib, int32_t s)
{
    return (ib[s >> 5] >> (s & 31)) & 1u;
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
    int32_t a, s0, s1, kb0;   // vertex, active slot range, first base slot
    T xa[3];
};

// Walk the slots of row r in batches of kBatch.  For every slot s, `fn(s,
// kb, b, L)` gets the base-pattern index kb (-1 for a slot inserted by
// pairs), the column b and the rest length L of the spring behind the block
// (negative: no spring).  Loads of a batch are issued before any use.
template <typename T, typename Fn>
__device__ __forceinline__ void for_each_slot(const RowArgs<T> &A, const Row<T> &r, int act,
                                              const uint32_t *ib, Fn &&fn)
{
    int32_t nins = 0;  // inserted slots seen so far in this row
    for (int32_t base = r.s0; base < r.s1; base += kBatch) {
        int32_t kb[kBatch], b[kBatch];
        T L[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int32_t s = base + j;
            const bool ins = act != 0 && s < r.s1 && slot_inserted(ib, s);
            kb[j] = (s < r.s1 && !ins) ? r.kb0 + (s - r.s0) - nins : -1;
            nins += ins ? 1 : 0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            b[j] = kb[j] >= 0 ? A.ci0[kb[j]] : -1;
            L[j] = (kb[j] >= 0 && A.springs_on) ? A.slot_rest[kb[j]] : T(-1);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (base + j < r.s1) fn(base + j, kb[j], b[j], L[j]);
    }
}

// ---------------------------------------------------------------------------
// Energy, gradient and Hessian rows.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ double eval_row(const RowArgs<T> &A, int act, const int32_t *cia,
                                           const uint32_t *ib, const Row<T> &r, int32_t sb,
                                           T *Hs, const T *__restrict__ x, T *__restrict__ g)
{
    T D[9], G[3] = {T(0), T(0), T(0)};
#pragma unroll
    for (int i = 0; i < 9; ++i) D[i] = T(0);
    double E = 0.0;
    int32_t dslot = r.s0;

    for_each_slot(A, r, act, ib, [&](int32_t s, int32_t kb, int32_t b, T L) {
        T *B = Hs + 9 * (s - sb);
        if (kb >= 0 && b == r.a) {
            dslot = s;
            return;
        }
        if (!(L >= T(0))) {  // inserted by a pair, or no spring behind the block
#pragma unroll
            for (int i = 0; i < 9; ++i) B[i] = T(0);
            return;
        }
        Dual2<T, 3> d[3];
#pragma unroll
        for (int c = 0; c < 3; ++c)
            d[c] = Dual2<T, 3>::var(r.xa[c] - x[int64_t(b) * 3 + c], c);
        const Dual2<T, 3> e = spring_energy(d, L, A.k);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            G[i] += e.g[i];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const T h = e.hess(i, j);
                B[3 * i + j] = -h;
                D[3 * i + j] += h;
            }
        }
        if (r.a < b) E += double(e.v);
    });

    if (A.inertia_on) {
        Dual2<T, 3> z[3];
#pragma unroll
        for (int c = 0; c < 3; ++c)
            z[c] = Dual2<T, 3>::var(r.xa[c] - A.x_tilde[int64_t(r.a) * 3 + c], c);
        const Dual2<T, 3> e = inertia_energy(z, A.c);
        E += double(e.v);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            G[i] += e.g[i];
#pragma unroll
            for (int j = 0; j < 3; ++j) D[3 * i + j] += e.hess(i, j);
        }
    }

    if (act != 0) {  // runtime pairs of this row, in pair order
        const int32_t *pp = A.pat.pinc_ptr[act];
        const int32_t *pl = A.pat.pinc[act];
        const int32_t *prs = A.pat.pairs[act];
        for (int32_t k = pp[r.a]; k < pp[r.a + 1]; ++k) {
            const int32_t q = pl[k];
            const int32_t i0 = prs[2 * q], i1 = prs[2 * q + 1];
            const int32_t b = i0 == r.a ? i1 : i0;
            T dz[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) dz[c] = r.xa[c] - x[int64_t(b) * 3 + c];
            const T l2 = dz[0] * dz[0] + dz[1] * dz[1] + dz[2] * dz[2];
            if (!(l2 < A.dhat * A.dhat)) continue;  // outside the barrier's support
            Dual2<T, 3> d[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(dz[c], c);
            const Dual2<T, 3> e = barrier_energy(d, A.kappa, A.dhat);
            if (i0 == r.a) E += double(e.v);
            T *B = Hs + 9 * (find_slot(cia, r.s0, r.s1, b) - sb);
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
    }

    T *B = Hs + 9 * (dslot - sb);
#pragma unroll
    for (int i = 0; i < 9; ++i) B[i] = D[i];
#pragma unroll
    for (int c = 0; c < 3; ++c) g[int64_t(r.a) * 3 + c] = G[c];
    return E;
}

template <typename T>
__global__ void __launch_bounds__(kRowThreads)
k_eval_rows(RowArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
            EnergySink esink)
{
    extern __shared__ __align__(16) unsigned char smem[];
    T *stage = reinterpret_cast<T *>(smem);
    const int act = A.state->active;
    const int32_t *rpa = A.pat.rp[act];
    const int32_t *cia = A.pat.ci[act];
    const uint32_t *ib = A.pat.ib[act];
    int c0, c1;
    chunk_range(A.nchunk, c0, c1);
    double eacc = 0.0;
    for (int c = c0; c < c1; ++c) {
        const int32_t v0 = A.chunk[c].v0, nrows = A.chunk[c].nown;
        const int32_t sb = rpa[v0];
        const int32_t nblk = rpa[v0 + nrows] - sb;
        // The insertion check keeps every chunk within the staging capacity;
        // a chunk that does not fit is never written.
        const bool fits = nblk <= A.lds_blocks;
        const int pad = stage_pad<T>(int64_t(sb) * 9);
        T *Hs = stage + pad;
        if (fits && int(threadIdx.x) < nrows) {
            Row<T> r;
            r.a = v0 + threadIdx.x;
            r.s0 = rpa[r.a];
            r.s1 = rpa[r.a + 1];
            r.kb0 = A.rp0[r.a];
#pragma unroll
            for (int k = 0; k < 3; ++k) r.xa[k] = x[int64_t(r.a) * 3 + k];
            eacc += eval_row(A, act, cia, ib, r, sb, Hs, x, g);
        }
        __syncthreads();
        if (fits) stream_out<kRowThreads>(hv + int64_t(sb) * 9, Hs, nblk * 9, pad);
        __syncthreads();
    }
    finish_energy<kRowThreads>(esink, block_sum<kRowThreads>(eacc, nullptr), nullptr);
}

// ---------------------------------------------------------------------------
// Matrix-free Hessian-vector product, y_a = sum over the row's terms of
// H_ab v_b, with the local Hessians formed in registers and never stored.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kRowThreads)
k_hvp_rows(RowArgs<T> A, const T *__restrict__ x, const T *__restrict__ v, T *__restrict__ y)
{
    const int act = A.state->active;
    const int32_t *rpa = A.pat.rp[act];
    const uint32_t *ib = A.pat.ib[act];
    int c0, c1;
    chunk_range(A.nchunk, c0, c1);
    for (int c = c0; c < c1; ++c) {
        const int32_t v0 = A.chunk[c].v0, nrows = A.chunk[c].nown;
        if (int(threadIdx.x) >= nrows) continue;
        Row<T> r;
        r.a = v0 + threadIdx.x;
        r.s0 = rpa[r.a];
        r.s1 = rpa[r.a + 1];
        r.kb0 = A.rp0[r.a];
        T va[3], Y[3] = {T(0), T(0), T(0)};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            r.xa[k] = x[int64_t(r.a) * 3 + k];
            va[k] = v[int64_t(r.a) * 3 + k];
        }
        // K (v_a - v_b) for the two-vertex term with local Hessian K.
        auto add_kv = [&](const Dual2<T, 3> &e, int32_t b) {
            T dv[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) dv[k] = va[k] - v[int64_t(b) * 3 + k];
#pragma unroll
            for (int i = 0; i < 3; ++i)
                Y[i] += e.hess(i, 0) * dv[0] + e.hess(i, 1) * dv[1] + e.hess(i, 2) * dv[2];
        };
        for_each_slot(A, r, act, ib, [&](int32_t, int32_t kb, int32_t b, T L) {
            if (kb < 0 || b == r.a || !(L >= T(0))) return;
            Dual2<T, 3> d[3];
#pragma unroll
            for (int k = 0; k < 3; ++k)
                d[k] = Dual2<T, 3>::var(r.xa[k] - x[int64_t(b) * 3 + k], k);
            add_kv(spring_energy(d, L, A.k), b);
        });
        if (A.inertia_on) {
#pragma unroll
            for (int k = 0; k < 3; ++k) Y[k] += A.c * va[k];
        }
        if (act != 0) {
            const int32_t *pp = A.pat.pinc_ptr[act];
            const int32_t *pl = A.pat.pinc[act];
            const int32_t *prs = A.pat.pairs[act];
            for (int32_t k = pp[r.a]; k < pp[r.a + 1]; ++k) {
                const int32_t q = pl[k];
                const int32_t i0 = prs[2 * q], i1 = prs[2 * q + 1];
                const int32_t b = i0 == r.a ? i1 : i0;
                T dz[3];
#pragma unroll
                for (int cc = 0; cc < 3; ++cc) dz[cc] = r.xa[cc] - x[int64_t(b) * 3 + cc];
                const T l2 = dz[0] * dz[0] + dz[1] * dz[1] + dz[2] * dz[2];
                if (!(l2 < A.dhat * A.dhat)) continue;
                Dual2<T, 3> d[3];
#pragma unroll
                for (int cc = 0; cc < 3; ++cc) d[cc] = Dual2<T, 3>::var(dz[cc], cc);
                add_kv(barrier_energy(d, A.kappa, A.dhat), b);
            }
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) y[int64_t(r.a) * 3 + k] = Y[k];
    }
}

}  // namespace

template <typename T>
int rows_lds_bytes(int lds_blocks)
{
    // the staging slice plus up to 16 bytes of alignment padding in front
    return int(((int64_t(lds_blocks) * 9 * int64_t(sizeof(T)) + 16) + 15) & ~int64_t(15));
}

template <typename T>
hipError_t rows_grid(int lds_blocks, int nchunk, int *grid_eval, int *grid_hvp)
{
    int dev = 0, cus = 0, occ_e = 0, occ_h = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_e, k_eval_rows<T>, kRowThreads,
                                                         rows_lds_bytes<T>(lds_blocks));
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_h, k_hvp_rows<T>, kRowThreads, 0);
    if (e != hipSuccess) return e;
    auto clamp = [&](int occ) {
        const int64_t full = int64_t(cus > 0 ? cus : 1) * (occ > 0 ? occ : 1);
        const int64_t g = nchunk < full ? nchunk : full;
        return int(g < 1 ? 1 : g);
    };
    *grid_eval = clamp(occ_e);
    *grid_hvp = clamp(occ_h);
    return hipSuccess;
}

template <typename T>
hipError_t launch_eval_rows(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                            int grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_eval_rows<T>), dim3(grid), dim3(kRowThreads),
                       rows_lds_bytes<T>(a.lds_blocks), s, a, x, g, hv, es);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hvp_rows(const RowArgs<T> &a, const T *x, const T *v, T *y, int grid,
                           hipStream_t s)
{
    hipLaunchKernelGGL((k_hvp_rows<T>), dim3(grid), dim3(kRowThreads), 0, s, a, x, v, y);
    return hipGetLastError();
}

#define LAD_ROWS_INST(T)                                                                          \
    template int rows_lds_bytes<T>(int);                                                          \
    template hipError_t rows_grid<T>(int, int, int *, int *);                                     \
    template hipError_t launch_eval_rows<T>(const RowArgs<T> &, const T *, T *, T *, EnergySink,  \
                                            int, hipStream_t);                                    \
    template hipError_t launch_hvp_rows<T>(const RowArgs<T> &, const T *, const T *, T *, int,    \
                                           hipStream_t);
LAD_ROWS_INST(float)
LAD_ROWS_INST(double)

}  // namespace lad
