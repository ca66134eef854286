// lad_vf.hip -- vertex-face contact elements, one thread per contact.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", section "Method" (element-level forward mode: each term is
// evaluated once on seeded inputs, its local gradient and Hessian come out
// of the same pass) and key design 4 (vertex-face interactions beside the
// vertex-vertex ones).
//
// A point-triangle term couples four vertices, so its row-owner evaluation
// would repeat the 9-variable second-order pass in each of the four rows
// (and hold a 55-value dual number per intermediate in every row kernel).
// Instead the term is evaluated once here, in its own thread, and the row
// kernels add the strip that belongs to their row:
//   k_vf_eval  energy, gradient and Hessian in the 12 vertex variables
//              (contact vertex p, then the face's t0, t1, t2);
//   k_vf_hvp   the 12-vector H_e u_e for the direction u.
// Results are stored per contact vertex m as the strip its row reads
// (contiguous, so a row takes it in a few 16-byte loads), together with the
// contact's vertex ids and, for the explicit Hessian, the block offsets of
// the contact's four vertices in each of the four rows: a touched row then
// needs no search.  Contacts are read from the active pattern buffer (the
// rows they touch have complete columns there); the grid walks
// [0, nvf[active]) with a stride loop.
//
// Both kernels work in fp64 whatever the storage type: the positions (and
// the direction) are widened on load and only the stored strips are rounded
// to the context's type.  A contact whose face has been squeezed into a
// sliver (edges of very different lengths) loses most of its significant
// digits in the face normal and in (t0 - p) . n, which fp32 cannot afford;
// there are only a few contacts per step, so the wider arithmetic costs
// little next to the row kernels.
#include <hip/hip_runtime.h>

#include "contact_vf.h"
#include "dual2.h"
#include "lad_internal.h"

namespace lad {

namespace {

constexpr int kVfThreads = 64;

constexpr int kScan = 8;  // columns of a row matched per step

// Vertex ids (p, t0, t1, t2) and positions of contact e.
template <typename T>
__device__ __forceinline__ void vf_load(const RowArgs<T> &A, int act, int32_t e,
                                        const T *__restrict__ x, int32_t w[4], double xp[3],
                                        double xt[3][3])
{
    w[0] = A.pat.vf[act][2 * int64_t(e)];
    const int32_t f = A.pat.vf[act][2 * int64_t(e) + 1];
#pragma unroll
    for (int i = 0; i < 3; ++i) w[1 + i] = A.pat.faces[3 * int64_t(f) + i];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        xp[c] = double(x[int64_t(w[0]) * 3 + c]);
#pragma unroll
        for (int i = 0; i < 3; ++i) xt[i][c] = double(x[int64_t(w[1 + i]) * 3 + c]);
    }
}

template <typename T>
__global__ void __launch_bounds__(kVfThreads)
k_vf_eval(RowArgs<T> A, const T *__restrict__ x)
{
    const int act = A.state->active;
    if (act == 0) return;
    const int32_t n = A.state->nvf[act];
    const int32_t *rp = A.pat.rp[act], *ci = A.pat.ci[act];
    for (int32_t e = int32_t(blockIdx.x * kVfThreads + threadIdx.x); e < n;
         e += int32_t(gridDim.x) * kVfThreads) {
        int32_t w[4];
        double xp[3], xt[3][3];
        vf_load(A, act, e, x, w, xp, xt);
        // the four rows' block offsets of the contact's four vertices: the
        // rows are scanned kScan columns at a time, all four rows' loads of a
        // window issued together and matched in registers
        int32_t s0[4], len[4], off[4][4];
#pragma unroll
        for (int li = 0; li < 4; ++li) {
            s0[li] = rp[w[li]];
            len[li] = rp[w[li] + 1] - s0[li];
#pragma unroll
            for (int m = 0; m < 4; ++m) off[li][m] = 0;
        }
        for (int32_t base = 0;; base += kScan) {
            bool more = false;
#pragma unroll
            for (int li = 0; li < 4; ++li) {
                int32_t col[kScan];
#pragma unroll
                for (int k = 0; k < kScan; ++k)
                    col[k] = base + k < len[li] ? ci[s0[li] + base + k] : -1;
#pragma unroll
                for (int k = 0; k < kScan; ++k)
#pragma unroll
                    for (int m = 0; m < 4; ++m) off[li][m] = col[k] == w[m] ? base + k : off[li][m];
                more |= base + kScan < len[li];
            }
            if (!more) break;
        }
#pragma unroll
        for (int li = 0; li < 4; ++li) {
            *reinterpret_cast<int4 *>(A.vf_slots + (4 * int64_t(e) + li) * 4) =
                make_int4(off[li][0], off[li][1], off[li][2], off[li][3]);
            A.vf_ids[4 * int64_t(e) + li] = w[li];
        }
        T *L[4];
#pragma unroll
        for (int li = 0; li < 4; ++li) L[li] = A.vf_eval + (4 * int64_t(e) + li) * kVfStrip;
        const int region = vf_region(xp, xt[0], xt[1], xt[2]);
        Dual2<double, 9> z[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int c = 0; c < 3; ++c)
                z[3 * i + c] = Dual2<double, 9>::var(xt[i][c] - xp[c], 3 * i + c);
        const Dual2<double, 9> d = vf_distance(z, region);
        const double dhat = double(A.dhat);
        if (!(d.v < dhat)) {  // outside the barrier's support: an all-zero term
#pragma unroll
            for (int li = 0; li < 4; ++li)
                for (int c = 0; c < kVfStrip; ++c) L[li][c] = T(0);
            continue;
        }
        const Dual2<double, 9> en = barrier_of_distance(d, double(A.kappa), dhat);
        // energy in the contact vertex's strip; gradient: d/dt_i = d/dz_i,
        // d/dp = -sum_i d/dz_i
        L[0][0] = T(en.v);
#pragma unroll
        for (int i = 0; i < 3; ++i) L[1 + i][0] = T(0);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            double gp = 0.0;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                gp -= en.g[3 * i + c];
                L[1 + i][1 + c] = T(en.g[3 * i + c]);
            }
            L[0][1 + c] = T(gp);
        }
        // Hessian rows over the columns (p, t0, t1, t2) x coordinate:
        //   (t_i, t_j) = Hz_ij,  (t_i, p) = -sum_j Hz_ij,
        //   (p, t_j) = -sum_i Hz_ij,  (p, p) = sum_ij Hz_ij
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                double pp = 0.0;
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    double pj = 0.0;
#pragma unroll
                    for (int i = 0; i < 3; ++i) pj -= en.hess(3 * i + r, 3 * j + c);
                    L[0][kVfHessOff + 12 * r + 3 * (1 + j) + c] = T(pj);
                    pp -= pj;
                }
                L[0][kVfHessOff + 12 * r + c] = T(pp);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    double ip = 0.0;
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        const double h = en.hess(3 * i + r, 3 * j + c);
                        L[1 + i][kVfHessOff + 12 * r + 3 * (1 + j) + c] = T(h);
                        ip -= h;
                    }
                    L[1 + i][kVfHessOff + 12 * r + c] = T(ip);
                }
            }
    }
}

// With st set (Newton-CG), nothing is done once the solve has ended.
template <typename T>
__global__ void __launch_bounds__(kVfThreads)
k_vf_hvp(RowArgs<T> A, const T *__restrict__ x, const T *__restrict__ u, const CgState *st)
{
    if (st && st->stop) return;
    const int act = A.state->active;
    if (act == 0) return;
    const int32_t n = A.state->nvf[act];
    for (int32_t e = int32_t(blockIdx.x * kVfThreads + threadIdx.x); e < n;
         e += int32_t(gridDim.x) * kVfThreads) {
        int32_t w[4];
        double xp[3], xt[3][3], up[3], ut[3][3];
        vf_load(A, act, e, x, w, xp, xt);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            up[c] = double(u[int64_t(w[0]) * 3 + c]);
#pragma unroll
            for (int i = 0; i < 3; ++i) ut[i][c] = double(u[int64_t(w[1 + i]) * 3 + c]);
        }
#pragma unroll
        for (int li = 0; li < 4; ++li) A.vf_ids[4 * int64_t(e) + li] = w[li];
        T *L = A.vf_hvp + 4 * int64_t(e) * kVfHvpStrip;
        const int region = vf_region(xp, xt[0], xt[1], xt[2]);
        // z_i = t_i - p seeded with the matching direction u_(t_i) - u_p
        DualHv<double, 9> z[9];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int c = 0; c < 3; ++c)
                z[3 * i + c] =
                    DualHv<double, 9>::var(xt[i][c] - xp[c], 3 * i + c, ut[i][c] - up[c]);
        const DualHv<double, 9> d = vf_distance(z, region);
        const double dhat = double(A.dhat);
        if (!(d.v < dhat)) {
            for (int c = 0; c < 4 * kVfHvpStrip; ++c) L[c] = T(0);
            continue;
        }
        const DualHv<double, 9> en = barrier_of_distance(d, double(A.kappa), dhat);
        // gt = Hz (u_t - u_p) in z; mapped as the gradient is
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            double yp = 0.0;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                yp -= en.gt[3 * i + c];
                L[(1 + i) * kVfHvpStrip + c] = T(en.gt[3 * i + c]);
            }
            L[c] = T(yp);
        }
#pragma unroll
        for (int li = 0; li < 4; ++li) L[li * kVfHvpStrip + 3] = T(0);
    }
}

int vf_grid(int32_t cap)
{
    const int64_t g = (int64_t(cap) + kVfThreads - 1) / kVfThreads;
    return int(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

template <typename T>
hipError_t launch_vf_eval(const RowArgs<T> &a, const T *x, hipStream_t s)
{
    if (!a.pat.vf[1] || !a.pat.vf[2] || !a.pat.faces || !a.vf_eval || !a.vf_ids ||
        !a.vf_slots || !a.pat.rp[1] || !a.pat.rp[2] || !a.pat.ci[1] || !a.pat.ci[2] ||
        a.vf_stride <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_vf_eval<T>, dim3(vf_grid(a.vf_stride)), dim3(kVfThreads), 0, s, a, x);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_vf_hvp(const RowArgs<T> &a, const T *x, const T *u, const CgState *st,
                         hipStream_t s)
{
    if (!a.pat.vf[1] || !a.pat.vf[2] || !a.pat.faces || !a.vf_hvp || !a.vf_ids ||
        a.vf_stride <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_vf_hvp<T>, dim3(vf_grid(a.vf_stride)), dim3(kVfThreads), 0, s, a, x, u,
                       st);
    return hipGetLastError();
}

template hipError_t launch_vf_eval<float>(const RowArgs<float> &, const float *, hipStream_t);
template hipError_t launch_vf_eval<double>(const RowArgs<double> &, const double *, hipStream_t);
template hipError_t launch_vf_hvp<float>(const RowArgs<float> &, const float *, const float *,
                                         const CgState *, hipStream_t);
template hipError_t launch_vf_hvp<double>(const RowArgs<double> &, const double *, const double *,
                                          const CgState *, hipStream_t);

}  // namespace lad
