// lad_eval.hip -- per-patch evaluation, differentiation and assembly on
// gfx950.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations":
//   * key design 1: per-element forward-mode AD, every intermediate in
//     registers or on-chip memory; global traffic is one read of the mesh
//     and one write of the final sparse derivatives;
//   * key design 2: one workgroup per patch, patch-local staging of
//     positions (owned + ribbon vertices) in LDS;
//   * section "Method": g = sum_j S_j^T g_j, H = sum_j S_j^T H_j S_j, plus the
//     matrix-free Hessian-vector product.
//
// gfx950 design: a patch owns a contiguous range of rows, so its whole slice
// of the block-CSR value array is accumulated in LDS (plain adds in colour
// phases, or LDS atomics) and then streamed to HBM once with 16-byte stores:
// nothing in HBM is zero-filled, read back or updated atomically, and the
// only HBM writes are the final values.  The element-once assembly instead
// sends each element's blocks in other patches' rows to HBM as global
// atomics (the page's own scheme, kept for comparison).
#include "dual2.h"
#include "energies.h"
#include "lad_device.h"
#include "lad_internal.h"

namespace lad {

namespace {

constexpr int kWaves = kThreads / 64;

template <bool ATOMIC, typename T>
__device__ __forceinline__ void lds_add(T *p, T v)
{
    if constexpr (ATOMIC)
        __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else
        *p += v;
}

// Add s * K (3x3 symmetric, packed in a Dual2<T,3> Hessian) into block B.
template <bool ATOMIC, typename T>
__device__ __forceinline__ void add_block3(T *B, const Dual2<T, 3> &e, T s)
{
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) lds_add<ATOMIC>(B + 3 * r + c, s * e.hess(r, c));
}

// Global float atomic add (the hardware instruction; relaxed, device scope).
template <typename T>
__device__ __forceinline__ void global_add(T *p, T v)
{
    (void)unsafeAtomicAdd(p, v);
}

// Element-once patches: where an element's contributions to the rows of
// other patches go.  rib: the patch's ribbon list (local id nown + i is
// vertex rib[i]); hv, g: the global value array and gradient.
template <typename T>
struct Foreign {
    T *hv;
    T *g;
    const int32_t *rib;
};

// ---------------------------------------------------------------------------
// Element bodies.  xs: staged positions (local ids); nown: owned count.
// ---------------------------------------------------------------------------

// Two-vertex spring, differentiated in z = x_a - x_b.  With K = d2f/dz2 and
// q = df/dz the element blocks are g = [q, -q], H = [[K, -K], [-K, K]].
//
// GA (element-once patches): the record is this element's only one, so its
// energy always counts here, and a non-owned endpoint f gets its blocks
// (f, f), (f, other) = gb[0], gb[1] and its gradient entries by global
// atomics.
template <bool ATOMIC, bool GA, typename T>
__device__ __forceinline__ void spring_eval(const SpringRec rec, T rest, T k, const T *xs,
                                            T *H, T *gs, const uint16_t *dtab, int nown,
                                            double &eacc, const Foreign<T> &fo = {},
                                            const int32_t *gb = nullptr)
{
    const int la = rec.lab & 0xFFFF, lb = rec.lab >> 16;
    Dual2<T, 3> d[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(xs[3 * la + c] - xs[3 * lb + c], c);
    const Dual2<T, 3> e = spring_energy(d, rest, k);
    if (GA || la < nown) eacc += double(e.v);
    if (la < nown) {
#pragma unroll
        for (int c = 0; c < 3; ++c) lds_add<ATOMIC>(gs + 3 * la + c, e.g[c]);
        add_block3<ATOMIC>(H + 9 * dtab[la], e, T(1));
        add_block3<ATOMIC>(H + 9 * (rec.blk & 0xFFFF), e, T(-1));
    }
    if (lb < nown) {
#pragma unroll
        for (int c = 0; c < 3; ++c) lds_add<ATOMIC>(gs + 3 * lb + c, -e.g[c]);
        add_block3<ATOMIC>(H + 9 * dtab[lb], e, T(1));
        add_block3<ATOMIC>(H + 9 * (rec.blk >> 16), e, T(-1));
    }
    if constexpr (GA) {
        if (la >= nown || lb >= nown) {
            const bool fa = la >= nown;
            const int64_t f = fo.rib[(fa ? la : lb) - nown];
            const T sg = fa ? T(1) : T(-1);
            T *Bff = fo.hv + int64_t(gb[0]) * 9;
            T *Bfo = fo.hv + int64_t(gb[1]) * 9;
#pragma unroll
            for (int c = 0; c < 3; ++c) global_add(fo.g + 3 * f + c, sg * e.g[c]);
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    global_add(Bff + 3 * r + c, e.hess(r, c));
                    global_add(Bfo + 3 * r + c, -e.hess(r, c));
                }
        }
    }
}

// Face: F = [x1-x0, x2-x0] M (M = Dm^-1), so dF[s][c]/dx_v[s] = w[v][c] with
// w1 = M row 0, w2 = M row 1, w0 = -(w1 + w2).  The 3x3 block (v, u) is
// B[s][t] = sum_{c,c'} w[v][c] w[u][c'] d2E/dF[s][c]dF[t][c'].
template <typename T>
struct FaceLocal {
    Dual2<T, 6> e;
    T w[3][2];
};

template <typename T>
__device__ __forceinline__ void face_local(const FaceRec &rec, const T *dm, T area, const T *xs,
                                           FaceLocal<T> &out)
{
    const T m00 = dm[0], m01 = dm[1], m10 = dm[2], m11 = dm[3];
    const T *x0 = xs + 3 * rec.l[0];
    const T *x1 = xs + 3 * rec.l[1];
    const T *x2 = xs + 3 * rec.l[2];
    Dual2<T, 6> F[6];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const T d0 = x1[r] - x0[r], d1 = x2[r] - x0[r];
        F[2 * r + 0] = Dual2<T, 6>::var(d0 * m00 + d1 * m10, 2 * r + 0);
        F[2 * r + 1] = Dual2<T, 6>::var(d0 * m01 + d1 * m11, 2 * r + 1);
    }
    out.e = face_energy(F, area);
    out.w[1][0] = m00;
    out.w[1][1] = m01;
    out.w[2][0] = m10;
    out.w[2][1] = m11;
    out.w[0][0] = -(m00 + m10);
    out.w[0][1] = -(m01 + m11);
}

// GA (element-once patches): energy always counts; the rows of non-owned
// vertices v get their blocks (v, u) = gb[3 v + u] and gradient entries by
// global atomics.
template <bool ATOMIC, bool GA, typename T>
__device__ __forceinline__ void face_eval(const FaceRec rec, const T *dm, T area, const T *xs,
                                          T *H, T *gs, int nown, double &eacc,
                                          const Foreign<T> &fo = {}, const int32_t *gb = nullptr)
{
    FaceLocal<T> fl;
    face_local(rec, dm, area, xs, fl);
    const Dual2<T, 6> &e = fl.e;
    if (GA || rec.l[0] < nown) eacc += double(e.v);
#pragma unroll
    for (int v = 0; v < 3; ++v) {
        const bool own = rec.l[v] < nown;
        if (!GA && !own) continue;
        T *gv = own ? gs + 3 * rec.l[v] : fo.g + 3 * int64_t(fo.rib[rec.l[v] - nown]);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const T gsv = fl.w[v][0] * e.g[2 * s] + fl.w[v][1] * e.g[2 * s + 1];
            if (own) lds_add<ATOMIC>(gv + s, gsv);
            else global_add(gv + s, gsv);
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            T *B = own ? H + 9 * rec.blk[3 * v + u] : fo.hv + int64_t(gb[3 * v + u]) * 9;
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    // (Q w_u) with Q = d2E/dF[s][.] dF[t][.]
                    const T q0 = e.hess(2 * s, 2 * t) * fl.w[u][0] +
                                 e.hess(2 * s, 2 * t + 1) * fl.w[u][1];
                    const T q1 = e.hess(2 * s + 1, 2 * t) * fl.w[u][0] +
                                 e.hess(2 * s + 1, 2 * t + 1) * fl.w[u][1];
                    const T bv = fl.w[v][0] * q0 + fl.w[v][1] * q1;
                    if (own) lds_add<ATOMIC>(B + 3 * s + t, bv);
                    else global_add(B + 3 * s + t, bv);
                }
        }
    }
}

// Flush of an element-once patch's LDS slice: entries of flagged units
// (blocks of 9 values, or vertices of 3; flag[] in LDS, one byte per unit)
// also receive other patches' atomics into slots zeroed beforehand, so they
// are added atomically (and skipped when this patch's part is zero); the
// rest are stored, in aligned 16-byte non-temporal vectors where no flagged
// unit touches the vector.  Same alignment contract as stream_out.
template <int NT, int UNIT, typename T>
__device__ __forceinline__ void flush_flagged(T *__restrict__ dst, const T *src, int n, int pad,
                                              const uint8_t *flag)
{
    constexpr int V = Vec<T>::n;
    using VT = typename Vec<T>::type;
    auto one = [&](int i) {
        const T val = src[i];
        if (flag[i / UNIT]) {
            if (val != T(0)) global_add(dst + i, val);
        } else {
            dst[i] = val;
        }
    };
    const int head = min(n, (V - pad) % V);
    for (int i = threadIdx.x; i < head; i += NT) one(i);
    const int nvec = (n - head) / V;
    VT *dv = reinterpret_cast<VT *>(dst + head);
    const VT *sv = reinterpret_cast<const VT *>(src + head);
    for (int i = threadIdx.x; i < nvec; i += NT) {
        const int e0 = head + V * i;
        if (flag[e0 / UNIT] | flag[(e0 + V - 1) / UNIT]) {
#pragma unroll
            for (int j = 0; j < V; ++j) one(e0 + j);
        } else {
            __builtin_nontemporal_store(sv[i], dv + i);
        }
    }
    for (int i = head + nvec * V + threadIdx.x; i < n; i += NT) one(i);
}

// ---------------------------------------------------------------------------
// Eval kernel: energy, gradient and Hessian block rows of one patch.
// ---------------------------------------------------------------------------
//
// MODE (PatchMode): kModeLdsAtomic and kModeColour evaluate every element
// touching an owned row and store the owned slice.  kModeBoundaryAtomic runs
// an element-once plan: elements are evaluated by one patch only, their
// contributions to other patches' rows go out as global atomics, and the
// owned entries that also receive such atomics (zeroed by a launch before
// this one; flagged per block and per vertex) are added, not stored.  That
// mode has no pairs, so the active pattern is the topology pattern.
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads)
k_eval_patch(PatchArgs<T> A, const T *__restrict__ x, T *__restrict__ g, T *__restrict__ hv,
             EnergySink esink)
{
    constexpr bool DET = MODE == kModeColour;
    constexpr bool GA = MODE == kModeBoundaryAtomic;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int V = Vec<T>::n;
    const int p = xcd_remap(blockIdx.x, gridDim.x);
    const PatchHdr h = A.hdr[p];
    const int tid = threadIdx.x;
    const int act = A.state->active;
    const int32_t *rpa = A.pat.rp[act];
    const int32_t ra0 = rpa[h.v0];
    const int32_t nact = rpa[h.v0 + h.nown] - ra0;
    const bool mapped = nact != h.nblk;

    // carve LDS (same order and sizes as lds_eval_bytes on the host)
    const int nloc = h.nown + h.nrib;
    int64_t off = 0;
    T *Hbase = reinterpret_cast<T *>(smem + off);
    off += dalign16((int64_t(h.nblk) * 9 + 4) * sizeof(T));
    T *gbase = reinterpret_cast<T *>(smem + off);
    off += dalign16((int64_t(h.nown) * 3 + 4) * sizeof(T));
    T *xs = reinterpret_cast<T *>(smem + off);
    off += dalign16(int64_t(nloc) * 3 * sizeof(T));
    uint16_t *dtab = reinterpret_cast<uint16_t *>(smem + off);
    off += dalign16(int64_t(h.nown) * 2);
    uint16_t *amap = reinterpret_cast<uint16_t *>(smem + off);
    off += dalign16(int64_t(h.amap_cap) * 2);
    double *red = reinterpret_cast<double *>(smem + off);

    const int hpad = mapped ? 0 : int((int64_t(ra0) * 9) % V);
    T *H = Hbase + hpad;
    const int gpad = int((int64_t(h.v0) * 3) % V);
    T *gs = gbase + gpad;

    // 1. zero the accumulators, stage positions (owned, then ribbon)
    for (int i = tid; i < h.nblk * 9; i += kThreads) H[i] = T(0);
    for (int i = tid; i < h.nown * 3; i += kThreads) gs[i] = T(0);
    const T *xo = x + int64_t(h.v0) * 3;
    for (int i = tid; i < h.nown * 3; i += kThreads) xs[i] = xo[i];
    for (int i = tid; i < h.nrib * 3; i += kThreads) {
        const int r = i / 3, c = i - 3 * r;
        xs[3 * h.nown + i] = x[int64_t(A.rib[h.rib_off + r]) * 3 + c];
    }
    for (int i = tid; i < h.nown; i += kThreads) dtab[i] = A.diag_rel[h.v0 + i];
    // element-once: boundary flags of the owned blocks, then of the owned
    // vertices, in the (otherwise unused) active-block map region, which
    // holds at least nblk + nown bytes
    uint8_t *bflag = reinterpret_cast<uint8_t *>(amap);
    uint8_t *vflag = bflag + h.nblk;
    if constexpr (GA) {
        for (int i = tid; i < h.nblk; i += kThreads) bflag[i] = A.blk_flag[h.blk0 + i];
        for (int i = tid; i < h.nown; i += kThreads) vflag[i] = A.vtx_flag[h.v0 + i];
    }
    const Foreign<T> fo{hv, g, A.rib + h.rib_off};
    __syncthreads();

    double eacc = 0.0;
    // 2. inertia: one owned vertex per thread, first writer of its blocks
    if (A.inertia_on) {
        for (int i = tid; i < h.nown; i += kThreads) {
            const T *xt = A.x_tilde + int64_t(h.v0 + i) * 3;
            Dual2<T, 3> z[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) z[c] = Dual2<T, 3>::var(xs[3 * i + c] - xt[c], c);
            const Dual2<T, 3> e = inertia_energy(z, A.c);
            eacc += double(e.v);
#pragma unroll
            for (int c = 0; c < 3; ++c) gs[3 * i + c] += e.g[c];
            add_block3<false>(H + 9 * dtab[i], e, T(1));
        }
        __syncthreads();
    }

    // 3. springs
    if (A.springs_on && h.nspr > 0) {
        const SpringRec *R = A.spr + h.spr_off;
        const T *L = A.spr_rest + h.spr_off;
        if constexpr (DET) {
            const int32_t *cb = A.col_bounds + h.col_off;
            for (int c = 0; c < h.nspr_col; ++c) {
                for (int e = cb[c] + tid; e < cb[c + 1]; e += kThreads)
                    spring_eval<false, false>(R[e], L[e], A.k, xs, H, gs, dtab, h.nown, eacc);
                __syncthreads();
            }
        } else {
            const int32_t *gb = GA ? A.spr_gblk + 2 * int64_t(h.spr_off) : nullptr;
            for (int e = tid; e < h.nspr; e += kThreads)
                spring_eval<true, GA>(R[e], L[e], A.k, xs, H, gs, dtab, h.nown, eacc, fo,
                                      GA ? gb + 2 * e : nullptr);
        }
    }

    // 4. faces
    if (A.faces_on && h.nfac > 0) {
        const FaceRec *R = A.fac + h.fac_off;
        const T *dm = A.fac_dm + int64_t(h.fac_off) * 4;
        const T *ar = A.fac_area + h.fac_off;
        if constexpr (DET) {
            const int32_t *cb = A.col_bounds + h.col_off + (h.nspr_col ? h.nspr_col + 1 : 0);
            for (int c = 0; c < h.nfac_col; ++c) {
                for (int e = cb[c] + tid; e < cb[c + 1]; e += kThreads)
                    face_eval<false, false>(R[e], dm + 4 * e, ar[e], xs, H, gs, h.nown, eacc);
                __syncthreads();
            }
        } else {
            const int32_t *gb = GA ? A.fac_gblk + 9 * int64_t(h.fac_off) : nullptr;
            for (int e = tid; e < h.nfac; e += kThreads)
                face_eval<true, GA>(R[e], dm + 4 * e, ar[e], xs, H, gs, h.nown, eacc, fo,
                                    GA ? gb + 9 * e : nullptr);
        }
    }
    __syncthreads();

    // 5. write the owned slice of the active pattern's value array
    T *dst = hv + int64_t(ra0) * 9;
    if constexpr (GA) {
        flush_flagged<kThreads, 9>(dst, H, h.nblk * 9, hpad, bflag);
        flush_flagged<kThreads, 3>(g + int64_t(h.v0) * 3, gs, h.nown * 3, gpad, vflag);
        store_energy(esink, block_sum<kThreads>(eacc, red));
        return;
    }
    if (!mapped) {
        stream_out<kThreads>(dst, H, h.nblk * 9, hpad);
    } else if (nact <= h.amap_cap) {
        // pairs inserted blocks into these rows: map every active block to
        // its base block, or to zero for an inserted one (a column that the
        // topology row does not hold; both rows are sorted)
        const int32_t *rp0 = A.pat.rp[0];
        const int32_t *ci0 = A.pat.ci[0];
        const int32_t *cia = A.pat.ci[act];
        for (int i = tid; i < h.nown; i += kThreads) {
            const int32_t a0 = rpa[h.v0 + i] - ra0, a1 = rpa[h.v0 + i + 1] - ra0;
            int32_t b = rp0[h.v0 + i];
            const int32_t bend = rp0[h.v0 + i + 1];
            for (int32_t j = a0; j < a1; ++j) {
                const bool base = b < bend && ci0[b] == cia[ra0 + j];
                amap[j] = base ? uint16_t(b - h.blk0) : kNone;
                b += base ? 1 : 0;
            }
        }
        __syncthreads();
        for (int i = tid; i < nact * 9; i += kThreads) {
            const int j = i / 9, c = i - 9 * j;
            const uint16_t m = amap[j];
            dst[i] = (m == kNone) ? T(0) : H[9 * m + c];
        }
    }
    stream_out<kThreads>(g + int64_t(h.v0) * 3, gs, h.nown * 3, gpad);

    store_energy(esink, block_sum<kThreads>(eacc, red));
}

// ---------------------------------------------------------------------------
// HVP kernel: y = H(x) v for the owned rows of one patch, H never formed.
// ---------------------------------------------------------------------------
// MODE as for k_eval_patch; with kModeBoundaryAtomic the y entries of
// flagged vertices are zeroed by an earlier launch and added to.
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads)
k_hvp_patch(PatchArgs<T> A, const T *__restrict__ x, const T *__restrict__ v, T *__restrict__ y)
{
    constexpr bool DET = MODE == kModeColour;
    constexpr bool GA = MODE == kModeBoundaryAtomic;
    extern __shared__ __align__(16) unsigned char smem[];
    const int p = xcd_remap(blockIdx.x, gridDim.x);
    const PatchHdr h = A.hdr[p];
    const int tid = threadIdx.x;
    const int nloc = h.nown + h.nrib;
    int64_t off = 0;
    T *xs = reinterpret_cast<T *>(smem + off);
    off += dalign16(int64_t(nloc) * 3 * sizeof(T));
    T *vs = reinterpret_cast<T *>(smem + off);
    off += dalign16(int64_t(nloc) * 3 * sizeof(T));
    T *ys = reinterpret_cast<T *>(smem + off);

    const T *xo = x + int64_t(h.v0) * 3;
    const T *vo = v + int64_t(h.v0) * 3;
    for (int i = tid; i < h.nown * 3; i += kThreads) {
        xs[i] = xo[i];
        vs[i] = vo[i];
        ys[i] = T(0);
    }
    for (int i = tid; i < h.nrib * 3; i += kThreads) {
        const int r = i / 3, c = i - 3 * r;
        const int64_t gi = int64_t(A.rib[h.rib_off + r]) * 3 + c;
        xs[3 * h.nown + i] = x[gi];
        vs[3 * h.nown + i] = v[gi];
    }
    __syncthreads();

    if (A.inertia_on) {
        for (int i = tid; i < h.nown * 3; i += kThreads) ys[i] += A.c * vs[i];
        __syncthreads();
    }

    // y entries of a local vertex: LDS for owned ones, HBM (global atomics)
    // for the ribbon vertices of an element-once patch
    const int32_t *rib = A.rib + h.rib_off;
    auto y_add = [&](int l, int r, T val, auto atomic_tag) {
        constexpr bool AT = decltype(atomic_tag)::value;
        if (l < h.nown) lds_add<AT>(ys + 3 * l + r, val);
        else if constexpr (GA) global_add(y + 3 * int64_t(rib[l - h.nown]) + r, val);
    };
    auto spring_hvp = [&](const SpringRec rec, T rest, auto atomic_tag) {
        const int la = rec.lab & 0xFFFF, lb = rec.lab >> 16;
        Dual2<T, 3> d[3];
        T dv[3];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            d[c] = Dual2<T, 3>::var(xs[3 * la + c] - xs[3 * lb + c], c);
            dv[c] = vs[3 * la + c] - vs[3 * lb + c];
        }
        const Dual2<T, 3> e = spring_energy(d, rest, A.k);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const T kv = e.hess(r, 0) * dv[0] + e.hess(r, 1) * dv[1] + e.hess(r, 2) * dv[2];
            y_add(la, r, kv, atomic_tag);
            y_add(lb, r, -kv, atomic_tag);
        }
    };
    auto face_hvp = [&](const FaceRec rec, const T *dm, T area, auto atomic_tag) {
        FaceLocal<T> fl;
        face_local(rec, dm, area, xs, fl);
        // dF = B v_j, yF = (d2E/dF2) dF, y_v = B_v^T yF
        T dF[6];
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dF[2 * s + c] = fl.w[0][c] * vs[3 * rec.l[0] + s] +
                                fl.w[1][c] * vs[3 * rec.l[1] + s] +
                                fl.w[2][c] * vs[3 * rec.l[2] + s];
        T yF[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            T acc = T(0);
#pragma unroll
            for (int j = 0; j < 6; ++j) acc += fl.e.hess(i, j) * dF[j];
            yF[i] = acc;
        }
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int s = 0; s < 3; ++s)
                y_add(rec.l[u], s, fl.w[u][0] * yF[2 * s] + fl.w[u][1] * yF[2 * s + 1],
                      atomic_tag);
    };
    using AtomicTag = std::integral_constant<bool, !DET>;

    if (A.springs_on && h.nspr > 0) {
        const SpringRec *R = A.spr + h.spr_off;
        const T *L = A.spr_rest + h.spr_off;
        if constexpr (DET) {
            const int32_t *cb = A.col_bounds + h.col_off;
            for (int c = 0; c < h.nspr_col; ++c) {
                for (int e = cb[c] + tid; e < cb[c + 1]; e += kThreads)
                    spring_hvp(R[e], L[e], AtomicTag{});
                __syncthreads();
            }
        } else {
            for (int e = tid; e < h.nspr; e += kThreads) spring_hvp(R[e], L[e], AtomicTag{});
        }
    }
    if (A.faces_on && h.nfac > 0) {
        const FaceRec *R = A.fac + h.fac_off;
        const T *dm = A.fac_dm + int64_t(h.fac_off) * 4;
        const T *ar = A.fac_area + h.fac_off;
        if constexpr (DET) {
            const int32_t *cb = A.col_bounds + h.col_off + (h.nspr_col ? h.nspr_col + 1 : 0);
            for (int c = 0; c < h.nfac_col; ++c) {
                for (int e = cb[c] + tid; e < cb[c + 1]; e += kThreads)
                    face_hvp(R[e], dm + 4 * e, ar[e], AtomicTag{});
                __syncthreads();
            }
        } else {
            for (int e = tid; e < h.nfac; e += kThreads)
                face_hvp(R[e], dm + 4 * e, ar[e], AtomicTag{});
        }
    }
    __syncthreads();
    T *yo = y + int64_t(h.v0) * 3;
    if constexpr (GA) {
        const uint8_t *vflag = A.vtx_flag + h.v0;
        for (int i = tid; i < h.nown * 3; i += kThreads) {
            const T val = ys[i];
            if (vflag[i / 3]) {
                if (val != T(0)) global_add(yo + i, val);
            } else {
                yo[i] = val;
            }
        }
    } else {
        for (int i = tid; i < h.nown * 3; i += kThreads) yo[i] = ys[i];
    }
}

// Zero the slots that element-once patches add into (one thread per value).
template <typename T>
__global__ void __launch_bounds__(kThreads)
k_zero_boundary(const int32_t *__restrict__ bnd_blk, int32_t nb, const int32_t *__restrict__ bnd_vtx,
                int32_t nvb, T *__restrict__ hv, T *__restrict__ vec)
{
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t nh = hv ? 9 * int64_t(nb) : 0;
    if (i < nh) {
        hv[9 * int64_t(bnd_blk[i / 9]) + i % 9] = T(0);
    } else if (i - nh < 3 * int64_t(nvb)) {
        const int64_t j = i - nh;
        vec[3 * int64_t(bnd_vtx[j / 3]) + j % 3] = T(0);
    }
}

// ---------------------------------------------------------------------------
// Pair terms: row gather.  One thread per row that has pairs; it evaluates
// each of the row's pairs (in pair order) and adds the row's contributions,
// so every block and gradient entry has a single writer and the summation
// order is fixed.  Runs after the patch kernel on the same stream.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t find_col(const int32_t *ci, int32_t lo, int32_t hi, int32_t b)
{
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (ci[mid] < b) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <typename T, bool HVP>
__global__ void __launch_bounds__(kThreads)
k_pairs(const DevState *__restrict__ st, PatternBufs pat, const T *__restrict__ x,
        const T *__restrict__ v, T *__restrict__ out_vec, T *__restrict__ hv,
        EnergySink esink, T kappa, T dhat)
{
    __shared__ double red[kWaves];
    const int act = st->active;
    const int t = blockIdx.x * kThreads + threadIdx.x;
    double eacc = 0.0;
    if (act != 0 && t < 2 * st->np[act]) {
        const int32_t *pp = pat.pinc_ptr[act];
        const int32_t a = pat.pinc_row[act][t];
        if (t == pp[a]) {
            const int32_t *prs = pat.pairs[act];
            const int32_t *rp = pat.rp[act], *ci = pat.ci[act];
            const int32_t r0 = rp[a], r1 = rp[a + 1];
            T xa[3], ga[3] = {T(0), T(0), T(0)}, Kd[9] = {};
#pragma unroll
            for (int c = 0; c < 3; ++c) xa[c] = x[int64_t(a) * 3 + c];
            for (int32_t k = pp[a]; k < pp[a + 1]; ++k) {
                const int32_t q = pat.pinc[act][k];
                const int32_t i = prs[2 * q], j = prs[2 * q + 1];
                const int32_t b = (i == a) ? j : i;
                T dz[3];
#pragma unroll
                for (int c = 0; c < 3; ++c) dz[c] = xa[c] - x[int64_t(b) * 3 + c];
                const T l2 = dz[0] * dz[0] + dz[1] * dz[1] + dz[2] * dz[2];
                if (!(l2 < dhat * dhat)) continue;
                Dual2<T, 3> d[3];
#pragma unroll
                for (int c = 0; c < 3; ++c) d[c] = Dual2<T, 3>::var(dz[c], c);
                const Dual2<T, 3> e = barrier_energy(d, kappa, dhat);
                if (i == a) eacc += double(e.v);
                if constexpr (HVP) {
#pragma unroll
                    for (int r = 0; r < 3; ++r) {
                        T kv = T(0);
#pragma unroll
                        for (int c = 0; c < 3; ++c)
                            kv += e.hess(r, c) * (v[int64_t(a) * 3 + c] - v[int64_t(b) * 3 + c]);
                        ga[r] += kv;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 3; ++c) ga[c] += e.g[c];
#pragma unroll
                    for (int r = 0; r < 3; ++r)
#pragma unroll
                        for (int c = 0; c < 3; ++c) Kd[3 * r + c] += e.hess(r, c);
                    const int32_t kb = find_col(ci, r0, r1, b);
                    if (kb < r1 && ci[kb] == b) {
                        T *B = hv + int64_t(kb) * 9;
#pragma unroll
                        for (int r = 0; r < 3; ++r)
#pragma unroll
                            for (int c = 0; c < 3; ++c) B[3 * r + c] -= e.hess(r, c);
                    }
                }
            }
            if constexpr (!HVP) {
                const int32_t ka = find_col(ci, r0, r1, a);
                if (ka < r1 && ci[ka] == a) {
                    T *B = hv + int64_t(ka) * 9;
#pragma unroll
                    for (int r = 0; r < 9; ++r) B[r] += Kd[r];
                }
            }
#pragma unroll
            for (int c = 0; c < 3; ++c) out_vec[int64_t(a) * 3 + c] += ga[c];
        }
    }
    if constexpr (!HVP) store_energy(esink, block_sum<kThreads>(eacc, red));
}

// Sum of n partial energies in index order (one workgroup).
__global__ void __launch_bounds__(kThreads)
k_energy_reduce(const double *__restrict__ parts, int32_t n, double *__restrict__ out)
{
    // thread t adds parts t, t + kThreads, ... in that order; the loads of
    // a round go out together (indices clamped, extras dropped), so a few
    // thousand partials cost one or two memory round trips
    constexpr int kRound = 8;
    __shared__ double red[kWaves];
    double s = 0.0;
    for (int32_t base = 0; base < n; base += kThreads * kRound) {
        double v[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j)
            v[j] = parts[min(base + j * kThreads + int32_t(threadIdx.x), n - 1)];
#pragma unroll
        for (int j = 0; j < kRound; ++j)
            if (base + j * kThreads + int32_t(threadIdx.x) < n) s += v[j];
    }
    const double tot = block_sum<kThreads>(s, red);
    if (threadIdx.x == 0) *out = tot;
}

}  // namespace

namespace {

// NaN or +-inf, from the exponent bits of the values read as integers (the
// device code is compiled with finite-math assumptions, under which a test
// on a floating-point value may be folded away)
__device__ __forceinline__ bool nonfinite_bits(uint32_t u)
{
    return (u & 0x7f800000u) == 0x7f800000u;
}

__device__ __forceinline__ bool nonfinite_bits(unsigned long long u)
{
    const unsigned long long e = 0x7ff0000000000000ull;
    return (u & e) == e;
}

// U: the unsigned integer of the values' width.  One flag per workgroup,
// no ordering needed: the latch is an OR.
template <typename U>
__global__ void __launch_bounds__(kThreads)
k_check_finite(DevState *st, const unsigned long long *__restrict__ energy,
               const U *__restrict__ vec, int64_t nvec, const U *__restrict__ hv)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t t0 = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    bool bad = t0 == 0 && energy && nonfinite_bits(*energy);
    for (int64_t i = t0; i < nvec; i += stride) bad |= nonfinite_bits(vec[i]);
    if (hv) {
        const int64_t nh = 9 * int64_t(st->nnzb[st->active]);
        for (int64_t i = t0; i < nh; i += stride) bad |= nonfinite_bits(hv[i]);
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) atomicOr(&st->err_latched, 8);
}

}  // namespace

hipError_t launch_check_finite(DevState *st, const double *energy, const void *vec, int64_t nvec,
                               const void *hv, int es, hipStream_t s)
{
    const unsigned grid = 1024;
    const auto *e = reinterpret_cast<const unsigned long long *>(energy);
    if (es == 8)
        hipLaunchKernelGGL(k_check_finite<unsigned long long>, dim3(grid), dim3(kThreads), 0, s,
                           st, e, static_cast<const unsigned long long *>(vec), nvec,
                           static_cast<const unsigned long long *>(hv));
    else
        hipLaunchKernelGGL(k_check_finite<uint32_t>, dim3(grid), dim3(kThreads), 0, s, st, e,
                           static_cast<const uint32_t *>(vec), nvec,
                           static_cast<const uint32_t *>(hv));
    return hipGetLastError();
}

hipError_t launch_energy_reduce(const double *parts, int32_t n, double *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_energy_reduce, dim3(1), dim3(kThreads), 0, s, parts, n, out);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_eval(const PatchArgs<T> &a, const T *x, T *g, T *hv, EnergySink es, int mode,
                       int lds_bytes, hipStream_t s)
{
    if (a.npatch == 0) return hipSuccess;
    const dim3 grid(a.npatch), block(kThreads);
    if (mode == kModeColour)
        hipLaunchKernelGGL((k_eval_patch<T, kModeColour>), grid, block, lds_bytes, s, a, x, g, hv,
                           es);
    else if (mode == kModeBoundaryAtomic)
        hipLaunchKernelGGL((k_eval_patch<T, kModeBoundaryAtomic>), grid, block, lds_bytes, s, a, x,
                           g, hv, es);
    else
        hipLaunchKernelGGL((k_eval_patch<T, kModeLdsAtomic>), grid, block, lds_bytes, s, a, x, g,
                           hv, es);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hvp(const PatchArgs<T> &a, const T *x, const T *v, T *y, int mode,
                      int lds_bytes, hipStream_t s)
{
    if (a.npatch == 0) return hipSuccess;
    const dim3 grid(a.npatch), block(kThreads);
    if (mode == kModeColour)
        hipLaunchKernelGGL((k_hvp_patch<T, kModeColour>), grid, block, lds_bytes, s, a, x, v, y);
    else if (mode == kModeBoundaryAtomic)
        hipLaunchKernelGGL((k_hvp_patch<T, kModeBoundaryAtomic>), grid, block, lds_bytes, s, a, x,
                           v, y);
    else
        hipLaunchKernelGGL((k_hvp_patch<T, kModeLdsAtomic>), grid, block, lds_bytes, s, a, x, v,
                           y);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_zero_boundary(const int32_t *bnd_blk, int32_t nb, const int32_t *bnd_vtx,
                                int32_t nvb, T *hv, T *vec, hipStream_t s)
{
    const int64_t n = (hv ? 9 * int64_t(nb) : 0) + 3 * int64_t(nvb);
    if (n == 0) return hipSuccess;
    const int64_t grid = (n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_zero_boundary<T>, dim3(unsigned(grid)), dim3(kThreads), 0, s, bnd_blk,
                       nb, bnd_vtx, nvb, hv, vec);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_pairs_eval(const DevState *st, PatternBufs pat, const T *x, T *g, T *hv,
                             EnergySink es, int nblocks, T kappa, T dhat, hipStream_t s)
{
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_pairs<T, false>), dim3(nblocks), dim3(kThreads), 0, s, st, pat, x,
                       (const T *)nullptr, g, hv, es, kappa, dhat);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_pairs_hvp(const DevState *st, PatternBufs pat, const T *x, const T *v, T *y,
                            int nblocks, T kappa, T dhat, hipStream_t s)
{
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_pairs<T, true>), dim3(nblocks), dim3(kThreads), 0, s, st, pat, x, v, y,
                       (T *)nullptr, EnergySink{}, kappa, dhat);
    return hipGetLastError();
}

template <typename T>
static hipError_t raise_lds_limit(int bytes)
{
    const void *fns[] = {(const void *)k_eval_patch<T, kModeLdsAtomic>,
                         (const void *)k_eval_patch<T, kModeColour>,
                         (const void *)k_eval_patch<T, kModeBoundaryAtomic>,
                         (const void *)k_hvp_patch<T, kModeLdsAtomic>,
                         (const void *)k_hvp_patch<T, kModeColour>,
                         (const void *)k_hvp_patch<T, kModeBoundaryAtomic>};
    for (const void *f : fns) {
        const hipError_t e =
            hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t raise_lds_limits(int bytes)
{
    const hipError_t e = raise_lds_limit<float>(bytes);
    return e == hipSuccess ? raise_lds_limit<double>(bytes) : e;
}

#define LAD_INST(T)                                                                                \
    template hipError_t launch_eval<T>(const PatchArgs<T> &, const T *, T *, T *, EnergySink, int, \
                                       int, hipStream_t);                                          \
    template hipError_t launch_hvp<T>(const PatchArgs<T> &, const T *, const T *, T *, int, int,   \
                                      hipStream_t);                                                \
    template hipError_t launch_zero_boundary<T>(const int32_t *, int32_t, const int32_t *,         \
                                                int32_t, T *, T *, hipStream_t);                   \
    template hipError_t launch_pairs_eval<T>(const DevState *, PatternBufs, const T *, T *, T *,   \
                                             EnergySink, int, T, T, hipStream_t);                  \
    template hipError_t launch_pairs_hvp<T>(const DevState *, PatternBufs, const T *, const T *,   \
                                            T *, int, T, T, hipStream_t);
LAD_INST(float)
LAD_INST(double)

}  // namespace lad
