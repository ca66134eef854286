// lad_terms.hip -- the term sets compiled into the library and their
// launchers.  A set is a compile-time list of user terms (user_terms.h);
// every kernel of terms_engine.h is instantiated for it.  To add a set,
// append its list to the table below (and its id to include/lad_terms.h).
#include <hip/hip_runtime.h>

#include "lad_terms_internal.h"
#include "terms_engine.h"
#include "user_terms.h"

namespace lad {
namespace terms {

template <typename... Ts>
struct TermList {
    static constexpr int n = sizeof...(Ts);
};

namespace {

template <typename Term>
TermInfo info_of(const char *name)
{
    return TermInfo{Term::kVerts, Term::kConsts, name};
}

// Fused: one launch over every term of the list.
template <typename T, typename... Ts>
void launch_eval_fused(TermList<Ts...>, const TermsArgs<T> &a, const T *x, T *g, T *hv,
                       EnergySink es, int grid, int lds, hipStream_t s)
{
    hipLaunchKernelGGL((k_terms_eval<T, false, true, Ts...>), dim3(grid), dim3(kRowThreads), lds, s,
                       a, x, g, hv, es);
}

template <typename T, bool ACC, typename Term>
void launch_eval_one(const TermsArgs<T> &a, int idx, const T *x, T *g, T *hv, EnergySink es,
                     int grid, int lds, hipStream_t s)
{
    TermsArgs<T> b = a;
    b.t[0] = a.t[idx];
    hipLaunchKernelGGL((k_terms_eval<T, ACC, false, Term>), dim3(grid), dim3(kRowThreads), lds, s,
                       b, x, g, hv, EnergySink{es.parts, es.part0 + idx * grid});
}

// Unfused: one launch per term, the later ones adding into g and H.
template <typename T, typename... Ts, size_t... I>
void launch_eval_unfused(TermList<Ts...>, std::index_sequence<I...>, const TermsArgs<T> &a,
                         const T *x, T *g, T *hv, EnergySink es, int grid, int lds, hipStream_t s)
{
    (launch_eval_one<T, (I > 0), Ts>(a, int(I), x, g, hv, es, grid, lds, s), ...);
}

template <typename T, typename... Ts>
void launch_hvp_fused(TermList<Ts...>, const TermsArgs<T> &a, const T *x, const T *v, T *y,
                      int grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_terms_hvp<T, false, Ts...>), dim3(grid), dim3(kTermsHvpThreads), 0, s, a,
                       x, v, y);
}

template <typename T, bool ACC, typename Term>
void launch_hvp_one(const TermsArgs<T> &a, int idx, const T *x, const T *v, T *y, int grid,
                    hipStream_t s)
{
    TermsArgs<T> b = a;
    b.t[0] = a.t[idx];
    hipLaunchKernelGGL((k_terms_hvp<T, ACC, Term>), dim3(grid), dim3(kTermsHvpThreads), 0, s, b, x,
                       v, y);
}

template <typename T, typename... Ts, size_t... I>
void launch_hvp_unfused(TermList<Ts...>, std::index_sequence<I...>, const TermsArgs<T> &a,
                        const T *x, const T *v, T *y, int grid, hipStream_t s)
{
    (launch_hvp_one<T, (I > 0), Ts>(a, int(I), x, v, y, grid, s), ...);
}

template <typename T, typename... Ts>
hipError_t occupancy(TermList<Ts...>, int lds, int *occ_e, int *occ_h)
{
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        occ_e, k_terms_eval<T, false, true, Ts...>, kRowThreads, lds);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(occ_h, k_terms_hvp<T, false, Ts...>,
                                                         kTermsHvpThreads, 0);
    return e;
}

// ---- the sets -------------------------------------------------------------
using SetCloth = TermList<Spring, Inertia>;
using SetArap = TermList<ArapFace>;
using SetSymDirichlet = TermList<SymDirichletFace>;
using SetArapCloth = TermList<ArapFace, Spring, Inertia>;
using SetClothQuad = TermList<Spring, Inertia, QuadPlanarity>;

// Calls f(list) for the set's term list; false for an unknown set.
template <typename F>
bool with_set(int set, F &&f)
{
    switch (set) {
    case kSetCloth: f(SetCloth{}); return true;
    case kSetArap: f(SetArap{}); return true;
    case kSetSymDirichlet: f(SetSymDirichlet{}); return true;
    case kSetArapCloth: f(SetArapCloth{}); return true;
    case kSetClothQuad: f(SetClothQuad{}); return true;
    default: return false;
    }
}

}  // namespace

int set_terms(int set, TermInfo out[kMaxTerms])
{
    const TermInfo spring = info_of<Spring>("spring");
    const TermInfo inertia = info_of<Inertia>("inertia");
    const TermInfo arap = info_of<ArapFace>("arap_face");
    const TermInfo sd = info_of<SymDirichletFace>("symmetric_dirichlet_face");
    const TermInfo quad = info_of<QuadPlanarity>("quad_planarity");
    switch (set) {
    case kSetCloth: out[0] = spring; out[1] = inertia; return 2;
    case kSetArap: out[0] = arap; return 1;
    case kSetSymDirichlet: out[0] = sd; return 1;
    case kSetArapCloth: out[0] = arap; out[1] = spring; out[2] = inertia; return 3;
    case kSetClothQuad: out[0] = spring; out[1] = inertia; out[2] = quad; return 3;
    default: return 0;
    }
}

template <typename T>
hipError_t terms_grid(int set, int lds, int nchunk, int nv, int *grid_eval, int *grid_hvp)
{
    int dev = 0, cus = 0, occ_e = 0, occ_h = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (!with_set(set, [&](auto list) { e = occupancy<T>(list, lds, &occ_e, &occ_h); }))
        return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    auto clamp = [&](int occ, int64_t units) {
        const int64_t full = int64_t(cus > 0 ? cus : 1) * (occ > 0 ? occ : 1);
        const int64_t g = units < full ? units : full;
        return int(g < 1 ? 1 : g);
    };
    // The explicit pass's workgroups are single waves: a resident count that
    // is not a multiple of the CU's four SIMDs leaves some SIMDs a wave more
    // work than others (10 per CU: 125 us for the cloth set at 1000^2, 8 per
    // CU: 92 us).
    if (occ_e > 4) occ_e -= occ_e % 4;
    *grid_eval = clamp(occ_e, nchunk);
    // The product's lanes each walk their own row's records, so a wave
    // touches a wide strip of lines; more than kTermsHvpGroupsPerCU resident
    // workgroups per CU overflow the L2 and refetch them (at 1000^2 cloth:
    // 509 MB fetched and 78 us with 8 per CU, 314 MB and 55 us with 4).
    *grid_hvp = clamp(occ_h < kTermsHvpGroupsPerCU ? occ_h : kTermsHvpGroupsPerCU,
                      (int64_t(nv) + kTermsHvpThreads - 1) / kTermsHvpThreads);
    return hipSuccess;
}

template <typename T>
hipError_t launch_terms_eval(int set, int fused, const TermsArgs<T> &a, const T *x, T *g, T *hv,
                             EnergySink es, int grid, int lds, hipStream_t s)
{
    const bool known = with_set(set, [&](auto list) {
        using L = decltype(list);
        if (fused || L::n == 1)
            launch_eval_fused<T>(list, a, x, g, hv, es, grid, lds, s);
        else
            launch_eval_unfused<T>(list, std::make_index_sequence<L::n>{}, a, x, g, hv, es, grid,
                                   lds, s);
    });
    return known ? hipGetLastError() : hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_terms_hvp(int set, int fused, const TermsArgs<T> &a, const T *x, const T *v,
                            T *y, int grid, hipStream_t s)
{
    const bool known = with_set(set, [&](auto list) {
        using L = decltype(list);
        if (fused || L::n == 1)
            launch_hvp_fused<T>(list, a, x, v, y, grid, s);
        else
            launch_hvp_unfused<T>(list, std::make_index_sequence<L::n>{}, a, x, v, y, grid, s);
    });
    return known ? hipGetLastError() : hipErrorInvalidValue;
}

#define LAD_TERMS_INST(T)                                                                        \
    template hipError_t terms_grid<T>(int, int, int, int, int *, int *);                         \
    template hipError_t launch_terms_eval<T>(int, int, const TermsArgs<T> &, const T *, T *, T *, \
                                             EnergySink, int, int, hipStream_t);                 \
    template hipError_t launch_terms_hvp<T>(int, int, const TermsArgs<T> &, const T *,           \
                                            const T *, T *, int, hipStream_t);
LAD_TERMS_INST(float)
LAD_TERMS_INST(double)

}  // namespace terms
}  // namespace lad
