// cg_device.h -- the scalar steps of the Newton-CG iteration as device
// functions, computed redundantly by every workgroup of the kernel that
// needs them (no single-workgroup launch between the vector kernels, no
// device-wide fence).  Included by the solver and the row HVP, which forms
// the direction itself.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "lad.h"
#include "lad_device.h"
#include "lad_solve.h"

namespace lad {

constexpr int kCgSumLoads = 4;  // partial sums each thread loads at once

// Sum of parts[0 .. n) by a workgroup of NTH threads, in one fixed order
// (thread t adds parts[t], parts[t + NTH], ...; then the workgroup
// reduction), returned to every thread.  The partial sums were written by
// other XCDs, so each thread issues kCgSumLoads loads before adding any.
// red: NTH / 64 doubles of LDS (unused for one wave); bc: one double.
template <int NTH>
__device__ __forceinline__ double cg_sum(const double *__restrict__ parts, int n, double *red,
                                         double *bc)
{
    double s = 0.0;
    for (int i0 = 0; i0 < n; i0 += NTH * kCgSumLoads) {
        double v[kCgSumLoads];
#pragma unroll
        for (int k = 0; k < kCgSumLoads; ++k) {
            const int i = i0 + k * NTH + int(threadIdx.x);
            v[k] = i < n ? parts[i] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kCgSumLoads; ++k) s += v[k];
    }
    s = block_sum<NTH>(s, red);  // valid in thread 0
    if constexpr (NTH == 64) {
        return __shfl(s, 0);
    } else {
        if (threadIdx.x == 0) *bc = s;
        __syncthreads();
        return *bc;
    }
}

// The stop flag, one value for the whole workgroup (thread 0's load), so
// that no wave of it returns while another waits at a barrier.
template <int NTH>
__device__ __forceinline__ int32_t cg_stop(const CgState *st, int32_t *bc)
{
    if constexpr (NTH == 64) {
        return __builtin_amdgcn_readfirstlane(st->stop);
    } else {
        if (threadIdx.x == 0) *bc = st->stop;
        __syncthreads();
        return *bc;
    }
}

// The step that closes update iter - 1 (iter >= 1), before direction iter:
// r.r of the new residual from its partial sums; below the threshold the
// solve has converged, else beta = r.r / the previous r.r.  With `writer`
// (one workgroup) thread 0 records it.  Returns beta; stop = 1 on
// convergence.
template <int NTH>
__device__ __forceinline__ double cg_beta_step(CgState *st, const double *__restrict__ rr_parts,
                                               int n_rr, int32_t iter, bool writer,
                                               int32_t &stop, double *red, double *bc)
{
    const double rr = cg_sum<NTH>(rr_parts, n_rr, red, bc);
    const double rr_old = st->rrv[(iter - 1) & 1];
    const bool conv = rr < st->eps2;
    const double beta = conv ? 0.0 : rr / rr_old;
    if (writer && threadIdx.x == 0) {
        st->rrv[iter & 1] = rr;
        st->iter = iter;
        st->beta = beta;
        if (conv) {
            st->reason = LAD_CG_CONVERGED;
            st->stop = 1;
        }
    }
    stop = conv ? 1 : 0;
    return beta;
}

}  // namespace lad
