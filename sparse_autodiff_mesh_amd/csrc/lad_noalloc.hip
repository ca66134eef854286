// lad_noalloc.hip -- lad_eval_energy_grad_hess_noalloc: the evaluation for
// callers that cannot allocate device memory (code being captured into a
// HIP graph, tight serving loops, harnesses that forbid hipMalloc).
//
// The evaluation's only scratch is one partial energy per workgroup of its
// launches (summed afterwards in a fixed order).  lad_eval_energy_grad_hess
// keeps them in a buffer the context allocated at build time; this variant
// keeps them in `scratch`, a file-scope device array of fixed size that
// every GPU holds from the library's load until the process ends.  The
// kernels are the same, so the results are bitwise those of
// lad_eval_energy_grad_hess.
//
// In host code the name `scratch` denotes a host-side stand-in, not device
// memory: the array's device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lad_internal.h"

// Partial energies of one evaluation at most (256 KiB of doubles).
constexpr int32_t kScratchDoubles = 32768;

static __device__ __align__(256) double scratch[kScratchDoubles];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
double *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (which must be current),
// looked up on the first call for that device.
hipError_t scratch_on(int dev, double **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<double *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" lad_status lad_eval_energy_grad_hess_noalloc(lad_ctx *ctx, const void *d_x,
                                                       double *d_energy, void *d_grad,
                                                       void *d_hvals,
                                                       int64_t hvals_capacity_blocks,
                                                       void *hip_stream)
{
    if (!ctx) return lad::ctx_fail(nullptr, LAD_ERR_ARG, "ctx is NULL");
    if (lad::ctx_vf_capacity(ctx) > 0)
        return lad::ctx_fail(ctx, LAD_ERR_STATE,
                             "lad_eval_energy_grad_hess_noalloc: contexts with vertex-face "
                             "capacity keep per-contact strips in context scratch; use "
                             "lad_eval_energy_grad_hess");
    if (lad::eval_scratch_doubles(ctx) > kScratchDoubles)
        return lad::ctx_fail(ctx, LAD_ERR_CAPACITY,
                             "lad_eval_energy_grad_hess_noalloc: the evaluation has more "
                             "workgroups than the 32768 partial energies of the static "
                             "scratch array");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return lad::ctx_fail(ctx, LAD_ERR_HIP, "lad_eval_energy_grad_hess_noalloc: hipGetDevice");
    if (dev != lad::ctx_device(ctx))
        return lad::ctx_fail(ctx, LAD_ERR_STATE,
                             "lad_eval_energy_grad_hess_noalloc: the context's device must be "
                             "the current device");
    double *parts = nullptr;
    e = scratch_on(dev, &parts);
    if (e != hipSuccess)
        return lad::ctx_fail(ctx, LAD_ERR_HIP,
                             "lad_eval_energy_grad_hess_noalloc: hipGetSymbolAddress failed");
    return lad::eval_with_parts(ctx, d_x, d_energy, d_grad, d_hvals, hvals_capacity_blocks, parts,
                                static_cast<hipStream_t>(hip_stream));
}
