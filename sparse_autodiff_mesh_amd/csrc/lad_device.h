// lad_device.h -- device helpers shared by the evaluation kernels: fixed-order
// workgroup reductions, per-workgroup partial energies, XCD-aware workgroup
// numbering and the LDS -> HBM streaming store.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "lad_internal.h"

namespace lad {

__device__ __forceinline__ int64_t dalign16(int64_t x) { return (x + 15) & ~int64_t(15); }

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Renumber them so that XCD x gets the contiguous run of logical ids
// [x*n/8, (x+1)*n/8): neighbouring work items, which read the same vertex
// positions, then meet in one L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n)
{
    const int q = n >> 3, r = n & 7;
    const int x = b & 7, i = b >> 3;
    return x * q + min(x, r) + i;
}

// First chunk of this workgroup in a persistent launch that takes the chunks
// round robin in the XCD-grouped numbering (w, w + G, w + 2G, ... for G
// workgroups).  At any moment the launch works on a window of about G
// consecutive chunks, each XCD on a contiguous part of it, so that the
// write stream of a launch whose chunks store their slices of H moves
// through memory as one front (1000 x 1000 cloth: 63.2 against 67.8 us with
// a contiguous range of chunks per workgroup), while neighbouring rows
// still meet in one L2.
__device__ __forceinline__ int first_chunk() { return xcd_remap(blockIdx.x, gridDim.x); }

// Sum of `v` over a workgroup of NT threads in a fixed order (butterfly
// within each wave, then waves in index order); valid in thread 0.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if constexpr (NT == 64) {
        return v;
    } else {
        constexpr int W = NT / 64;
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[w] = v;
        __syncthreads();
        double s = 0.0;
        if (threadIdx.x == 0)
#pragma unroll
            for (int i = 0; i < W; ++i) s += red[i];
        return s;
    }
}

// Store this workgroup's partial energy (thread 0's `part`).  The partials
// are summed by k_energy_reduce, a separate launch on the same stream, so no
// workgroup waits on another and no device-wide fence is needed: on a GPU
// whose XCDs each have their own L2, an agent-scope release fence writes the
// whole L2 back, which costs far more than a second launch.
__device__ __forceinline__ void store_energy(const EnergySink &es, double part)
{
    if (threadIdx.x == 0) es.parts[es.part0 + blockIdx.x] = part;
}

template <typename T>
struct Vec;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
template <>
struct Vec<float> {
    using type = f32x4;
    static constexpr int n = 4;
};
template <>
struct Vec<double> {
    using type = f64x2;
    static constexpr int n = 2;
};

// Elements of padding in front of an LDS staging area so that its body is
// 16-byte aligned exactly where the global destination `dst_elem_off` is.
template <typename T>
__device__ __forceinline__ int stage_pad(int64_t dst_elem_off)
{
    return int(dst_elem_off % Vec<T>::n);
}

// Copy n elements from LDS src to global dst with NT threads.  The caller
// placed src `pad` elements after a 16-byte boundary, with pad equal to
// dst's misalignment in elements, so the body moves in aligned 16-byte
// nontemporal vector stores and only the head and tail are scalar.
template <int NT, typename T>
__device__ __forceinline__ void stream_out(T *__restrict__ dst, const T *src, int n, int pad)
{
    constexpr int V = Vec<T>::n;
    using VT = typename Vec<T>::type;
    const int head = min(n, (V - pad) % V);
    for (int i = threadIdx.x; i < head; i += NT) dst[i] = src[i];
    const int nvec = (n - head) / V;
    VT *dv = reinterpret_cast<VT *>(dst + head);
    const VT *sv = reinterpret_cast<const VT *>(src + head);
    for (int i = threadIdx.x; i < nvec; i += NT) __builtin_nontemporal_store(sv[i], dv + i);
    for (int i = head + nvec * V + threadIdx.x; i < n; i += NT) dst[i] = src[i];
}

// Zero the first n elements of the 16-byte aligned LDS area p with NT
// threads in 16-byte stores (n is rounded up to a whole vector, which the
// caller's allocation must hold).
template <int NT, typename T>
__device__ __forceinline__ void zero_lds(T *p, int n)
{
    using VT = typename Vec<T>::type;
    const int nvec = (n + Vec<T>::n - 1) / Vec<T>::n;
    const VT z = {};
    for (int i = threadIdx.x; i < nvec; i += NT) reinterpret_cast<VT *>(p)[i] = z;
}

}  // namespace lad
