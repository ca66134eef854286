// lad_pattern.hip -- symbolic block-CSR construction and prefix scan.
//
// Page "Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
// Computations", key design 3: the block sparsity of H is fixed by the mesh
// connectivity and the declared neighbourhoods, so the CSR structure is
// preallocated at initialisation by a parallel analysis plus a prefix sum
// for the row offsets.
//
// Rows are vertices; row a holds {a} and every vertex sharing a face or a
// spring with a, ascending and unique.  Steps: per-row raw count (atomics)
// -> exclusive scan -> fill (atomic cursors) -> per-row insertion sort and
// de-duplication in place -> scan of unique counts -> compaction.
#include "lad_internal.h"

namespace lad {

namespace {

constexpr int kWaves = kThreads / 64;
constexpr int kItems = 4;
constexpr int kTile = kThreads * kItems;

// Exclusive scan of one int per thread over the workgroup; *total gets the
// workgroup sum.  Wave-level inclusive scan by shuffles, then wave totals
// through LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = wsum[i];
        before += (i < w) ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

__global__ void __launch_bounds__(kThreads) k_scan_reduce(const int32_t *__restrict__ in, int32_t n,
                                                          int32_t *__restrict__ tmp)
{
    __shared__ int wsum[kWaves];
    const int64_t base = int64_t(blockIdx.x) * kTile + int64_t(threadIdx.x) * kItems;
    int s = 0;
#pragma unroll
    for (int k = 0; k < kItems; ++k)
        if (base + k < n) s += in[base + k];
    int tot;
    block_exclusive_scan(s, wsum, tot);
    if (threadIdx.x == 0) tmp[blockIdx.x] = tot;
}

// Down-sweep: tile b adds the sum of tiles 0..b-1 (read from tmp, summed
// by this workgroup in a fixed order) to its own exclusive scan.  The last
// tile also writes the total at out[n].  The per-tile top-level scan is thus
// folded into this launch.
template <typename Out>
__global__ void __launch_bounds__(kThreads) k_scan_down(const int32_t *__restrict__ in, int32_t n,
                                                        const int32_t *__restrict__ tmp, int32_t nb,
                                                        Out out)
{
    __shared__ int wsum[kWaves];
    int32_t *o = out.get();
    int before = 0;
    for (int32_t t0 = 0; t0 < int32_t(blockIdx.x); t0 += kThreads) {
        const int32_t t = t0 + threadIdx.x;
        int tot;
        block_exclusive_scan(t < int32_t(blockIdx.x) ? tmp[t] : 0, wsum, tot);
        before += tot;
    }
    const int64_t base = int64_t(blockIdx.x) * kTile + int64_t(threadIdx.x) * kItems;
    int v[kItems];
    int s = 0;
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        v[k] = (base + k < n) ? in[base + k] : 0;
        s += v[k];
    }
    int tot;
    int run = before + block_exclusive_scan(s, wsum, tot);
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        if (base + k < n) o[base + k] = run + out.add(base + k);
        run += v[k];
    }
    if (blockIdx.x == nb - 1 && threadIdx.x == kThreads - 1) o[n] = run + out.add(n);
}

// Scan destinations: where the output goes, and what is added to each
// element of it.
struct DirectOut {
    int32_t *p;
    __device__ int32_t *get() const { return p; }
    __device__ int32_t add(int64_t) const { return 0; }
};

// ---------------------------------------------------------------- pattern
__global__ void k_pat_init(int32_t nv, int32_t *__restrict__ cnt)
{
    const int32_t v = blockIdx.x * kThreads + threadIdx.x;
    if (v < nv) cnt[v] = 1;  // the diagonal
}

__global__ void k_pat_count(int32_t nf, const int32_t *__restrict__ faces, int32_t ns,
                            const int32_t *__restrict__ springs, int32_t *__restrict__ cnt)
{
    const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (t < 3 * int64_t(nf)) {
        atomicAdd(&cnt[faces[t]], 2);
    } else if (t < 3 * int64_t(nf) + 2 * int64_t(ns)) {
        atomicAdd(&cnt[springs[t - 3 * int64_t(nf)]], 1);
    }
}

__global__ void k_pat_self(int32_t nv, const int32_t *__restrict__ off, int32_t *__restrict__ raw,
                           int32_t *__restrict__ cur)
{
    const int32_t v = blockIdx.x * kThreads + threadIdx.x;
    if (v < nv) {
        raw[off[v]] = v;
        cur[v] = 1;
    }
}

__global__ void k_pat_fill(int32_t nf, const int32_t *__restrict__ faces, int32_t ns,
                           const int32_t *__restrict__ springs, const int32_t *__restrict__ off,
                           int32_t *__restrict__ raw, int32_t *__restrict__ cur)
{
    const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (t < int64_t(nf)) {
        const int32_t *f = faces + 3 * t;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (i != j) raw[off[f[i]] + atomicAdd(&cur[f[i]], 1)] = f[j];
    } else if (t < int64_t(nf) + ns) {
        const int32_t *s = springs + 2 * (t - nf);
        raw[off[s[0]] + atomicAdd(&cur[s[0]], 1)] = s[1];
        raw[off[s[1]] + atomicAdd(&cur[s[1]], 1)] = s[0];
    }
}

// Sort one row (insertion sort; rows are short) and keep the unique prefix
// in place.  A row of up to kUniqLds raw entries is sorted in this thread's
// part of LDS (entry i of thread t at i * kThreads + t, so the lanes of a
// wave touch distinct banks), where each step of the sort costs an LDS
// round trip instead of a global one (1000 x 1000 cloth, 19 raw entries per
// row: 940 us in global memory); longer rows are sorted where they are.
constexpr int kUniqLds = 32;

__device__ __forceinline__ int32_t sort_unique(int32_t *r, int32_t n, int32_t stride)
{
    for (int32_t i = 1; i < n; ++i) {
        const int32_t key = r[i * stride];
        int32_t j = i - 1;
        while (j >= 0 && r[j * stride] > key) {
            r[(j + 1) * stride] = r[j * stride];
            --j;
        }
        r[(j + 1) * stride] = key;
    }
    int32_t u = 0;
    for (int32_t i = 0; i < n; ++i)
        if (i == 0 || r[i * stride] != r[(u - 1) * stride]) r[(u++) * stride] = r[i * stride];
    return u;
}

__global__ void __launch_bounds__(kThreads)
k_pat_unique(int32_t nv, const int32_t *__restrict__ off, int32_t *__restrict__ raw,
             int32_t *__restrict__ ucnt)
{
    __shared__ int32_t buf[kUniqLds * kThreads];
    const int32_t v = blockIdx.x * kThreads + threadIdx.x;
    if (v >= nv) return;  // no barrier below: each thread uses only its own LDS
    int32_t *r = raw + off[v];
    const int32_t n = off[v + 1] - off[v];
    if (n <= kUniqLds) {
        int32_t *b = buf + threadIdx.x;
        for (int32_t i = 0; i < n; ++i) b[i * kThreads] = r[i];
        const int32_t u = sort_unique(b, n, kThreads);
        for (int32_t i = 0; i < u; ++i) r[i] = b[i * kThreads];
        ucnt[v] = u;
    } else {
        ucnt[v] = sort_unique(r, n, 1);
    }
}

__global__ void k_pat_compact(int32_t nv, const int32_t *__restrict__ off,
                              const int32_t *__restrict__ raw, const int32_t *__restrict__ row_ptr,
                              int32_t *__restrict__ col_idx)
{
    const int32_t v = blockIdx.x * kThreads + threadIdx.x;
    if (v >= nv) return;
    const int32_t *r = raw + off[v];
    int32_t *o = col_idx + row_ptr[v];
    const int32_t n = row_ptr[v + 1] - row_ptr[v];
    for (int32_t i = 0; i < n; ++i) o[i] = r[i];
}

inline unsigned blocks_for(int64_t n) { return unsigned((n + kThreads - 1) / kThreads); }

}  // namespace

int64_t scan_tmp_size(int64_t n) { return (n + kTile - 1) / kTile + 2; }

template <typename Out>
static hipError_t scan_impl(const int32_t *in, Out out, int32_t n, int32_t *tmp, hipStream_t s)
{
    const int32_t nb = n > 0 ? int32_t((int64_t(n) + kTile - 1) / kTile) : 1;
    hipLaunchKernelGGL(k_scan_reduce, dim3(nb), dim3(kThreads), 0, s, in, n, tmp);
    hipLaunchKernelGGL((k_scan_down<Out>), dim3(nb), dim3(kThreads), 0, s, in, n,
                       (const int32_t *)tmp, nb, out);
    return hipGetLastError();
}

hipError_t launch_scan(const int32_t *in, int32_t *out, int32_t n, int32_t *tmp, hipStream_t s)
{
    return scan_impl(in, DirectOut{out}, n, tmp, s);
}

hipError_t launch_pattern_count(int32_t nv, int32_t nf, const int32_t *faces, int32_t ns,
                                const int32_t *springs, PatternScratch sc, hipStream_t s)
{
    hipLaunchKernelGGL(k_pat_init, dim3(blocks_for(nv)), dim3(kThreads), 0, s, nv, sc.cnt);
    const int64_t items = 3 * int64_t(nf) + 2 * int64_t(ns);
    if (items > 0)
        hipLaunchKernelGGL(k_pat_count, dim3(blocks_for(items)), dim3(kThreads), 0, s, nf, faces,
                           ns, springs, sc.cnt);
    return launch_scan(sc.cnt, sc.off, nv, sc.tmp, s);
}

hipError_t launch_pattern_fill(int32_t nv, int32_t nf, const int32_t *faces, int32_t ns,
                               const int32_t *springs, PatternScratch sc, hipStream_t s)
{
    hipLaunchKernelGGL(k_pat_self, dim3(blocks_for(nv)), dim3(kThreads), 0, s, nv, sc.off, sc.raw,
                       sc.cur);
    const int64_t items = int64_t(nf) + ns;
    if (items > 0)
        hipLaunchKernelGGL(k_pat_fill, dim3(blocks_for(items)), dim3(kThreads), 0, s, nf, faces,
                           ns, springs, sc.off, sc.raw, sc.cur);
    return hipGetLastError();
}

hipError_t launch_pattern_unique(int32_t nv, PatternScratch sc, hipStream_t s)
{
    hipLaunchKernelGGL(k_pat_unique, dim3(blocks_for(nv)), dim3(kThreads), 0, s, nv, sc.off,
                       sc.raw, sc.ucnt);
    return hipGetLastError();
}

hipError_t launch_pattern_compact(int32_t nv, PatternScratch sc, const int32_t *row_ptr,
                                  int32_t *col_idx, hipStream_t s)
{
    hipLaunchKernelGGL(k_pat_compact, dim3(blocks_for(nv)), dim3(kThreads), 0, s, nv, sc.off,
                       sc.raw, row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace lad
