// lad_terms_internal.h -- host-visible structures and launchers of the term
// front end (kernels in terms_engine.h, sets in lad_terms.hip, the C ABI in
// lad_terms_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lad_internal.h"

namespace lad {
namespace terms {

constexpr int kMaxTerms = 4;   // term types of one set
constexpr int kMaxVerts = 4;   // vertices per element (offsets pack into 24 bits)
constexpr int kTermsHvpThreads = 256;  // threads per workgroup of the product kernel
constexpr int kTermsHvpGroupsPerCU = 4;  // resident product workgroups per CU, at most

// Set ids (the values of LAD_TERMS_* in include/lad_terms.h).
constexpr int kSetCloth = 1;
constexpr int kSetArap = 2;
constexpr int kSetSymDirichlet = 3;
constexpr int kSetArapCloth = 4;
constexpr int kSetClothQuad = 5;

// One element seen from the row of one of its vertices: e is the element
// id; pk holds the row vertex's position i in the element (bits 0-1), for
// b = 1 .. K-1 the block offset within the row of the element's vertex
// (i + b) % K (bits 8b .. 8b+7), and whether this record is that block's
// first writer in the row (bit 1 + b): the first record, in the set's term
// order and then the row's record order, whose element holds the column,
// which stores its part instead of adding it (the fused explicit pass
// starts from unwritten staging).
struct alignas(8) TermInc {
    int32_t e;
    uint32_t pk;
};

// Terms of at most kInlineVerts vertices keep, in each row's incidence
// record, the element's other vertex and its constants, so a row streams
// its records instead of gathering the element's data by element id (each
// element is stored once per vertex, twice at most).  Larger stencils keep
// one copy of each element's data, which the rows of its vertices share
// through the caches.
constexpr int kInlineVerts = 2;
// Rows per slice of the transposed small-stencil records (one wave reads
// record j of 64 consecutive rows with one coalesced load).
constexpr int kTermSliceRows = 64;

// pk as in TermInc; other: the element's other vertex (two-vertex terms);
// c: the element's constants.
template <typename T, int NC>
struct alignas(8) InlineRec {
    uint32_t pk;
    int32_t other;
    T c[NC > 0 ? NC : 1];
};

template <typename T>
constexpr size_t inline_rec_bytes(int nconst)
{
    return (8 + size_t(nconst > 0 ? nconst : 1) * sizeof(T) + 7) & ~size_t(7);
}
static_assert(sizeof(InlineRec<float, 2>) == inline_rec_bytes<float>(2), "record layout");
static_assert(sizeof(InlineRec<float, 4>) == inline_rec_bytes<float>(4), "record layout");
static_assert(sizeof(InlineRec<float, 1>) == inline_rec_bytes<float>(1), "record layout");
static_assert(sizeof(InlineRec<double, 2>) == inline_rec_bytes<double>(2), "record layout");
static_assert(sizeof(InlineRec<double, 4>) == inline_rec_bytes<double>(4), "record layout");
static_assert(sizeof(InlineRec<double, 1>) == inline_rec_bytes<double>(1), "record layout");

template <typename T>
struct TermData {
    const int32_t *inc_ptr;      // [nv+1] incidence offsets
    const TermInc *inc;          // incident elements of each row, by element id
                                 // (terms of more than kInlineVerts vertices)
    const void *inl;             // the same as InlineRec<T, kConsts> records
                                 // (terms of at most kInlineVerts vertices),
                                 // rows in order (the explicit pass)
    const void *inl_sl;          // the same records transposed per slice of
                                 // kTermSliceRows rows (the product): record
                                 // j of row a is inl_sl[sl_ptr[a / 64] +
                                 // 64 j + a % 64]
    const int32_t *sl_ptr;       // [nslice + 1] first record of each slice
    const int32_t *elems;        // [ne][K] vertex ids (larger terms only)
    const T *consts;             // [ne][kConsts] (larger terms only)
};

template <typename T>
struct TermsArgs {
    const PatchHdr *chunk;       // v0, nown of each chunk of up to 64 rows
    int32_t nchunk;
    int32_t nv;
    const int32_t *rp, *ci;      // pattern
    const int32_t *diag;         // [nv] offset of the diagonal block in its row
    int32_t lds_blocks;          // staging capacity per workgroup, in blocks
    TermData<T> t[kMaxTerms];    // the launch's terms, in list order
};

struct TermInfo {
    int arity;                   // vertices per element
    int nconst;                  // constants per element
    const char *name;
};

// Terms of a set (their number; 0 for an unknown set).
int set_terms(int set, TermInfo out[kMaxTerms]);

template <typename T>
hipError_t terms_grid(int set, int lds, int nchunk, int nv, int *grid_eval, int *grid_hvp);
// Fused: one launch, partial energies at es.part0 + [0, grid).  Unfused:
// one launch per term t, partial energies at es.part0 + t * grid + [0, grid).
template <typename T>
hipError_t launch_terms_eval(int set, int fused, const TermsArgs<T> &a, const T *x, T *g, T *hv,
                             EnergySink es, int grid, int lds, hipStream_t s);
template <typename T>
hipError_t launch_terms_hvp(int set, int fused, const TermsArgs<T> &a, const T *x, const T *v,
                            T *y, int grid, hipStream_t s);

}  // namespace terms
}  // namespace lad
