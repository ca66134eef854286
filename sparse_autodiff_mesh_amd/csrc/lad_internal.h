// lad_internal.h -- types shared by the host side of liblad (patcher, API)
// and its HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <string>
#include <vector>

#include "lad.h"
#include "lad_solve.h"

namespace lad {

constexpr int kThreads = 256;          // threads per workgroup, patch kernels
constexpr uint16_t kNone = 0xFFFFu;    // "this row is not owned by the patch"
constexpr int kMaxLocal = 65535;       // local vertex / block ids are uint16
constexpr int kMaxColors = 256;        // colour phases per element kind
constexpr int kDefaultPatchLds = 40 * 1024;   // patch LDS budget by default
constexpr int kMaxPatchLds = 159 * 1024;      // leaves room for static LDS

// One two-vertex element seen from one patch.  lab = la | lb << 16 are the
// patch-local vertex ids (owned vertices first, then ribbon vertices);
// blk = blk_ab | blk_ba << 16 are patch-relative block indices of (a, b) in
// row a and of (b, a) in row b (kNone when that row is not owned).
struct SpringRec {
    uint32_t lab;
    uint32_t blk;
};

// One triangle seen from one patch: local vertex ids and the patch-relative
// block index of (v_i, v_j) in row v_i for every ordered pair (kNone when
// v_i is not owned).  24 bytes.
struct FaceRec {
    uint16_t l[3];
    uint16_t blk[9];
};

// Per-patch header.  The patch owns vertices [v0, v0 + nown) and thereby
// the contiguous block range [blk0, blk0 + nblk) of the topology pattern.
struct PatchHdr {
    int32_t v0, nown;        // owned vertex range
    int32_t rib_off, nrib;   // ribbon (ghost) vertex list
    int32_t spr_off, nspr;   // spring records
    int32_t fac_off, nfac;   // face records
    int32_t blk0, nblk;      // base block range of the owned rows
    int32_t col_off;         // offset into the colour-bound list
    int32_t nspr_col;        // spring colours (bounds at col_off .. +nspr_col)
    int32_t nfac_col;        // face colours (bounds follow the spring bounds)
    int32_t amap_cap;        // reserved LDS map entries for an active chunk
    int32_t lds_eval;        // LDS bytes this patch needs in the eval kernel
    int32_t lds_hvp;         // ... and in the HVP kernel
};
static_assert(sizeof(PatchHdr) == 64, "PatchHdr layout");

// Device-side state of the double-buffered pattern.  Kernels read `active`
// (0 = topology pattern, 1 or 2 = a pair buffer); only the commit kernel of
// lad_insert_pairs writes it.
struct DevState {
    int32_t active;
    int32_t err_latched;     // sticky error bits: 1 = bad pair, 2 = capacity,
                             // 4 = the insertion's tile chain did not complete
    int32_t err_cur;         // error bits of the insert in flight (zero
                             // between inserts: the commit clears it)
    int32_t np[3];           // pairs of each buffer
    int32_t nnzb[3];         // blocks of each buffer
    int32_t nvf[3];          // vertex-face contacts of each buffer
    int32_t ins_back;        // buffer the insert in flight writes (set by its
                             // first kernel, so the commit may flip `active`
                             // while later workgroups still run)
    uint32_t ins_seq;        // inserts so far: tags the tile chain's status
    int32_t pad[2];
};

// ---------------------------------------------------------------------------
// Host-side patch plan (built by the patcher, uploaded by the API).
// ---------------------------------------------------------------------------
struct Plan {
    int elem_size = 4;                     // sizeof(T)
    std::vector<PatchHdr> hdr;
    std::vector<int32_t> rib;              // ribbon vertex ids, sorted per patch
    std::vector<SpringRec> spr;
    std::vector<int32_t> spr_src;          // spring id behind each record
    std::vector<FaceRec> fac;
    std::vector<int32_t> fac_src;          // face id behind each record
    std::vector<int32_t> col_bounds;       // colour bounds (record offsets)
    std::vector<uint16_t> diag_rel;        // [nv] patch-relative diagonal block
    std::vector<int32_t> vpatch;           // [nv] owning patch of each vertex
    int32_t lds_eval = 0, lds_hvp = 0, max_colors = 0;
    // Element-once plans (boundary atomics) only.  Each element is kept by
    // the patch that owns its lowest vertex id; its other vertices may lie
    // in other patches ("foreign" rows).  spr_gblk[2 r + 0 / 1]: global
    // blocks (f, f) and (f, o) of spring record r's foreign endpoint f (o the
    // other endpoint), -1 when both are owned; fac_gblk[9 r + 3 v + u]:
    // global block (v, u) of face record r when its vertex v is foreign,
    // else -1.  bnd_blk / bnd_vtx: the blocks and vertices that receive a
    // foreign contribution (ascending); blk_flag [nnzb] / vtx_flag [nv]: 1
    // for those, else 0.
    std::vector<int32_t> spr_gblk, fac_gblk, bnd_blk, bnd_vtx;
    std::vector<uint8_t> blk_flag, vtx_flag;
};

struct PlanInput {
    int32_t nv = 0;
    int32_t nf = 0;
    const int32_t *faces = nullptr;
    int32_t ns = 0;
    const int32_t *springs = nullptr;
    int32_t face_energy = 0;
    const int32_t *row_ptr = nullptr;      // topology pattern (host copies)
    const int32_t *col_idx = nullptr;
    int32_t elem_size = 4;
    int32_t lds_budget = 0;
    int32_t element_once = 0;              // 1: each element in one patch only
};

// LDS bytes of one patch in the eval and HVP kernels (same formula the
// kernels use to carve their dynamic LDS).
int64_t lds_eval_bytes(int elem_size, int nblk, int nown, int nloc, int amap_cap);
int64_t lds_hvp_bytes(int elem_size, int nown, int nloc);
int32_t amap_capacity(int nblk);

// Returns "" on success, else an error message.
std::string build_plan(const PlanInput &in, Plan &out);

// Row chunks for the row-owner kernels: up to kRowsPerChunk consecutive rows
// whose topology blocks fit kRowBaseBlocks; every chunk reserves
// kRowLdsBlocks blocks of LDS staging (the slack takes pair insertions).
constexpr int kRowLdsBlocks = 512;
constexpr int kRowBaseBlocks = 456;

// One triangle seen from the row of one of its vertices (row-owner face
// terms, explicit kernel).  f is the face id; with i the row vertex's
// position in the face, o1 and o2 are the face's vertices at positions
// (i+1)%3 and (i+2)%3; pk packs i (bits 0-1) and, for face position k = 0,
// 1, 2, the offset of that vertex's block within the row's topology pattern
// (bits 8k+8 .. 8k+15).
struct alignas(16) FaceInc {
    int32_t f, o1, o2;
    uint32_t pk;
};
constexpr int kMaxRowFaceSlots = 256;   // slot offsets fit 8 bits
constexpr int kSliceRows = 64;          // rows per slice of the product kernels: one wave

// Face terms in the product kernels.  Every slice lists the faces incident
// to its rows once; the kernel evaluates each listed face once per slice,
// in rounds of kFaceRound faces (one per lane, results in LDS), and every
// row then gathers its part of the faces of the round.  A face whose
// vertices lie in two slices is evaluated by both (each writes only its own
// rows); on a grid numbered row by row that is every face, against three
// evaluations (one per vertex row) when each row evaluates its faces
// itself.  The list takes each row's first incident face, then each row's
// second, and so on, so that every round holds about as many faces of
// every row.
constexpr int kFaceRound = 64;
struct alignas(16) SliceFace {
    int32_t v[3];   // the face's vertices, in face order
    int32_t f;      // face id (rest data)
};
// One face seen from one of its rows in the product kernels: lf is its
// position in the slice's list, i (bits 0-1 of pi) the row vertex's
// position in the face.
struct RowFace {
    uint32_t lf;
    uint32_t pi;
};

struct RowPlan {
    std::vector<PatchHdr> chunk;     // v0, nown (rows), blk0, nblk, amap_cap, and spr_off:
                                     // the spring slice whose rows the chunk is, when
                                     // every off-diagonal block of its rows has a
                                     // spring behind it, else -1
    std::vector<double> slot_rest;   // [nnzb] rest length behind each block, -1: none
    // face term on:
    std::vector<int32_t> fptr;       // [nv+1] offsets of each row's faces in finc and rfinc
    std::vector<FaceInc> finc;       // each row's faces, by face id
    std::vector<RowFace> rfinc;      // each row's faces, by position in its slice's list
    std::vector<int32_t> sf_ptr;     // [nslice+1] offsets of each slice's face list
    std::vector<SliceFace> sface;    // the slices' face lists
    // Slices of the product kernels: slice t's lane l takes row
    // kSliceRows * t + l, or, with the face term on, sl_rows[kSliceRows * t
    // + l] (breadth-first patches of the mesh, -1 for padding; every row in
    // exactly one slice).  Spring slices: slice t holds sl_ptr[t + 1] -
    // sl_ptr[t] = kSliceRows * W_t entries, W_t the most springs any of its
    // rows has.  Spring j of lane l's row (its j-th spring neighbour in
    // ascending column order) is entry sl_ptr[t] + kSliceRows * j + l: a
    // wave reads one spring of each of its rows with one coalesced load.
    // Padding entries name the row itself (the last row for a padding lane)
    // with rest length -1.
    std::vector<int32_t> sl_rows;
    std::vector<int32_t> sl_ptr;     // [nslice + 1]
    std::vector<int32_t> sl_nb;      // neighbour vertex
    std::vector<double> sl_rest;     // rest length
    // The same neighbours as 16-bit differences from the entry's row
    // (the last row for a padding lane): filled when every difference fits,
    // which halves the neighbour bytes the kernels stream; else empty.
    std::vector<int16_t> sl_d16;
};

// Returns "" when the row path applies (rest lengths >= 0, at most one
// spring per vertex pair, rows short enough), else the reason.
std::string build_row_plan(const PlanInput &in, const double *rest_len, RowPlan &out);

// The largest block count of a half chunk (its first kRowsPerChunk / 2 rows,
// or the rest) over the chunks, with rp the topology row pointer: the
// staging capacity of the face kernel, which stages one half at a time.
int32_t half_chunk_blocks(const std::vector<PatchHdr> &chunks, const int32_t *rp);

// ---------------------------------------------------------------------------
// Kernel argument bundles and launchers (defined in the .hip files).
// ---------------------------------------------------------------------------
struct PatternBufs {
    const int32_t *rp[3];
    const int32_t *ci[3];
    const int32_t *pairs[3];
    const int32_t *pinc_ptr[3];  // per-row pair incidence (buffers 1, 2)
    const int32_t *pinc[3];
    const int32_t *pinc_row[3];
    const int32_t *trow[3];      // per incidence entry: its row if the entry is
                                 // the row's first, else -1 (touched rows)
    const int32_t *pnew[3];      // per touched row, at 3 x its first incidence
                                 // entry: its columns that the topology row
                                 // lacks, ascending
    const int32_t *rins1[3];     // per row: its smallest inserted column
                                 // (INT32_MAX: none)
    const int4 *pslot[3];        // per incidence entry: the active slot of a
                                 // pair's (row, partner) block (-1 for a
                                 // vertex-face entry), of the row's diagonal
                                 // block, the pair's partner p as 2 p + 1 when
                                 // the row's vertex is the pair's first, 2 p
                                 // when second (for a vertex-face entry -2 - i,
                                 // i the row's vertex's place in the contact,
                                 // or -1 when not recorded), and the row's
                                 // first active slot s0 (-1 - s0 when the row
                                 // gains more than kMaxIns columns)
    const int32_t *vf[3];        // vertex-face contacts: (vertex, face id)
    const int32_t *faces;        // [nf][3] mesh faces (contacts on)
};

template <typename T>
struct PatchArgs {
    const PatchHdr *hdr;
    int32_t npatch;
    const int32_t *rib;
    const SpringRec *spr;
    const T *spr_rest;
    const FaceRec *fac;
    const T *fac_dm;             // [records][4]
    const T *fac_area;
    const int32_t *col_bounds;
    const uint16_t *diag_rel;
    const T *x_tilde;            // null = no inertia
    T k, c;
    int32_t springs_on, faces_on, inertia_on;
    const DevState *state;
    PatternBufs pat;
    // element-once plans (boundary atomics): see Plan
    const int32_t *spr_gblk;
    const int32_t *fac_gblk;
    const uint8_t *blk_flag;
    const uint8_t *vtx_flag;
};

// Where a launch puts its partial energies: workgroup b stores its sum at
// parts[part0 + b].  launch_energy_reduce then sums parts[0 .. n) in index
// order (fixed order, independent of scheduling).
struct EnergySink {
    double *parts;
    int32_t part0;
};

hipError_t launch_energy_reduce(const double *parts, int32_t n, double *out, hipStream_t s);
// Debug check: bit 8 of st->err_latched if the energy (if given), any of
// the nvec vector entries, or any value of the active pattern's blocks in
// hv (if given) is not finite; es = 4 or 8 bytes per value.
hipError_t launch_check_finite(DevState *st, const double *energy, const void *vec, int64_t nvec,
                               const void *hv, int es, hipStream_t s);

// Assembly of the patch kernels: LDS atomics, colour phases (fixed order),
// or element-once patches whose contributions to other patches' rows are
// added with global float atomics into slots zeroed beforehand.
enum PatchMode { kModeLdsAtomic = 0, kModeColour = 1, kModeBoundaryAtomic = 2 };

template <typename T>
hipError_t launch_eval(const PatchArgs<T> &a, const T *x, T *g, T *hvals,
                       EnergySink es, int mode, int lds_bytes, hipStream_t s);
template <typename T>
hipError_t launch_hvp(const PatchArgs<T> &a, const T *x, const T *v, T *y,
                      int mode, int lds_bytes, hipStream_t s);
// Zero the nb blocks bnd_blk[] of hv (if hv is given) and the entries of
// the nvb vertices bnd_vtx[] of vec: the slots that element-once patches
// add into with global atomics.
template <typename T>
hipError_t launch_zero_boundary(const int32_t *bnd_blk, int32_t nb, const int32_t *bnd_vtx,
                                int32_t nvb, T *hv, T *vec, hipStream_t s);

// Row-owner kernels for two-vertex radial terms (springs, runtime pairs) and
// vertex terms (inertia): one lane per block row, 64 rows per chunk.
constexpr int kRowThreads = 64;
constexpr int kRowsPerChunk = kRowThreads;
// Threads per workgroup of the row product kernels (HVP, Gauss-Newton),
// which share nothing between lanes: four waves, since the per-CU cap on
// workgroups holds single-wave groups to 4 waves per SIMD.
constexpr int kHvpThreads = 256;

template <typename T>
struct RowArgs {
    const PatchHdr *chunk;       // row chunks: v0, nown (rows), amap_cap (blocks)
    int32_t nchunk;
    int32_t nv;                  // rows
    const int32_t *rp0, *ci0;    // topology pattern
    const T *slot_rest;          // [nnzb_base] rest length of the spring behind
                                 // each block (< 0: no spring)
    const int32_t *sl_rows;      // product slices' rows (RowPlan; null: contiguous)
    const int32_t *sl_ptr;       // spring slices (RowPlan): entry offsets,
    const int32_t *sl_nb;        // neighbour vertices (null when sl_d16 is set)
    const int16_t *sl_d16;       // or their differences from the row
    const T *sl_rest;            // and rest lengths (< 0: padding)
    const T *x_tilde;            // null = no inertia
    const int32_t *fptr;         // [nv+1] offsets of each row's faces (faces on)
    const FaceInc *finc;         // each row's faces, by id (explicit kernel)
    const RowFace *rfinc;        // each row's faces, by slice list position (products)
    const int32_t *sf_ptr;       // [nslice+1] offsets of each slice's face list
    const SliceFace *sface;      // the slices' face lists
    const T *face_dm;            // [nf][4] row-major Dm^-1
    const T *face_area;          // [nf]
    T k, c, kappa, dhat;
    int32_t springs_on, inertia_on, faces_on;
    int32_t pairs_on;            // pair capacity > 0 (pairs may be active)
    int32_t lds_blocks;          // staging capacity per workgroup, in blocks
    const DevState *state;
    PatternBufs pat;
    // HVP only: per-workgroup partial sums of v.y into hvp_dot[blockIdx]
    // (null: none)
    double *hvp_dot;
    // vertex-face contacts: per-contact local terms formed by launch_vf_eval
    // / launch_vf_hvp (contact e's vertex m = 0..3 is the contact vertex, then
    // the face's three; strip 4e + m holds what row "vertex m" needs)
    T *vf_eval;                  // [4 cap][kVfStrip]
    T *vf_hvp;                   // [4 cap][kVfHvpStrip]
    int32_t *vf_ids;             // [cap][4] the contact's vertex ids
    int32_t *vf_slots;           // [4 cap][4] block offset, in row m, of vertex 0..3
    int32_t vf_stride;           // vertex-face capacity (0: contacts off)
};

// One contact seen from the row of its vertex m: the energy (kept in m = 0's
// strip only, else 0), the gradient's 3 entries of vertex m, then the
// Hessian's 3 rows of vertex m over the 12 columns (vertex, coordinate),
// row-major; for the product, H_e u_e's 3 entries of vertex m (and one pad).
constexpr int kVfHessOff = 4;
constexpr int kVfStrip = kVfHessOff + 36;
constexpr int kVfHvpStrip = 4;

template <typename T>
int rows_lds_bytes(int lds_blocks);
template <typename T>
hipError_t rows_grid(int lds_blocks, int nchunk, int faces, int pairs, int *grid_eval,
                     int *grid_hvp);
template <typename T>
hipError_t launch_eval_rows(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                            int grid, hipStream_t s);
// The rows that current pairs touch (after launch_eval_rows, same stream).
template <typename T>
hipError_t launch_eval_pair_rows(const RowArgs<T> &a, const T *x, T *g, T *hv, EnergySink es,
                                 int grid, hipStream_t s);
// Newton-CG direction formed inside the row HVP: every workgroup first
// takes the step that closes the previous update (cg_device.h: convergence
// or beta, from the partial sums of r.r; workgroup 0 records it in *st),
// then uses v = -r + beta d_old, and every row stores its v into d_new.  At
// iter 0 beta is 0 (d_old = -g).  With r null the HVP's operand is v itself.
template <typename T>
struct CgDir {
    const T *r = nullptr;
    const T *d_old = nullptr;
    T *d_new = nullptr;
    CgState *st = nullptr;
    const double *rr_parts = nullptr;  // partial sums of r.r after update iter - 1
    int32_t n_rr = 0;
    int32_t iter = 0;                  // updates completed before this direction
};
template <typename T>
hipError_t launch_hvp_rows(const RowArgs<T> &a, const T *x, const T *v, T *y, int grid,
                           hipStream_t s, const CgDir<T> &cg = CgDir<T>{});
// Vertex-face contact terms of the active buffer, one thread per contact;
// enqueued before the row kernels that add them (same stream).
template <typename T>
hipError_t launch_vf_eval(const RowArgs<T> &a, const T *x, hipStream_t s);
// H_e u_e of every contact of the active buffer (before
// launch_hvp_pair_rows, which adds them); with st set, nothing once the
// Newton-CG solve has ended.
template <typename T>
hipError_t launch_vf_hvp(const RowArgs<T> &a, const T *x, const T *u, const CgState *st,
                         hipStream_t s);
// The runtime contacts' part of y = H v for the rows they touch, added to
// what launch_hvp_rows stored (same stream, after it and launch_vf_hvp);
// with dot set, workgroup b stores its partial sum of v.(the added part)
// at dot[b].  grid = pair_rows_grid(the pattern's incidence capacity).
template <typename T>
hipError_t launch_hvp_pair_rows(const RowArgs<T> &a, const T *x, const T *v, T *y, double *dot,
                                int grid, const CgState *st, hipStream_t s);
template <typename T>
hipError_t launch_pairs_eval(const DevState *st, PatternBufs pat, const T *x,
                             T *g, T *hvals, EnergySink es, int nblocks,
                             T kappa, T dhat, hipStream_t s);
template <typename T>
hipError_t launch_pairs_hvp(const DevState *st, PatternBufs pat, const T *x,
                            const T *v, T *y, int nblocks, T kappa, T dhat,
                            hipStream_t s);
// Allow the patch kernels `bytes` of dynamic LDS (needed above 64 KiB).
hipError_t raise_lds_limits(int bytes);

// Exclusive scan: out[0..n] with out[n] = total.  tmp needs
// scan_tmp_size(n) int32 entries.
int64_t scan_tmp_size(int64_t n);
hipError_t launch_scan(const int32_t *in, int32_t *out, int32_t n, int32_t *tmp,
                       hipStream_t s);

// Pattern builder: topology rows from faces and springs.
struct PatternScratch {
    int32_t *cnt;      // [nv]
    int32_t *off;      // [nv + 1]
    int32_t *raw;      // [raw total]
    int32_t *cur;      // [nv]
    int32_t *ucnt;     // [nv]
    int32_t *tmp;      // scan scratch
};
hipError_t launch_pattern_count(int32_t nv, int32_t nf, const int32_t *faces,
                                int32_t ns, const int32_t *springs,
                                PatternScratch sc, hipStream_t s);
hipError_t launch_pattern_fill(int32_t nv, int32_t nf, const int32_t *faces,
                               int32_t ns, const int32_t *springs,
                               PatternScratch sc, hipStream_t s);
hipError_t launch_pattern_unique(int32_t nv, PatternScratch sc, hipStream_t s);
hipError_t launch_pattern_compact(int32_t nv, PatternScratch sc,
                                  const int32_t *row_ptr, int32_t *col_idx,
                                  hipStream_t s);

// Pair insertion (double-buffered).  Mutable views of buffers 1 and 2.
struct InsertBufs {
    int32_t *rp[3];
    int32_t *ci[3];
    int32_t *pairs[3];
    int32_t *pinc_ptr[3];
    int32_t *pinc[3];
    int32_t *pinc_row[3];
    int32_t *pnew[3];            // distinct new partners per row, kept until the
                                 // buffer is next written (the row kernels
                                 // read those of the active buffer)
    int32_t *trow[3];            // touched-row list, see PatternBufs::trow
    int4 *pslot[3];              // see PatternBufs::pslot
    int32_t *rins1[3];           // see PatternBufs::rins1
    int32_t *vf[3];              // vertex-face contacts: (vertex, face id)
    const int32_t *faces;        // [nf][3] mesh faces (contacts on)
    // Insertion tiles: runs of whole units (row chunks on the row path, fixed
    // row blocks on the patch path) of at most kInsTileRows rows.
    int32_t ntiles;
    const int32_t *tile_row;     // [ntiles+1] first row of each tile
    const int32_t *tile_unit;    // [ntiles+1] first chunk of each tile (row path)
    const int32_t *row_tile;     // [nv] tile of each row
    const int32_t *row_unit;     // [nv] chunk of each row (row path)
    unsigned long long *tstat;   // [ntiles * kStatStride] look-back status of each tile,
                                 // one per 128-byte line (polled by many workgroups)
    // The count kernel's output: per tile and count workgroup, the number of
    // the workgroup's entries in the tile and their offset in its part of
    // seg (tile-major); seg holds kInsWgEnt entries (two int4 each) per
    // workgroup; erank is scratch beside seg.
    int32_t max_wg;              // count workgroups at the contact capacity
    int32_t *hist;               // [ntiles][max_wg]
    int32_t *hoff;               // [ntiles][max_wg]
    int4 *seg;                   // [max_wg * kInsWgEnt][2]
    int32_t *erank;              // [max_wg * kInsWgEnt]
};
// A touched row whose active row has at most kMaxIns columns beyond its
// topology row has its topology terms evaluated by the main row kernel,
// each block moved to its active slot; its contact terms are added
// afterwards.  A row with more is evaluated whole by the touched-row kernel.
constexpr int kMaxIns = 4;
constexpr int kInsTileRows = 2048;   // rows per insertion tile, at most
constexpr int kStatStride = 16;      // 8-byte words per tile status
constexpr int kInsTileUnits = 256;   // row chunks per insertion tile, at most
constexpr int kInsMaxTiles = 8192;   // tiles per pattern, at most (a count of each in LDS)
constexpr int kInsMaxWg = 1024;      // count workgroups (of kThreads elements) per insert, at most
constexpr int kInsWgEnt = 4 * kThreads;  // incidence entries of a count workgroup, at most
// Tiles of the insertion over the row ranges `units` (contiguous, in row
// order, covering 0 .. nv): whole units up to kInsTileRows rows and
// kInsTileUnits units per tile when align_units, else kInsTileRows rows per
// tile.  Empty string on success, else why the pattern cannot be tiled.
struct InsertTiles {
    std::vector<int32_t> tile_row, tile_unit, row_tile, row_unit;
};
std::string build_insert_tiles(const std::vector<PatchHdr> &units, int32_t nv, bool align_units,
                               InsertTiles &out);
// complete_cols = 0 writes the columns of pair-touched rows only (row
// path); launch_complete_cols then fills in the other rows of the active
// buffer on demand.
hipError_t launch_insert(DevState *st, const int32_t *d_pairs, int32_t np, const int32_t *d_vf,
                         int32_t nvf, int32_t nv, int32_t nf, InsertBufs b, const PatchHdr *hdr,
                         int32_t npatch, int complete_cols, hipStream_t s);
hipError_t launch_complete_cols(DevState *st, InsertBufs b, const PatchHdr *hdr,
                                int32_t npatch, hipStream_t s);
hipError_t launch_restore_topology(DevState *st, hipStream_t s);

// ---------------------------------------------------------------------------
// Context internals for entry points defined outside lad_api.cpp.
// ---------------------------------------------------------------------------
// lad_eval_energy_grad_hess with the per-workgroup partial energies in
// `parts` (at least eval_scratch_doubles(ctx) doubles, every one written
// before it is read); argument checks and errors as that entry point.
lad_status eval_with_parts(lad_ctx *ctx, const void *d_x, double *d_energy, void *d_grad,
                           void *d_hvals, int64_t hvals_capacity_blocks, double *parts,
                           hipStream_t s);
int32_t eval_scratch_doubles(const lad_ctx *ctx);
int32_t ctx_device(const lad_ctx *ctx);        // device the context was built on
int32_t ctx_vf_capacity(const lad_ctx *ctx);
lad_status ctx_fail(lad_ctx *ctx, lad_status st, const char *msg);  // sets lad_last_error

}  // namespace lad
