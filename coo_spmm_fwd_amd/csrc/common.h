// common.h -- internal declarations of the coospmm HIP library (gfx950).
//
// The library implements the truly sparse COO layer of "Beyond Masked
// Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU" (Abstract):
// only the stored connections of W are kept and touched.  This header is
// private to the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/coospmm.h"

namespace csp {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------------------
// Layer state.  All arrays live in device memory owned by the layer.
//   canonical order  : entries sorted by (row, col)
//   transposed view  : canonical indices sorted by (col, row)
// ---------------------------------------------------------------------------
struct Workspace {
    // Sort and restructure scratch, sized at create from nnz and the shape.
    void *key_a = nullptr, *key_b = nullptr;  // nkey_cap keys (8 bytes each)
    int32_t *idx_a = nullptr, *idx_b = nullptr;  // nkey_cap
    uint32_t *u_a = nullptr, *u_b = nullptr;     // nkey_cap (flags / scans)
    uint32_t *hist = nullptr;                    // radix histograms + scan partials
    int32_t *rows_k = nullptr, *cols_k = nullptr;  // nnz: kept entries during restructure
    void *vals_k = nullptr;                        // nnz values
    int32_t *rp_k = nullptr;                       // out + 1: kept row offsets
    int32_t *rp_new = nullptr;                     // out + 1: row offsets of regrown positions
    uint64_t *acc_a = nullptr, *acc_b = nullptr;   // nnz: accepted regrow positions
    uint32_t *sel = nullptr;                       // kSelAllocWords: select state, flags, counts
    int64_t nkey_cap = 0;
    size_t hist_words = 0;
    // Position bitmaps of the restructure (when they fit, see plan_bitmap):
    // one bit per weight position, row-major, occ_row_words words per row
    // (a multiple of 8), occ_rows rows (out padded to a multiple of 64).
    // occ holds the current layer, occ_next is built by the restructure; each
    // has its exclusive rank array (occ_words + 1 entries).  tcnt holds the
    // per-column counts of the transposition tiles.
    bool bitmap = false;
    int64_t occ_words = 0, occ_row_words = 0, occ_rows = 0, tcnt_words = 0;
    uint32_t *occ = nullptr, *occ_next = nullptr, *occ_pref = nullptr, *occ_pref_next = nullptr;
    uint32_t *tcnt = nullptr;
    uint64_t *hash = nullptr;  // hash_slots: regrow candidates by position
    uint32_t *score = nullptr; // occ_words * 32: gradient regrow score keys (first use)
    int64_t hash_slots = 0, bm_batch_cap = 0;
};

// Batch rows per slice of a product call: one batch-minor chunk.  The
// operand workspace is sized for one slice at create; larger batches run
// slice after slice.
constexpr int64_t kSliceRows = 64;

struct ActBuffer {
    // Batch-minor copies of dense operands ([n][ld], ld <= kSliceRows) and
    // split-segment partial sums, allocated at create for one slice.
    void *a = nullptr, *b = nullptr;
    size_t bytes = 0;
    float *partial = nullptr;
    size_t partial_bytes = 0;
    int cus = 0;  // compute units of the layer's device (sizes persistent grids)
};

// Segments (rows for the row-order passes, columns for the transposed ones)
// are cut into tasks of at most kTaskChunk entries; one wavefront runs one
// task.  A segment cut into several tasks ("split") gets its output from a
// separate fixup launch that adds the tasks' partial sums in task order, so
// results do not depend on scheduling and no cross-wave fence is needed.
constexpr int kTaskChunk = 512;

// Packed row list (forward passes at batch widths of at most 4, one entry
// per lane).  Consecutive whole rows of at most kTaskChunk entries each are
// packed into one task, up to kPackEntries entries and at most the kPackSegs
// rows of one aligned row window; rows longer than kTaskChunk are split as
// in the plain list.  kPackEntries leaves room for the 8-entry alignment of
// the window the packed task body loads (kb rounded down to a multiple of 8).
constexpr int kPackSegs = 64;
constexpr int kPackEntries = kTaskChunk - 7;

// Layout of the small state buffer Workspace::sel (uint32 words).
constexpr int kSelAllocWords = 16384;
constexpr int kSelCounts = 12288;  // [0] row tasks, [1] column tasks, [2] split rows, [3] split columns,
                                   // [4] regrown positions taken, [5] the same before the current batch,
                                   // [6] packed row tasks, [7] split rows of the packed list,
                                   // [8 + 4 l + c] split segments of list l (rows, columns,
                                   // packed rows) in size class c
constexpr int kSplitClasses = 4;
constexpr int kSelClassWords = 8;
constexpr int kSelCountWords = kSelClassWords + 3 * kSplitClasses;  // words read back after a build
constexpr int kSelAsyncShort = kSelCounts + kSelCountWords;  // set when a restructure_async regrew too few

// Split segments are also kept by size class (their task count p): class 0
// p > 8, class 1 5..8, class 2 3..4, class 3 p = 2, so that one 16-wave
// workgroup can finish 1, 2, 4 or 8 of them (kGroupWaves >> c waves each).
__host__ __device__ inline int split_class(uint32_t p) { return p > 8 ? 0 : p > 4 ? 1 : p > 2 ? 2 : 3; }

// LDS tiles (fp32 layers, batch chunks of 33..64).  A view of the layer -- the
// rows over the X columns, or the columns (transposed view) over the dY
// columns -- is cut into tiles of kTileRows segments x kTileCols operand
// columns; one workgroup stages a tile's operand rows in LDS once and runs
// the tile's entries against them.  ptr[s * (ncb + 1) + k] is the first entry
// of segment s whose index is at least k * kTileCols (k = ncb: the segment's
// end); rows holds, per tile, its local segments ordered by their entry count
// in the tile (most first), so that the four segments a wave runs side by
// side have similar lengths.
constexpr int kTileCols = 512;
constexpr int kTileRows = 512;

struct Tiles {
    int32_t *ptr = nullptr;   // [nseg][ncb + 1]
    // [nrb * ncb][kTileRows], tile = row block * ncb + column block: per slot, in
    // the order the tile kernels take them, {first entry of the segment in the
    // tile, local segment << 16 | its entry count in the tile}
    int2 *slots = nullptr;
    int64_t nseg = 0, nop = 0, ncb = 0, nrb = 0;
};

struct TaskList {
    int4 *desc = nullptr;   // [cap] {segment, first entry, end entry, partial slot or -1}
    int4 *split = nullptr;  // [nseg] {segment, first task, task count, 0} of split segments
    int4 *split_cls = nullptr;  // [kSplitClasses][nseg] the same records by size class
    int64_t ncls[kSplitClasses] = {};  // records per class
    int32_t *seg_first = nullptr;  // [nseg + 1] first task of each segment
    int64_t count = 0;      // tasks in use
    int64_t nsplit = 0;     // split segments in use
    int64_t cap = 0;
};

}  // namespace csp

struct csp_layer {
    int64_t out = 0, in = 0, nnz = 0;
    int dtype = CSP_F32;
    int esz = 4;  // bytes per value
    int device = 0;
    int32_t *rows = nullptr, *cols = nullptr;
    void *vals = nullptr;
    int32_t *row_ptr = nullptr;
    int32_t *perm_c = nullptr, *rows_by_col = nullptr, *col_ptr = nullptr;
    void *vals_c = nullptr;  // values in transposed (col, row) order: vals_c[j] = vals[perm_c[j]]
    csp::TaskList row_tasks, col_tasks;
    csp::TaskList row_packed;  // whole rows packed per task (forward at B <= 4); seg_first unused
    // The packed list is built at create, and again by a restructure only
    // once a forward at B <= 4 has been asked for (narrow_seen); a forward
    // after a restructure that skipped it uses the plain row list.
    bool packed_valid = false, packed_pending = false, narrow_seen = false;
    bool created = false;  // set once sparse_layer_create has finished
    // Set when a restructure fails part way: its offsets, transposed view and
    // task lists may then describe a layer that was never completed, so every
    // later call but destroy refuses the layer.
    bool broken = false;
    // LDS tiles of the row view (value gradient, forward) and of the column
    // view (input gradient), and the partial sums of the segment passes:
    // [ncb][nseg][64] floats for the larger view.  Allocated at create for
    // fp32 layers with at least one tile per compute unit in both views.
    csp::Tiles tiles_r, tiles_c;
    float *tile_partial = nullptr;
    bool tile_ptr_ready = false;  // a bitmap rebuild wrote both views' tile offsets
    // Set by restructure_async: the host's task counts are those of the layer
    // before it, until tasks_ready reads back the new ones.
    bool counts_stale = false;
    // Set by restructure_async on a layer with LDS tiles, which leaves the task
    // lists unbuilt (the tile kernels never read them): tasks_ready builds
    // them before the first call that does.
    bool tasks_pending = false;
    // Host state cannot follow graph replays.  async_in_graph: a
    // restructure_async was captured, so any replay may have changed the
    // layer: every call that needs the task lists rebuilds (layers with tiles)
    // and reads them back first, and none may be captured.  tasks_in_graph: a
    // call that reads the task lists was captured, whose launch sizes a
    // captured restructure_async would make stale: capturing one is refused.
    bool async_in_graph = false, tasks_in_graph = false;
    csp::Workspace ws;
    csp::ActBuffer act;
    hipEvent_t time_before = nullptr, time_after = nullptr;  // one-shot main-kernel timing request
};

namespace csp {

// Error reporting (layer.hip).
csp_status set_error(csp_status st, const char *fmt, ...);
csp_status hip_error(hipError_t e, const char *what);

#define CSP_HIP(call)                                         \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return ::csp::hip_error(e_, #call); \
    } while (0)

#define CSP_LAUNCHED(what)                                    \
    do {                                                      \
        hipError_t e_ = hipGetLastError();                    \
        if (e_ != hipSuccess) return ::csp::hip_error(e_, what); \
    } while (0)

__host__ __device__ inline int bits_for(uint64_t max_value) {  // bits needed to represent max_value
    int b = 0;
    while (b < 64 && (max_value >> b) != 0) ++b;
    return b;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// sort.hip : integer building blocks (all enqueue on `s`, no host sync)
// ---------------------------------------------------------------------------
// Words of scratch that radix_sort_pairs / exclusive_scan need for n items.
size_t sort_hist_words(int64_t n);
// Stable LSD radix sort of (key, value) pairs on bits [0, end_bit).  Keys are
// uint32 (key_bytes 4) or uint64 (key_bytes 8).  Result in keys_out/vals_out;
// keys_tmp/vals_tmp are ping-pong scratch.  keys_in may equal keys_tmp.
csp_status radix_sort_pairs(int key_bytes, const void *keys_in, const int32_t *vals_in, void *keys_out,
                            int32_t *vals_out, void *keys_tmp, int32_t *vals_tmp, int64_t n, int end_bit,
                            uint32_t *hist, hipStream_t s);
// Exclusive prefix sum of n uint32 (in place allowed); optional *total on device.
csp_status exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *partials, uint32_t *total,
                              hipStream_t s);
// pref[i] = number of set bits in words[0..i), for i in [0, n] (pref has n + 1 entries).
csp_status exclusive_scan_popc(const uint32_t *words, uint32_t *pref, int64_t n, uint32_t *partials, hipStream_t s);
// ptr[i] = first index j with sorted[j] >= i, for i in [0, nseg]  (sorted int32, length n)
csp_status segment_offsets(const int32_t *sorted, int64_t n, int32_t *ptr, int64_t nseg, hipStream_t s);
csp_status fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// build.hip : canonical order and the transposed view
// ---------------------------------------------------------------------------
// Sorts input triples into the layer arrays; sets bit 1 of flags[0] on a bad
// index and bit 2 on a duplicate.
csp_status build_canonical(csp_layer *L, const int32_t *rows, const int32_t *cols, const void *vals,
                           uint32_t *flags, hipStream_t s);
// Rebuilds row_ptr, perm_c, rows_by_col, col_ptr, vals_c and both task lists
// from the canonical arrays.  Synchronizes on s (reads back the task counts).
csp_status build_index(csp_layer *L, hipStream_t s);
// The three task lists from row_ptr / col_ptr (plain rows, plain columns,
// packed rows; two or three launches, no host sync); the counts land in
// sel[kSelCounts + 0..3, 6..7] for set_task_counts.
csp_status build_task_lists(csp_layer *L, hipStream_t s, bool with_packed);
// Entry limit of a packed task of several rows for this layer.
int32_t pack_limit(const csp_layer *L);
// Takes the kSelCountWords counts read back from sel[kSelCounts]; checks the capacities.
csp_status set_task_counts(csp_layer *L, const uint32_t *counts);
// After restructure_async: builds the task lists if it left them pending,
// then reads back the task counts (a synchronization on s; refused on a
// stream that is being captured) and the short-regrow flag (which leaves the
// layer refused).  Nothing to do otherwise.
csp_status tasks_ready(csp_layer *L, hipStream_t s);
// Before a restructure: the short-regrow flag of a pending restructure_async
// is checked as in tasks_ready, but task lists it left pending stay so (the
// restructure rebuilds them).
csp_status async_checked(csp_layer *L, hipStream_t s);
// True while s is being captured into a graph.
bool stream_capturing(hipStream_t s);
// vals_c[j] = vals[perm_c[j]] after the canonical values changed.
csp_status refresh_column_values(csp_layer *L, hipStream_t s);
// Tiles of both views from row_ptr / cols and col_ptr / rows_by_col (four
// launches, no host sync); nothing to do for a layer without tiles.
csp_status build_tiles(csp_layer *L, hipStream_t s);
inline int64_t task_cap(int64_t nseg, int64_t nnz) { return nseg + (nnz + kTaskChunk - 1) / kTaskChunk; }

// ---------------------------------------------------------------------------
// spmm.hip : the three products
// ---------------------------------------------------------------------------
// Forward epilogue: y = sum + bias (bias optional), pre = y (optional), out = GELU(y) if gelu else y.
struct FwdEpilogue {
    const void *bias = nullptr;
    void *pre = nullptr;
    int gelu = 0;
};
// Workspace of a forward call: the batch-minor copy of the operand slice and
// the split tasks' partial sums.  launch_fwd uses the layer's own workspace
// unless one is passed.
struct FwdWork {
    void *operand = nullptr;
    float *partial = nullptr;
};
// Caller-held batch-minor copies [n][ld], ld = the power of two >= B (one
// slice: 2 <= B <= 64), of the gathered operands (used in place of the call's
// own copy) and of the output (written beside the row-major one; pad slots
// b >= B untouched): spmm_fwd_bm and spmm_bwd_bm.
struct BmIO {
    const void *xt = nullptr;   // X (forward, value gradient)
    const void *dyt = nullptr;  // dY (input gradient, value gradient)
    void *outt = nullptr;       // Y (forward) or dX (input gradient)
};
// fe == nullptr: plain forward.  act_in != nullptr: the input gradient is
// multiplied by GELU'(act_in[b, c]) (act_in [B, in], layer dtype).
csp_status launch_fwd(csp_layer *L, const void *X, int64_t B, void *Y, const FwdEpilogue *fe, hipStream_t s,
                      const FwdWork *work = nullptr, const BmIO &io = BmIO{});
// Bytes of each FwdWork buffer a forward of B rows needs (its largest slice).
csp_status fwd_work_bytes(csp_layer *L, int64_t B, size_t *operand_bytes, size_t *partial_bytes);
csp_status launch_bwd_input(csp_layer *L, const void *dY, int64_t B, void *dX, const void *act_in, hipStream_t s,
                            const BmIO &io = BmIO{});
csp_status launch_bwd_values(csp_layer *L, const void *dY, const void *X, int64_t B, float *dW, hipStream_t s,
                             const BmIO &io = BmIO{});
csp_status launch_bwd(csp_layer *L, const void *dY, const void *X, int64_t B, void *dX, float *dW, const void *act_in,
                      hipStream_t s, const BmIO &io = BmIO{});
// The batch-minor copy [n][ld] of a row-major operand [B, n] (esz bytes per element).
csp_status batch_minor_copy(int esz, int64_t B, const void *src, int64_t n, void *dst, hipStream_t s);

// ---------------------------------------------------------------------------
// restructure.hip
// ---------------------------------------------------------------------------
// occupancy.hip: chooses the bitmap restructure for this shape (fills the
// Workspace sizes, allocates nothing); scratch words it needs in hist; sets
// the row-major bitmap from the canonical arrays; the restructure itself.
bool plan_bitmap(csp_layer *L);
size_t bitmap_hist_words(const csp_layer *L);
csp_status occupancy_init(csp_layer *L, hipStream_t s);
csp_status restructure_bitmap(csp_layer *L, int64_t n_prune, uint64_t seed, uint64_t step, uint32_t regrow_bits,
                              hipStream_t s);
// The same step with one batch of candidates and no host synchronization
// (restructure_async); the Philox step is read from and advanced at step_dev.
csp_status restructure_bitmap_async(csp_layer *L, int64_t n_prune, uint64_t seed, const uint64_t *step_dev,
                                    uint32_t regrow_bits, hipStream_t s);
// Candidates of that one batch; 0 when it would not fit the workspace.
int64_t async_batch(const csp_layer *L, int64_t n_prune);
// Prune as restructure; regrow the empty positions with the largest |dY^T X|.
csp_status restructure_gradient(csp_layer *L, int64_t n_prune, const void *dY, const void *X, int64_t B,
                                uint32_t regrow_bits, hipStream_t s);
csp_status run_restructure(csp_layer *L, int64_t n_prune, uint64_t seed, uint64_t step, uint32_t regrow_bits,
                           hipStream_t s);
int64_t regrow_batch_cap(const csp_layer *L);

}  // namespace csp
