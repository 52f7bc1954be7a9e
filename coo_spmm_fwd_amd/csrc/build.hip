// build.hip -- the COO builder: canonical (row, col) order, row offsets, and
// the transposed (col, row) view used by the input-gradient pass.
//
// "Beyond Masked Sparsity: SNACK ..." (Abstract) stores only the non-zero
// connections, as COO.  Here the triples are put in row-major canonical order
// with a flat key row*in + col (one LSD radix sort), so each output row is a
// contiguous segment; a second stable sort by column of the canonical indices
// gives the column segments.  Offsets come from a binary search per segment.
#include <cstdlib>

#include "common.h"
#include "device_util.h"

namespace csp {
namespace {

template <typename K>
__global__ void k_make_keys(const int32_t *__restrict__ rows, const int32_t *__restrict__ cols, int64_t nnz,
                            int64_t out, int64_t in, K *__restrict__ keys, int32_t *__restrict__ idx,
                            uint32_t *flags)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    int32_t r = rows[k], c = cols[k];
    bool bad = r < 0 || r >= out || c < 0 || c >= in;
    if (bad) atomicOr(flags, 2u);
    keys[k] = bad ? K(0) : (K)r * (K)in + (K)c;
    idx[k] = (int32_t)k;
}

template <typename K, typename V>
__global__ void k_gather_canon(const K *__restrict__ keys, const int32_t *__restrict__ src, int64_t nnz, int64_t in,
                               const V *__restrict__ vals_in, int32_t *__restrict__ rows, int32_t *__restrict__ cols,
                               V *__restrict__ vals, uint32_t *flags)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    K key = keys[k];
    rows[k] = (int32_t)(key / (K)in);
    cols[k] = (int32_t)(key % (K)in);
    vals[k] = vals_in[src[k]];
    if (k > 0 && keys[k - 1] == key) atomicOr(flags, 4u);
}

__global__ void k_col_keys(const int32_t *__restrict__ cols, int64_t nnz, uint32_t *__restrict__ keys,
                           int32_t *__restrict__ idx)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    keys[k] = (uint32_t)cols[k];
    idx[k] = (int32_t)k;
}

__global__ void k_rows_by_col(const int32_t *__restrict__ rows, const int32_t *__restrict__ perm, int64_t nnz,
                              int32_t *__restrict__ rows_by_col)
{
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < nnz) rows_by_col[j] = rows[perm[j]];
}

template <typename V>
__global__ void k_gather_vals(const V *__restrict__ vals, const int32_t *__restrict__ perm, int64_t n,
                              V *__restrict__ out)
{
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) out[j] = vals[perm[j]];
}

// Tasks per segment: one for a segment of at most kTaskChunk entries (also
// for an empty one, which still owns its zero output), else one per chunk.
__device__ __forceinline__ uint32_t seg_pieces(const int32_t *ptr, int64_t i)
{
    const int64_t len = (int64_t)ptr[i + 1] - ptr[i];
    return len <= kTaskChunk ? 1u : (uint32_t)((len + kTaskChunk - 1) / kTaskChunk);
}

// The three task lists (plain rows, plain columns, packed rows) are built by
// the same launches: blocks [0, tiles0) work on list 0, the next tiles1 on
// list 1 and the rest on list 2.  Lists 0 and 1 take one segment per
// thread; list 2 takes one window of kPackSegs rows per workgroup.
constexpr int kTaskThreads = 1024;
constexpr int kLists = 3;

struct TaskBuild {
    const int32_t *ptr[kLists];
    int64_t nseg[kLists];
    int64_t tiles[kLists];
    int4 *desc[kLists];
    int4 *split[kLists];
    int4 *split_cls[kLists];     // class c at c * cls_stride
    int64_t cls_stride[kLists];
    int32_t *seg_first[kLists];  // list 2: none
    int64_t cap[kLists];
    uint32_t *partials[kLists];  // tiles + 1 words each
    uint32_t *counts;            // [0], [1], [6] tasks; [2], [3], [7] split segments
    int64_t rows2;               // rows of list 2 (its nseg counts windows)
    int32_t pack_limit;          // entries of a task of several rows, at most kPackEntries
};
__device__ __forceinline__ int task_count_word(int l) { return l < 2 ? l : 6; }
__device__ __forceinline__ int split_count_word(int l) { return l < 2 ? 2 + l : 7; }

// One split segment's record, in the list's split array and in its class.
__device__ __forceinline__ void emit_split(const TaskBuild &tb, int l, int4 rec, uint32_t p)
{
    tb.split[l][atomicAdd(&tb.counts[split_count_word(l)], 1u)] = rec;
    const int c = split_class(p);
    const uint32_t k = atomicAdd(&tb.counts[kSelClassWords + kSplitClasses * l + c], 1u);
    tb.split_cls[l][c * tb.cls_stride[l] + k] = rec;
}

__device__ __forceinline__ void task_tile(const TaskBuild &tb, int &l, int64_t &tile)
{
    tile = blockIdx.x;
    l = 0;
    while (l < kLists - 1 && tile >= tb.tiles[l]) tile -= tb.tiles[l++];
}

// Greedy packing of the rows [s0, s1) of one window (kPackSegs rows), in
// order, by one wave: lane j loads the bounds of row s0 + j, and every lane
// walks the window reading them with readlane (no memory access inside the
// walk).  A row longer than kTaskChunk closes the open task and is cut into
// kTaskChunk pieces (a split row, as in the plain list).  Any other row joins
// the open task unless that would take the task past pack_limit
// (<= kPackEntries) entries; then the open task is closed first.  Empty rows
// join like any other (the task stores their zero outputs).  Returns the
// number of tasks; with kEmit, lane 0 also writes them from descriptor f on:
// {first row, first entry, end entry, -(rows)} for a packed task (-1: one
// row, as in the plain list) and {row, first entry, end entry, task index}
// for each piece of a split row, plus the split records.
template <bool kEmit>
__device__ uint32_t pack_window(const TaskBuild &tb, int64_t s0, int64_t s1, int32_t f)
{
    const int lane = threadIdx.x & 63;
    const int nr = (int)(s1 - s0);  // 1 .. kPackSegs
    // fields used in the walk, read once (the build struct may sit in private memory)
    const int32_t *ptr = tb.ptr[2];
    int4 *const desc = tb.desc[2];
    const int64_t cap = tb.cap[2];
    const int32_t lim = tb.pack_limit;
    const int32_t ej = ptr[s0 + (lane < nr ? lane + 1 : nr)];  // end of row s0 + lane
    const bool w0 = kEmit && lane == 0;
    uint32_t n = 0;
    int32_t open = -1, open_kb = 0, cnt = 0;
    int32_t b = __builtin_amdgcn_readfirstlane(ptr[s0]);
    for (int j = 0; j < nr; ++j) {
        const int32_t r = (int32_t)(s0 + j);
        const int32_t e = __builtin_amdgcn_readlane(ej, j), len = e - b;
        if (len > kTaskChunk) {
            if (cnt) {
                if (w0 && f + n < cap) desc[f + n] = make_int4(open, open_kb, b, -cnt);
                ++n;
                cnt = 0;
            }
            const uint32_t p = (uint32_t)((len + kTaskChunk - 1) / kTaskChunk);
            if (w0) {
                for (uint32_t k = 0; k < p && (int64_t)f + n + k < cap; ++k) {
                    const int32_t kb = b + (int32_t)k * kTaskChunk;
                    const int32_t ke = kb + kTaskChunk < e ? kb + kTaskChunk : e;
                    desc[f + n + k] = make_int4(r, kb, ke, (int32_t)(f + n + k));
                }
                emit_split(tb, 2, make_int4(r, (int32_t)(f + n), (int32_t)p, 0), p);
            }
            n += p;
        } else {
            if (cnt && e - open_kb > lim) {
                if (w0 && f + n < cap) desc[f + n] = make_int4(open, open_kb, b, -cnt);
                ++n;
                cnt = 0;
            }
            if (!cnt) {
                open = r;
                open_kb = b;
            }
            ++cnt;
        }
        b = e;
    }
    if (cnt) {
        if (w0 && f + n < cap) desc[f + n] = make_int4(open, open_kb, b, -cnt);
        ++n;
    }
    return n;
}

// Work item of a thread: a segment of lists 0 and 1 (item = thread), a
// window of kPackSegs rows of list 2 (item = the block's first wave; nseg[2]
// counts windows, rows2 rows).  The walk is scalar work, and a compute unit
// has one scalar unit for all its waves, so one window per workgroup spreads
// the walks over the compute units (16 windows per workgroup measured 12 us
// per launch on a 4096-row layer).  item_tasks returns the item's task count
// in the lane that owns it (every lane of lists 0 and 1, lane 0 of the
// list-2 wave) and 0 elsewhere.
__device__ __forceinline__ int64_t item_index(const TaskBuild &tb, int l, int64_t tile)
{
    if (l < 2) return tile * kTaskThreads + threadIdx.x;
    return threadIdx.x < 64 ? tile : tb.nseg[2];
}
__device__ __forceinline__ uint32_t item_tasks(const TaskBuild &tb, int l, int64_t i)
{
    if (i >= tb.nseg[l]) return 0u;
    if (l < 2) return seg_pieces(tb.ptr[l], i);
    const int64_t s0 = i * kPackSegs, s1 = s0 + kPackSegs < tb.rows2 ? s0 + kPackSegs : tb.rows2;
    const uint32_t n = pack_window<false>(tb, s0, s1, 0);
    return (threadIdx.x & 63) == 0 ? n : 0u;
}

__global__ __launch_bounds__(kTaskThreads) void k_tasks_count(TaskBuild tb)
{
    __shared__ uint32_t lds[17];
    int l;
    int64_t tile;
    task_tile(tb, l, tile);
    const int64_t i = item_index(tb, l, tile);
    uint32_t total;
    block_exclusive_scan(item_tasks(tb, l, i), lds, &total);
    if (threadIdx.x == 0) tb.partials[l][tile] = total;
    if (blockIdx.x == 0 && threadIdx.x < kLists) tb.counts[split_count_word(threadIdx.x)] = 0;
    if (blockIdx.x == 0 && threadIdx.x < kLists * kSplitClasses) tb.counts[kSelClassWords + threadIdx.x] = 0;
}

// kLists blocks: block l scans the tile sums of list l in place and stores
// the list's task count (lists 0 and 1 also as seg_first[nseg]).
__global__ __launch_bounds__(kTaskThreads) void k_tasks_scan(TaskBuild tb)
{
    __shared__ uint32_t lds[17];
    const int l = blockIdx.x;
    uint32_t *part = tb.partials[l];
    const int64_t nb = tb.tiles[l];
    const int64_t per = ceil_div(nb, kTaskThreads);
    const int64_t b0 = (int64_t)threadIdx.x * per;
    uint32_t sum = 0;
    for (int64_t i = b0; i < b0 + per && i < nb; ++i) sum += part[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan(sum, lds, &total);
    for (int64_t i = b0; i < b0 + per && i < nb; ++i) {
        const uint32_t v = part[i];
        part[i] = run;
        run += v;
    }
    if (threadIdx.x == 0) {
        tb.counts[task_count_word(l)] = total;
        if (l < 2) tb.seg_first[l][tb.nseg[l]] = (int32_t)total;
    }
}

// kPrefix: the tile sums are still raw (k_tasks_scan skipped); each block
// adds up those of the tiles before it, and the last tile of a list stores
// the list's task count as k_tasks_scan would.  Used up to kPrefixTaskTiles
// tiles per list.
constexpr int64_t kPrefixTaskTiles = 1024;
template <bool kPrefix>
__global__ __launch_bounds__(kTaskThreads) void k_tasks_emit(TaskBuild tb)
{
    __shared__ uint32_t lds[17];
    int l;
    int64_t tile;
    task_tile(tb, l, tile);
    const int64_t i = item_index(tb, l, tile);
    const bool live = i < tb.nseg[l];
    const uint32_t p = item_tasks(tb, l, i);
    uint32_t before, total;
    if constexpr (kPrefix) {
        uint32_t v = 0;
        for (int64_t j = threadIdx.x; j < tile; j += kTaskThreads) v += tb.partials[l][j];
        block_exclusive_scan(v, lds, &before);
    } else {
        before = tb.partials[l][tile];
    }
    const int32_t f = (int32_t)(block_exclusive_scan(p, lds, &total) + before);
    if (kPrefix && tile == tb.tiles[l] - 1 && threadIdx.x == 0) {
        tb.counts[task_count_word(l)] = before + total;
        if (l < 2) tb.seg_first[l][tb.nseg[l]] = (int32_t)(before + total);
    }
    if (!live) return;
    if (l == 2) {  // the window's first descriptor is its lane 0's offset
        const int64_t s0 = i * kPackSegs, s1 = s0 + kPackSegs < tb.rows2 ? s0 + kPackSegs : tb.rows2;
        pack_window<true>(tb, s0, s1, __builtin_amdgcn_readfirstlane(f));
        return;
    }
    tb.seg_first[l][i] = f;
    const int32_t b = tb.ptr[l][i], e = tb.ptr[l][i + 1];
    for (int32_t j = 0; j < (int32_t)p && (int64_t)f + j < tb.cap[l]; ++j) {
        const int32_t kb = b + j * kTaskChunk;
        const int32_t ke = kb + kTaskChunk < e ? kb + kTaskChunk : e;
        tb.desc[l][f + j] = make_int4((int32_t)i, kb, ke, p > 1 ? f + j : -1);
    }
    if (p > 1) emit_split(tb, l, make_int4((int32_t)i, f, (int32_t)p, 0), p);
}

}  // namespace

// Rows are packed only while the layer still has about as many tasks as the
// device has wave slots (32 per CU): packing a layer with fewer entries per
// slot would only lengthen each wave's chain of dependent loads.
// COOSPMM_PACK_LIMIT overrides the entry limit (1 turns packing off).
int32_t pack_limit(const csp_layer *L)
{
    int64_t lim = L->nnz / ((int64_t)(L->act.cus > 0 ? L->act.cus : 256) * 32);
    if (const char *e = std::getenv("COOSPMM_PACK_LIMIT")) lim = std::atoll(e);
    return (int32_t)(lim < 1 ? 1 : lim > kPackEntries ? kPackEntries : lim);
}

// Lists 0 and 1: seg_first[0..nseg) = exclusive scan of the per-segment task
// counts, seg_first[nseg] = the total; then one descriptor per task and one
// record per split segment (their order is irrelevant: each record is
// self-contained).  List 2 packs windows of rows (pack_window).
csp_status build_task_lists(csp_layer *L, hipStream_t s, bool with_packed)
{
    L->packed_pending = with_packed;
    L->tasks_pending = false;
    if (!with_packed) L->packed_valid = false;  // the list no longer matches the layer
    TaskBuild tb;
    TaskList *T[kLists] = {&L->row_tasks, &L->col_tasks, &L->row_packed};
    const int32_t *ptr[kLists] = {L->row_ptr, L->col_ptr, L->row_ptr};
    const int64_t nseg[kLists] = {L->out, L->in, with_packed ? ceil_div(L->out, kPackSegs) : 0};
    uint32_t *part = L->ws.hist;
    for (int l = 0; l < kLists; ++l) {
        tb.ptr[l] = ptr[l];
        tb.nseg[l] = nseg[l];
        tb.tiles[l] = l < 2 ? ceil_div(nseg[l], kTaskThreads) : nseg[l];  // list 2: a window per workgroup
        tb.desc[l] = T[l]->desc;
        tb.split[l] = T[l]->split;
        tb.split_cls[l] = T[l]->split_cls;
        tb.cls_stride[l] = l == 1 ? L->in : L->out;
        tb.seg_first[l] = T[l]->seg_first;
        tb.cap[l] = T[l]->cap;
        tb.partials[l] = part;
        part += tb.tiles[l] + 1;
    }
    tb.rows2 = L->out;
    tb.pack_limit = pack_limit(L);
    tb.counts = L->ws.sel + kSelCounts;
    const unsigned grid = (unsigned)(tb.tiles[0] + tb.tiles[1] + tb.tiles[2]);
    k_tasks_count<<<grid, kTaskThreads, 0, s>>>(tb);
    CSP_LAUNCHED("k_tasks_count");
    if (tb.tiles[0] <= kPrefixTaskTiles && tb.tiles[1] <= kPrefixTaskTiles && tb.tiles[2] <= kPrefixTaskTiles) {
        k_tasks_emit<true><<<grid, kTaskThreads, 0, s>>>(tb);
    } else {
        k_tasks_scan<<<kLists, kTaskThreads, 0, s>>>(tb);
        CSP_LAUNCHED("k_tasks_scan");
        k_tasks_emit<false><<<grid, kTaskThreads, 0, s>>>(tb);
    }
    CSP_LAUNCHED("k_tasks_emit");
    return CSP_OK;
}

csp_status set_task_counts(csp_layer *L, const uint32_t *counts)
{
    L->row_tasks.count = counts[0];
    L->col_tasks.count = counts[1];
    L->row_tasks.nsplit = counts[2];
    L->col_tasks.nsplit = counts[3];
    L->row_packed.count = counts[6];
    L->row_packed.nsplit = counts[7];
    L->packed_valid = L->packed_pending;
    TaskList *T[3] = {&L->row_tasks, &L->col_tasks, &L->row_packed};
    for (int l = 0; l < 3; ++l)
        for (int c = 0; c < kSplitClasses; ++c) T[l]->ncls[c] = counts[kSelClassWords + kSplitClasses * l + c];
    if (L->row_packed.count > L->row_packed.cap)
        return set_error(CSP_ERR_HIP, "packed task list overflow (%lld/%lld)", (long long)L->row_packed.count,
                         (long long)L->row_packed.cap);
    if (L->row_tasks.count > L->row_tasks.cap || L->col_tasks.count > L->col_tasks.cap)
        return set_error(CSP_ERR_HIP, "task list overflow (%lld/%lld, %lld/%lld)", (long long)L->row_tasks.count,
                         (long long)L->row_tasks.cap, (long long)L->col_tasks.count, (long long)L->col_tasks.cap);
    return CSP_OK;
}

// The counts and the short-regrow flag that restructure_async left on the
// device, read back; the flag leaves the layer refused.
static csp_status read_async_counts(csp_layer *L, hipStream_t s, uint32_t *counts)
{
    static_assert(kSelAsyncShort == kSelCounts + kSelCountWords, "the flag follows the counts");
    CSP_HIP(hipMemcpyAsync(counts, L->ws.sel + kSelCounts, (kSelCountWords + 1) * sizeof(uint32_t),
                           hipMemcpyDeviceToHost, s));
    CSP_HIP(hipStreamSynchronize(s));
    L->counts_stale = false;
    if (counts[kSelCountWords]) {
        L->broken = true;
        return set_error(CSP_ERR_INVALID_ARG, "a restructure_async found fewer empty positions than it pruned in "
                                              "its batch of candidates; the layer is incomplete");
    }
    return CSP_OK;
}

bool stream_capturing(hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

// A captured restructure_async leaves the layer's task state unknown after
// any replay: it is taken as pending at every call.
static void assume_replayed(csp_layer *L)
{
    if (!L->async_in_graph) return;
    L->counts_stale = true;
    if (L->tile_partial) L->tasks_pending = true;
}

csp_status tasks_ready(csp_layer *L, hipStream_t s)
{
    if (stream_capturing(s)) {
        if (L->async_in_graph)
            return set_error(CSP_ERR_INVALID_ARG, "this call reads the layer's task lists, which a captured "
                                                  "restructure_async changes at every replay: it cannot be captured");
        if (L->counts_stale || L->tasks_pending)
            return set_error(CSP_ERR_INVALID_ARG, "this call needs the task lists that restructure_async left "
                                                  "pending: call sparse_layer_sync before capturing it");
        L->tasks_in_graph = true;
        return CSP_OK;
    }
    assume_replayed(L);
    if (!L->counts_stale && !L->tasks_pending) return CSP_OK;
    if (L->tasks_pending) {
        const csp_status st = build_task_lists(L, s, L->narrow_seen);
        if (st != CSP_OK) return st;
    }
    uint32_t counts[kSelCountWords + 1] = {};  // the counts, then the short-regrow flag
    const csp_status st = read_async_counts(L, s, counts);
    if (st != CSP_OK) return st;
    return set_task_counts(L, counts);
}

csp_status async_checked(csp_layer *L, hipStream_t s)
{
    assume_replayed(L);
    if (!L->tasks_pending) return tasks_ready(L, s);
    if (!L->counts_stale) return CSP_OK;
    uint32_t counts[kSelCountWords + 1] = {};
    return read_async_counts(L, s, counts);  // the counts wait for the task lists
}

// ------------------------------------------------------------- LDS tiles
// ptr[s * (ncb + 1) + k] = first entry of segment s whose index is at least
// k * kTileCols, one wave per segment: entry e of block b sets the slots k of
// (b', b], b' the block of the segment's previous entry (-1 at its first
// entry), then the slots after the last entry's block (all of them for an
// empty segment) get the segment's end.  Every slot is written exactly once.
__global__ __launch_bounds__(256) void k_tile_ptr(const int32_t *__restrict__ seg_ptr, const int32_t *__restrict__ idx,
                                                  int64_t nseg, int64_t ncb, int32_t *__restrict__ tile_ptr)
{
    const int64_t sg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (sg >= nseg) return;
    const int lane = threadIdx.x & 63;
    const int32_t beg = seg_ptr[sg], end = seg_ptr[sg + 1];
    int32_t *t = tile_ptr + sg * (ncb + 1);
    int32_t carry = -1;  // block of the entry before the current chunk
    for (int32_t base = beg; base < end; base += kWave) {
        const int32_t e = base + lane;
        const int32_t b = e < end ? idx[e] / kTileCols : (int32_t)ncb;
        const int32_t up = __shfl_up(b, 1, kWave);
        const int32_t prev = lane == 0 ? carry : up;
        if (e < end)
            for (int32_t k = prev + 1; k <= b; ++k) t[k] = e;
        carry = __shfl(b, kWave - 1, kWave);
    }
    const int32_t last = end > beg ? idx[end - 1] / kTileCols : -1;
    for (int64_t k = last + 1 + lane; k <= ncb; k += kWave) t[k] = end;
}

// One block per tile (tile = row block * ncb + column block): its local
// segments by entry count in the tile, most first (counts of kTileRows - 2 and
// more share a bin; segments past the view count -1 and come last), by a
// counting sort.  Segments of equal count land in any order: the order only
// pairs segments for the waves of the tile kernels, whose sums do not depend
// on it.  Each slot records its segment's entry range in the tile beside the
// segment, so that a tile kernel's wave finds its work with one load.  One
// launch takes both views: the row view's tiles first, then the column
// view's.
struct TileRowsView {
    const int32_t *tile_ptr;
    int64_t nseg, ncb, ntiles;
    int2 *slots;
};

__global__ __launch_bounds__(kTileRows) void k_tile_rows(TileRowsView v0, TileRowsView v1)
{
    static_assert(kTileRows % kWave == 0 && kTileRows <= 1024, "one thread per row and per bin");
    __shared__ uint32_t bin_n[kTileRows], bin_at[kTileRows];
    __shared__ uint32_t lds[17];
    const bool first = blockIdx.x < v0.ntiles;
    const int32_t *__restrict__ tile_ptr = first ? v0.tile_ptr : v1.tile_ptr;
    int2 *__restrict__ slots = first ? v0.slots : v1.slots;
    const int64_t nseg = first ? v0.nseg : v1.nseg, ncb = first ? v0.ncb : v1.ncb;
    const int64_t tile = first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - v0.ntiles, rb = tile / ncb,
                  cb = tile - rb * ncb;
    const int l = threadIdx.x;
    const int64_t r = rb * kTileRows + l;
    const int32_t beg = r < nseg ? tile_ptr[r * (ncb + 1) + cb] : 0;
    const int32_t c = r < nseg ? tile_ptr[r * (ncb + 1) + cb + 1] - beg : -1;
    const int bin = (c < kTileRows - 2 ? c : kTileRows - 2) + 1;  // 0 .. kTileRows - 1
    bin_n[l] = 0;
    __syncthreads();
    atomicAdd(&bin_n[bin], 1u);
    __syncthreads();
    // bins in descending count order: thread l holds bin kTileRows - 1 - l
    uint32_t total;
    const uint32_t before = block_exclusive_scan(bin_n[kTileRows - 1 - l], lds, &total);
    bin_at[kTileRows - 1 - l] = before;
    __syncthreads();
    const uint32_t pos = atomicAdd(&bin_at[bin], 1u);
    static_assert(kTileRows <= 32768 && kTileCols < 65536, "segment and count share one word");
    slots[tile * kTileRows + pos] = make_int2(beg, (l << 16) | (c > 0 ? c : 0));
}

csp_status build_tiles(csp_layer *L, hipStream_t s)
{
    if (!L->tile_partial) return CSP_OK;
    const Tiles *T[2] = {&L->tiles_r, &L->tiles_c};
    const int32_t *seg_ptr[2] = {L->row_ptr, L->col_ptr}, *idx[2] = {L->cols, L->rows_by_col};
    TileRowsView tv[2];
    for (int v = 0; v < 2; ++v) {
        if (!L->tile_ptr_ready) {
            k_tile_ptr<<<(unsigned)ceil_div(T[v]->nseg, 4), 256, 0, s>>>(seg_ptr[v], idx[v], T[v]->nseg, T[v]->ncb,
                                                                         T[v]->ptr);
            CSP_LAUNCHED("k_tile_ptr");
        }
        tv[v] = TileRowsView{T[v]->ptr, T[v]->nseg, T[v]->ncb, T[v]->nrb * T[v]->ncb, T[v]->slots};
    }
    k_tile_rows<<<(unsigned)(tv[0].ntiles + tv[1].ntiles), kTileRows, 0, s>>>(tv[0], tv[1]);
    CSP_LAUNCHED("k_tile_rows");
    L->tile_ptr_ready = false;
    return CSP_OK;
}

csp_status refresh_column_values(csp_layer *L, hipStream_t s)
{
    if (L->nnz == 0) return CSP_OK;
    const unsigned grid = (unsigned)ceil_div(L->nnz, 256);
    if (L->esz == 4)
        k_gather_vals<uint32_t><<<grid, 256, 0, s>>>((const uint32_t *)L->vals, L->perm_c, L->nnz,
                                                     (uint32_t *)L->vals_c);
    else
        k_gather_vals<uint16_t><<<grid, 256, 0, s>>>((const uint16_t *)L->vals, L->perm_c, L->nnz,
                                                     (uint16_t *)L->vals_c);
    CSP_LAUNCHED("k_gather_vals");
    return CSP_OK;
}

csp_status build_index(csp_layer *L, hipStream_t s)
{
    const int64_t nnz = L->nnz;
    csp_status st = segment_offsets(L->rows, nnz, L->row_ptr, L->out, s);
    if (st != CSP_OK) return st;
    if (nnz > 0) {
        const unsigned grid = (unsigned)ceil_div(nnz, 256);
        k_col_keys<<<grid, 256, 0, s>>>(L->cols, nnz, L->ws.u_a, L->ws.idx_a);
        CSP_LAUNCHED("k_col_keys");
        st = radix_sort_pairs(4, L->ws.u_a, L->ws.idx_a, L->ws.key_a, L->perm_c, L->ws.key_b, L->ws.idx_b, nnz,
                              bits_for((uint64_t)(L->in - 1)), L->ws.hist, s);
        if (st != CSP_OK) return st;
        k_rows_by_col<<<grid, 256, 0, s>>>(L->rows, L->perm_c, nnz, L->rows_by_col);
        CSP_LAUNCHED("k_rows_by_col");
        st = refresh_column_values(L, s);
        if (st != CSP_OK) return st;
    }
    st = segment_offsets((const int32_t *)L->ws.key_a, nnz, L->col_ptr, L->in, s);
    if (st != CSP_OK) return st;

    st = build_task_lists(L, s, !L->created || L->narrow_seen);
    if (st != CSP_OK) return st;
    uint32_t counts[kSelCountWords] = {};
    CSP_HIP(hipMemcpyAsync(counts, L->ws.sel + kSelCounts, sizeof counts, hipMemcpyDeviceToHost, s));
    CSP_HIP(hipStreamSynchronize(s));
    return set_task_counts(L, counts);
}

template <typename K>
static csp_status build_canonical_k(csp_layer *L, const int32_t *rows, const int32_t *cols, const void *vals,
                                    uint32_t *flags, hipStream_t s)
{
    const int64_t nnz = L->nnz;
    const unsigned grid = (unsigned)ceil_div(nnz, 256);
    K *ka = (K *)L->ws.key_a, *kb = (K *)L->ws.key_b;
    k_make_keys<K><<<grid, 256, 0, s>>>(rows, cols, nnz, L->out, L->in, ka, L->ws.idx_a, flags);
    CSP_LAUNCHED("k_make_keys");
    const int end_bit = bits_for((uint64_t)(L->out * L->in - 1));
    csp_status st = radix_sort_pairs((int)sizeof(K), ka, L->ws.idx_a, kb, L->ws.idx_b, ka, L->ws.idx_a, nnz, end_bit,
                                     L->ws.hist, s);
    if (st != CSP_OK) return st;
    if (L->esz == 4)
        k_gather_canon<K, uint32_t><<<grid, 256, 0, s>>>(kb, L->ws.idx_b, nnz, L->in, (const uint32_t *)vals,
                                                         L->rows, L->cols, (uint32_t *)L->vals, flags);
    else
        k_gather_canon<K, uint16_t><<<grid, 256, 0, s>>>(kb, L->ws.idx_b, nnz, L->in, (const uint16_t *)vals,
                                                         L->rows, L->cols, (uint16_t *)L->vals, flags);
    CSP_LAUNCHED("k_gather_canon");
    return CSP_OK;
}

csp_status build_canonical(csp_layer *L, const int32_t *rows, const int32_t *cols, const void *vals,
                           uint32_t *flags, hipStream_t s)
{
    if (L->nnz == 0) return CSP_OK;
    if ((uint64_t)(L->out * L->in - 1) <= 0xFFFFFFFFull)
        return build_canonical_k<uint32_t>(L, rows, cols, vals, flags, s);
    return build_canonical_k<uint64_t>(L, rows, cols, vals, flags, s);
}

}  // namespace csp
