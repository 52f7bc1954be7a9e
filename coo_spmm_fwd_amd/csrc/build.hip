// build.hip -- the COO builder: canonical (row, col) order, row offsets, and
// the transposed (col, row) view used by the input-gradient pass.
//
// "Beyond Masked Sparsity: SNACK ..." (Abstract) stores only the non-zero
// connections, as COO.  Here the triples are put in row-major canonical order
// with a flat key row*in + col (one LSD radix sort), so each output row is a
// contiguous segment; a second stable sort by column of the canonical indices
// gives the column segments.  Offsets come from a binary search per segment.
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

// Both task lists (rows, then columns) are built by the same three launches:
// blocks [0, tiles0) work on list 0 and the rest on list 1, one segment per thread.
constexpr int kTaskThreads = 1024;

struct TaskBuild {
    const int32_t *ptr[2];
    int64_t nseg[2];
    int64_t tiles[2];
    int4 *desc[2];
    int4 *split[2];
    int32_t *seg_first[2];
    int64_t cap[2];
    uint32_t *partials[2];  // tiles + 1 words each
    uint32_t *counts;       // [0], [1] tasks; [2], [3] split segments
};

__device__ __forceinline__ void task_tile(const TaskBuild &tb, int &l, int64_t &tile)
{
    l = (int64_t)blockIdx.x < tb.tiles[0] ? 0 : 1;
    tile = l ? (int64_t)blockIdx.x - tb.tiles[0] : (int64_t)blockIdx.x;
}

__global__ __launch_bounds__(kTaskThreads) void k_tasks_count(TaskBuild tb)
{
    __shared__ uint32_t lds[17];
    int l;
    int64_t tile;
    task_tile(tb, l, tile);
    const int64_t i = tile * kTaskThreads + threadIdx.x;
    uint32_t total;
    block_exclusive_scan(i < tb.nseg[l] ? seg_pieces(tb.ptr[l], i) : 0u, lds, &total);
    if (threadIdx.x == 0) tb.partials[l][tile] = total;
    if (blockIdx.x == 0 && threadIdx.x < 2) tb.counts[2 + threadIdx.x] = 0;
}

// Two blocks: block l scans the tile sums of list l in place and stores the
// list's task count (also as seg_first[nseg]).
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
        tb.counts[l] = total;
        tb.seg_first[l][tb.nseg[l]] = (int32_t)total;
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
    const int64_t i = tile * kTaskThreads + threadIdx.x;
    const bool live = i < tb.nseg[l];
    const uint32_t p = live ? seg_pieces(tb.ptr[l], i) : 0u;
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
        tb.counts[l] = before + total;
        tb.seg_first[l][tb.nseg[l]] = (int32_t)(before + total);
    }
    if (!live) return;
    tb.seg_first[l][i] = f;
    const int32_t b = tb.ptr[l][i], e = tb.ptr[l][i + 1];
    for (int32_t j = 0; j < (int32_t)p && (int64_t)f + j < tb.cap[l]; ++j) {
        const int32_t kb = b + j * kTaskChunk;
        const int32_t ke = kb + kTaskChunk < e ? kb + kTaskChunk : e;
        tb.desc[l][f + j] = make_int4((int32_t)i, kb, ke, p > 1 ? f + j : -1);
    }
    if (p > 1) tb.split[l][atomicAdd(&tb.counts[2 + l], 1u)] = make_int4((int32_t)i, f, (int32_t)p, 0);
}

}  // namespace

// seg_first[0..nseg) = exclusive scan of the per-segment task counts,
// seg_first[nseg] = the total; then one descriptor per task and one record
// per split segment (their order is irrelevant: each record is self-contained).
csp_status build_task_lists(csp_layer *L, hipStream_t s)
{
    TaskBuild tb;
    TaskList *T[2] = {&L->row_tasks, &L->col_tasks};
    const int32_t *ptr[2] = {L->row_ptr, L->col_ptr};
    const int64_t nseg[2] = {L->out, L->in};
    uint32_t *part = L->ws.hist;
    for (int l = 0; l < 2; ++l) {
        tb.ptr[l] = ptr[l];
        tb.nseg[l] = nseg[l];
        tb.tiles[l] = ceil_div(nseg[l], kTaskThreads);
        tb.desc[l] = T[l]->desc;
        tb.split[l] = T[l]->split;
        tb.seg_first[l] = T[l]->seg_first;
        tb.cap[l] = T[l]->cap;
        tb.partials[l] = part;
        part += tb.tiles[l] + 1;
    }
    tb.counts = L->ws.sel + kSelCounts;
    const unsigned grid = (unsigned)(tb.tiles[0] + tb.tiles[1]);
    k_tasks_count<<<grid, kTaskThreads, 0, s>>>(tb);
    CSP_LAUNCHED("k_tasks_count");
    if (tb.tiles[0] <= kPrefixTaskTiles && tb.tiles[1] <= kPrefixTaskTiles) {
        k_tasks_emit<true><<<grid, kTaskThreads, 0, s>>>(tb);
    } else {
        k_tasks_scan<<<2, kTaskThreads, 0, s>>>(tb);
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
    if (L->row_tasks.count > L->row_tasks.cap || L->col_tasks.count > L->col_tasks.cap)
        return set_error(CSP_ERR_HIP, "task list overflow (%lld/%lld, %lld/%lld)", (long long)L->row_tasks.count,
                         (long long)L->row_tasks.cap, (long long)L->col_tasks.count, (long long)L->col_tasks.cap);
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

    st = build_task_lists(L, s);
    if (st != CSP_OK) return st;
    uint32_t counts[4] = {0, 0, 0, 0};
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
