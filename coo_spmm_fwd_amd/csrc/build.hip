// build.hip -- the COO builder: canonical (row, col) order, row offsets, and
// the transposed (col, row) view used by the input-gradient pass.
//
// "Beyond Masked Sparsity: SNACK ..." (Abstract) stores only the non-zero
// connections, as COO.  Here the triples are put in row-major canonical order
// with a flat key row*in + col (one LSD radix sort), so each output row is a
// contiguous segment; a second stable sort by column of the canonical indices
// gives the column segments.  Offsets come from a binary search per segment.
#include "common.h"

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
__global__ void k_seg_pieces(const int32_t *__restrict__ ptr, int64_t nseg, uint32_t *__restrict__ pieces)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nseg) return;
    int64_t len = (int64_t)ptr[i + 1] - ptr[i];
    pieces[i] = len <= kTaskChunk ? 1u : (uint32_t)((len + kTaskChunk - 1) / kTaskChunk);
}

__global__ void k_emit_tasks(const int32_t *__restrict__ ptr, const int32_t *__restrict__ first, int64_t nseg,
                             int4 *__restrict__ desc, int64_t cap, int4 *__restrict__ split,
                             uint32_t *__restrict__ nsplit)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nseg) return;
    const int32_t f = first[i], p = first[i + 1] - f, b = ptr[i], e = ptr[i + 1];
    for (int32_t j = 0; j < p && (int64_t)f + j < cap; ++j) {
        const int32_t kb = b + j * kTaskChunk;
        const int32_t ke = kb + kTaskChunk < e ? kb + kTaskChunk : e;
        desc[f + j] = make_int4((int32_t)i, kb, ke, p > 1 ? f + j : -1);
    }
    if (p > 1) split[atomicAdd(nsplit, 1u)] = make_int4((int32_t)i, f, p, 0);
}

// seg_first[0..nseg) = exclusive scan of the per-segment task counts,
// seg_first[nseg] = the total; then one descriptor per task and one record
// per split segment (their order is irrelevant: each record is self-contained).
csp_status build_tasks(TaskList &T, const int32_t *ptr, int64_t nseg, uint32_t *partials, uint32_t *nsplit,
                       hipStream_t s)
{
    const unsigned grid = (unsigned)ceil_div(nseg, 256);
    uint32_t *first = (uint32_t *)T.seg_first;
    k_seg_pieces<<<grid, 256, 0, s>>>(ptr, nseg, first);
    CSP_LAUNCHED("k_seg_pieces");
    csp_status st = exclusive_scan_u32(first, first, nseg, partials, first + nseg, s);
    if (st != CSP_OK) return st;
    st = fill_u32(nsplit, 0u, 1, s);
    if (st != CSP_OK) return st;
    k_emit_tasks<<<grid, 256, 0, s>>>(ptr, T.seg_first, nseg, T.desc, T.cap, T.split, nsplit);
    CSP_LAUNCHED("k_emit_tasks");
    return CSP_OK;
}

}  // namespace

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

    // Task lists for the row-order and column-order passes (scan partials in
    // the now free radix histogram area); the task and split counts are read back.
    uint32_t *nsplit = L->ws.sel + 512;  // two words outside the select state
    st = build_tasks(L->row_tasks, L->row_ptr, L->out, L->ws.hist, nsplit, s);
    if (st != CSP_OK) return st;
    st = build_tasks(L->col_tasks, L->col_ptr, L->in, L->ws.hist, nsplit + 1, s);
    if (st != CSP_OK) return st;
    int32_t counts[4] = {0, 0, 0, 0};
    CSP_HIP(hipMemcpyAsync(&counts[0], L->row_tasks.seg_first + L->out, 4, hipMemcpyDeviceToHost, s));
    CSP_HIP(hipMemcpyAsync(&counts[1], L->col_tasks.seg_first + L->in, 4, hipMemcpyDeviceToHost, s));
    CSP_HIP(hipMemcpyAsync(&counts[2], nsplit, 8, hipMemcpyDeviceToHost, s));
    CSP_HIP(hipStreamSynchronize(s));
    L->row_tasks.count = counts[0];
    L->col_tasks.count = counts[1];
    L->row_tasks.nsplit = counts[2];
    L->col_tasks.nsplit = counts[3];
    if (L->row_tasks.count > L->row_tasks.cap || L->col_tasks.count > L->col_tasks.cap)
        return set_error(CSP_ERR_HIP, "task list overflow (%lld/%lld, %lld/%lld)", (long long)L->row_tasks.count,
                         (long long)L->row_tasks.cap, (long long)L->col_tasks.count, (long long)L->col_tasks.cap);
    return CSP_OK;
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
