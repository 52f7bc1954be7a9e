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

}  // namespace

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
    }
    return segment_offsets((const int32_t *)L->ws.key_a, nnz, L->col_ptr, L->in, s);
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
