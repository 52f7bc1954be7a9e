// restructure.hip -- prune-and-regrow for dynamic sparse training on the COO
// layer ("Beyond Masked Sparsity: SNACK ...", Abstract: an API to restructure
// the connections of a truly sparse layer during dynamic sparse training).
//
// Rule implemented (nnz stays constant):
//  1. prune the n_prune entries that come first in the order
//     (bit pattern of |v|, canonical index): found with a radix select on the
//     magnitude bits (threshold T and how many entries equal to T go), then a
//     stable compaction of the kept entries, which stay in canonical order;
//  2. regrow n_prune positions from a counter-based stream: candidate i is
//     word (i mod 4) of the Philox4x64-10 block (counter (i div 4, step, 0, 0),
//     key (seed, 0)) mapped to floor(u * out*in / 2^64).  Walking i upwards, a
//     candidate is taken when its position is empty after the prune and not
//     taken before.  In parallel: a batch of candidates is generated, occupied
//     ones are dropped (binary search in the kept row segment), the rest are
//     sorted by position (stable, so a repeated position keeps its first i),
//     and the n_prune smallest i among the first occurrences are taken; if a
//     batch falls short, the next batch continues the stream;
//  3. kept and new entries are merged back into canonical order (each side
//     finds its place by binary search in the other), and the offsets and the
//     transposed view are rebuilt.
// Every step is integer work or a bit-exact move of values.
#include <cstdlib>

#include "common.h"
#include "device_util.h"
#include "regrow.h"

namespace csp {
namespace {

constexpr int kSelState = 0;     // sel[0] prefix, sel[1] mask, sel[2] still to select
constexpr int kSelTotal = 8;     // sel[8] count read back by the host
constexpr int kSelHist = 16;     // sel[16..272) digit histogram
constexpr int kSelWords = 1024;

__global__ void k_sel_init(uint32_t *sel, uint32_t n_prune)
{
    const int t = threadIdx.x;
    for (int i = t; i < kSelWords; i += blockDim.x) sel[i] = 0;
    __syncthreads();
    if (t == 0) sel[kSelState + 2] = n_prune;
}

// Digit histogram of the entries whose higher magnitude bits match the
// prefix found so far.  The top digits of |v| cluster in a few bins, so each
// wave adds one count per distinct digit (its lowest lane does the LDS atomic).
template <typename V>
__global__ __launch_bounds__(256) void k_sel_hist(const V *__restrict__ vals, int64_t n, int shift,
                                                  uint32_t *__restrict__ sel)
{
    __shared__ uint32_t h[256];
    const int t = threadIdx.x, lane = t & 63;
    h[t] = 0;
    __syncthreads();
    const uint32_t prefix = sel[kSelState], mask = sel[kSelState + 1];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + (t - lane); base < n; base += stride) {
        const int64_t k = base + lane;
        const uint32_t key = k < n ? mag_key<V>(vals[k]) : 0u;
        const bool take = k < n && (key & mask) == prefix;
        const uint32_t d = (key >> shift) & 255u;
        const uint64_t m = lanes_with_same_byte(d, take);
        if (take && (m & lanes_below()) == 0) atomicAdd(&h[d], (uint32_t)__popcll(m));
    }
    __syncthreads();
    if (h[t]) atomicAdd(&sel[kSelHist + t], h[t]);
}

// One block of 256: find the digit that holds the still-needed rank, extend the prefix, clear the histogram.
__global__ __launch_bounds__(256) void k_sel_pick(uint32_t *sel, int shift)
{
    __shared__ uint32_t wsum[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const uint32_t h = sel[kSelHist + t];
    uint32_t x = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t before = x - h;
    for (int i = 0; i < w; ++i) before += wsum[i];
    const uint32_t need = sel[kSelState + 2];
    __syncthreads();
    if (before < need && need <= before + h) {
        sel[kSelState] |= (uint32_t)t << shift;
        sel[kSelState + 1] |= 255u << shift;
        sel[kSelState + 2] = need - before;
    }
    sel[kSelHist + t] = 0;
}

template <typename V>
__global__ void k_eq_flags(const V *__restrict__ vals, int64_t n, const uint32_t *__restrict__ sel,
                           uint32_t *__restrict__ eq)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) eq[k] = mag_key<V>(vals[k]) == sel[kSelState] ? 1u : 0u;
}

template <typename V>
__device__ inline bool is_pruned(V v, uint32_t eqrank, uint32_t T, uint32_t rem)
{
    uint32_t key = mag_key<V>(v);
    return key < T || (key == T && eqrank < rem);
}

template <typename V>
__global__ void k_keep_flags(const V *__restrict__ vals, int64_t n, const uint32_t *__restrict__ sel,
                             const uint32_t *__restrict__ eqrank, uint32_t *__restrict__ keep)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) keep[k] = is_pruned<V>(vals[k], eqrank[k], sel[kSelState], sel[kSelState + 2]) ? 0u : 1u;
}

template <typename V>
__global__ void k_compact_kept(const int32_t *__restrict__ rows, const int32_t *__restrict__ cols,
                               const V *__restrict__ vals, int64_t n, const uint32_t *__restrict__ sel,
                               const uint32_t *__restrict__ eqrank, const uint32_t *__restrict__ kpos,
                               int32_t *__restrict__ rows_k, int32_t *__restrict__ cols_k, V *__restrict__ vals_k)
{
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    V v = vals[k];
    if (is_pruned<V>(v, eqrank[k], sel[kSelState], sel[kSelState + 2])) return;
    uint32_t p = kpos[k];
    rows_k[p] = rows[k];
    cols_k[p] = cols[k];
    vals_k[p] = v;
}

__device__ inline bool contains_i32(const int32_t *a, int64_t n, int32_t x)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo < n && a[lo] == x;
}

__device__ inline int64_t lower_bound_u64(const uint64_t *a, int64_t n, uint64_t x)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ inline int64_t lower_bound_i32(const int32_t *a, int64_t n, int32_t x)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

template <typename K>
__global__ void k_regrow_candidates(uint64_t seed, uint64_t step, uint64_t i0, int64_t M, int64_t in,
                                    uint64_t npos, const int32_t *__restrict__ cols_k,
                                    const int32_t *__restrict__ rp_k, const uint64_t *__restrict__ acc, int64_t nacc,
                                    K *__restrict__ keys, int32_t *__restrict__ idx)
{
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= M) return;
    const uint64_t p = regrow_position(seed, step, i0 + (uint64_t)j, npos);
    const int64_t r = (int64_t)(p / (uint64_t)in);
    const int32_t c = (int32_t)(p - (uint64_t)r * (uint64_t)in);
    const int32_t a = rp_k[r], b = rp_k[r + 1];
    bool occ = contains_i32(cols_k + a, b - a, c);
    if (!occ && nacc > 0) {
        int64_t q = lower_bound_u64(acc, nacc, p);
        occ = q < nacc && acc[q] == p;
    }
    keys[j] = occ ? (K)npos : (K)p;
    idx[j] = (int32_t)j;
}

template <typename K>
__device__ inline bool first_free(const K *keys, int64_t t, K sentinel)
{
    K p = keys[t];
    return p != sentinel && (t == 0 || keys[t - 1] != p);
}

template <typename K>
__global__ void k_first_by_i(const K *__restrict__ keys, const int32_t *__restrict__ idx, int64_t M, K sentinel,
                             uint32_t *__restrict__ flag_by_i)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < M) flag_by_i[idx[t]] = first_free<K>(keys, t, sentinel) ? 1u : 0u;
}

template <typename K>
__global__ void k_take_flags(const K *__restrict__ keys, const int32_t *__restrict__ idx, int64_t M, K sentinel,
                             const uint32_t *__restrict__ rank_by_i, uint32_t need, uint32_t *__restrict__ take)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < M) take[t] = (first_free<K>(keys, t, sentinel) && rank_by_i[idx[t]] < need) ? 1u : 0u;
}

template <typename K>
__global__ void k_compact_taken(const K *__restrict__ keys, const int32_t *__restrict__ idx, int64_t M, K sentinel,
                                const uint32_t *__restrict__ rank_by_i, uint32_t need,
                                const uint32_t *__restrict__ tpos, uint64_t *__restrict__ out)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < M && first_free<K>(keys, t, sentinel) && rank_by_i[idx[t]] < need) out[tpos[t]] = (uint64_t)keys[t];
}

// Union of two disjoint sorted position lists.
__global__ void k_merge_positions(const uint64_t *__restrict__ a, int64_t na, const uint64_t *__restrict__ b,
                                  int64_t nb, uint64_t *__restrict__ dst)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < na) dst[t + lower_bound_u64(b, nb, a[t])] = a[t];
    else if (t < na + nb) {
        int64_t y = t - na;
        dst[y + lower_bound_u64(a, na, b[y])] = b[y];
    }
}

__global__ void k_copy_u64(const uint64_t *__restrict__ a, uint64_t *__restrict__ b, int64_t n)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) b[t] = a[t];
}

// First new position of each row: new_rp[r] = first index with newp >= r*in.
__global__ void k_new_row_offsets(const uint64_t *__restrict__ newp, int64_t nnew, int64_t out, int64_t in,
                                  int32_t *__restrict__ new_rp)
{
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r <= out) new_rp[r] = (int32_t)lower_bound_u64(newp, nnew, (uint64_t)r * (uint64_t)in);
}

// Kept entry x of row r lands after x kept entries and after the new entries
// of earlier rows and of row r with a smaller column.
template <typename V>
__global__ void k_merge_kept(const int32_t *__restrict__ rows_k, const int32_t *__restrict__ cols_k,
                             const V *__restrict__ vals_k, int64_t nkept, int64_t in,
                             const uint64_t *__restrict__ newp, const int32_t *__restrict__ new_rp,
                             int32_t *__restrict__ rows, int32_t *__restrict__ cols, V *__restrict__ vals)
{
    int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= nkept) return;
    const int32_t r = rows_k[x], c = cols_k[x];
    const int32_t a = new_rp[r], b = new_rp[r + 1];
    const uint64_t key = (uint64_t)r * (uint64_t)in + (uint64_t)c;
    const int64_t pos = x + a + lower_bound_u64(newp + a, b - a, key);
    rows[pos] = r;
    cols[pos] = c;
    vals[pos] = vals_k[x];
}

template <typename V>
__global__ void k_merge_new(const uint64_t *__restrict__ newp, int64_t nnew, int64_t in,
                            const int32_t *__restrict__ cols_k, const int32_t *__restrict__ rp_k, V regrow,
                            int32_t *__restrict__ rows, int32_t *__restrict__ cols, V *__restrict__ vals)
{
    int64_t y = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (y >= nnew) return;
    const uint64_t p = newp[y];
    const int64_t r = (int64_t)(p / (uint64_t)in);
    const int32_t c = (int32_t)(p - (uint64_t)r * (uint64_t)in);
    const int32_t a = rp_k[r], b = rp_k[r + 1];
    const int64_t pos = y + a + lower_bound_i32(cols_k + a, b - a, c);
    rows[pos] = (int32_t)r;
    cols[pos] = c;
    vals[pos] = regrow;
}

inline unsigned grid_for(int64_t n) { return (unsigned)ceil_div(n, 256); }

template <typename V>
csp_status prune(csp_layer *L, int64_t n_prune, hipStream_t s)
{
    Workspace &W = L->ws;
    const int64_t n = L->nnz;
    const V *vals = (const V *)L->vals;
    k_sel_init<<<1, 256, 0, s>>>(W.sel, (uint32_t)n_prune);
    CSP_LAUNCHED("k_sel_init");
    const int top = sizeof(V) == 4 ? 24 : 8;
    const unsigned hist_grid = (unsigned)(ceil_div(n, 256) < 2048 ? ceil_div(n, 256) : 2048);
    for (int shift = top; shift >= 0; shift -= 8) {
        k_sel_hist<V><<<hist_grid, 256, 0, s>>>(vals, n, shift, W.sel);
        CSP_LAUNCHED("k_sel_hist");
        k_sel_pick<<<1, 256, 0, s>>>(W.sel, shift);
        CSP_LAUNCHED("k_sel_pick");
    }
    k_eq_flags<V><<<grid_for(n), 256, 0, s>>>(vals, n, W.sel, W.u_a);
    CSP_LAUNCHED("k_eq_flags");
    csp_status st = exclusive_scan_u32(W.u_a, W.u_a, n, W.hist, nullptr, s);
    if (st != CSP_OK) return st;
    k_keep_flags<V><<<grid_for(n), 256, 0, s>>>(vals, n, W.sel, W.u_a, W.u_b);
    CSP_LAUNCHED("k_keep_flags");
    st = exclusive_scan_u32(W.u_b, W.u_b, n, W.hist, nullptr, s);
    if (st != CSP_OK) return st;
    k_compact_kept<V><<<grid_for(n), 256, 0, s>>>(L->rows, L->cols, vals, n, W.sel, W.u_a, W.u_b, W.rows_k,
                                                  W.cols_k, (V *)W.vals_k);
    CSP_LAUNCHED("k_compact_kept");
    return CSP_OK;
}

template <typename K>
csp_status regrow(csp_layer *L, int64_t n_prune, int64_t nkept, uint64_t seed, uint64_t step, hipStream_t s)
{
    Workspace &W = L->ws;
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    const K sentinel = (K)npos;
    const int end_bit = bits_for(npos);
    int64_t nacc = 0;  // accepted positions so far, sorted, in W.acc_a
    uint64_t i0 = 0;
    int64_t cap = regrow_batch_cap(L);
    if (const char *e = std::getenv("COOSPMM_REGROW_BATCH")) {  // test hook: smaller batches
        long long v = std::atoll(e);
        if (v >= 1 && v < cap) cap = v;
    }
    K *ka = (K *)W.key_a, *kb = (K *)W.key_b;
    int64_t batches = 0;
    while (nacc < n_prune) {
        if (++batches > 4096)
            return set_error(CSP_ERR_INVALID_ARG, "regrow found only %lld of %lld empty positions in %llu draws",
                             (long long)nacc, (long long)n_prune, (unsigned long long)i0);
        const int64_t need = n_prune - nacc;
        const double free_frac = (double)(npos - (uint64_t)nkept - (uint64_t)nacc) / (double)npos;
        double want = (double)need / free_frac * 1.1 + 1024.0;
        int64_t M = want > (double)cap ? cap : (int64_t)want;
        if (M < 1) M = 1;
        k_regrow_candidates<K><<<grid_for(M), 256, 0, s>>>(seed, step, i0, M, L->in, npos, W.cols_k,
                                                           W.rp_k, W.acc_a, nacc, ka, W.idx_a);
        CSP_LAUNCHED("k_regrow_candidates");
        // sorted result in (kb, idx_b); (ka, idx_a) double as scratch
        csp_status st = radix_sort_pairs((int)sizeof(K), ka, W.idx_a, kb, W.idx_b, ka, W.idx_a, M, end_bit, W.hist, s);
        if (st != CSP_OK) return st;
        k_first_by_i<K><<<grid_for(M), 256, 0, s>>>(kb, W.idx_b, M, sentinel, W.u_a);
        CSP_LAUNCHED("k_first_by_i");
        st = exclusive_scan_u32(W.u_a, W.u_b, M, W.hist, W.sel + kSelTotal, s);
        if (st != CSP_OK) return st;
        uint32_t firsts = 0;
        CSP_HIP(hipMemcpyAsync(&firsts, W.sel + kSelTotal, sizeof firsts, hipMemcpyDeviceToHost, s));
        CSP_HIP(hipStreamSynchronize(s));
        const int64_t taken = (int64_t)firsts < need ? (int64_t)firsts : need;
        if (taken > 0) {
            k_take_flags<K><<<grid_for(M), 256, 0, s>>>(kb, W.idx_b, M, sentinel, W.u_b, (uint32_t)need, W.u_a);
            CSP_LAUNCHED("k_take_flags");
            st = exclusive_scan_u32(W.u_a, W.u_a, M, W.hist, nullptr, s);
            if (st != CSP_OK) return st;
            uint64_t *dst = nacc == 0 ? W.acc_a : W.acc_b;
            k_compact_taken<K><<<grid_for(M), 256, 0, s>>>(kb, W.idx_b, M, sentinel, W.u_b, (uint32_t)need, W.u_a, dst);
            CSP_LAUNCHED("k_compact_taken");
            if (nacc > 0) {
                uint64_t *merged = (uint64_t *)W.key_a;  // free until the next batch
                k_merge_positions<<<grid_for(nacc + taken), 256, 0, s>>>(W.acc_a, nacc, W.acc_b, taken, merged);
                CSP_LAUNCHED("k_merge_positions");
                k_copy_u64<<<grid_for(nacc + taken), 256, 0, s>>>(merged, W.acc_a, nacc + taken);
                CSP_LAUNCHED("k_copy_u64");
            }
            nacc += taken;
        }
        i0 += (uint64_t)M;
    }
    return CSP_OK;
}

template <typename V>
csp_status restructure_v(csp_layer *L, int64_t n_prune, uint64_t seed, uint64_t step, V regrow_word, hipStream_t s)
{
    Workspace &W = L->ws;
    const int64_t nkept = L->nnz - n_prune;
    csp_status st = prune<V>(L, n_prune, s);
    if (st != CSP_OK) return st;
    st = segment_offsets(W.rows_k, nkept, W.rp_k, L->out, s);
    if (st != CSP_OK) return st;
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    st = npos <= 0xFFFFFFFFull ? regrow<uint32_t>(L, n_prune, nkept, seed, step, s)
                               : regrow<uint64_t>(L, n_prune, nkept, seed, step, s);
    if (st != CSP_OK) return st;
    if (nkept > 0) {
        k_new_row_offsets<<<grid_for(L->out + 1), 256, 0, s>>>(W.acc_a, n_prune, L->out, L->in, W.rp_new);
        CSP_LAUNCHED("k_new_row_offsets");
        k_merge_kept<V><<<grid_for(nkept), 256, 0, s>>>(W.rows_k, W.cols_k, (const V *)W.vals_k, nkept, L->in,
                                                        W.acc_a, W.rp_new, L->rows, L->cols, (V *)L->vals);
        CSP_LAUNCHED("k_merge_kept");
    }
    k_merge_new<V><<<grid_for(n_prune), 256, 0, s>>>(W.acc_a, n_prune, L->in, W.cols_k, W.rp_k, regrow_word,
                                                     L->rows, L->cols, (V *)L->vals);
    CSP_LAUNCHED("k_merge_new");
    return build_index(L, s);
}

}  // namespace

int64_t regrow_batch_cap(const csp_layer *L)
{
    // Candidate buffers hold max(nnz, 65536) keys; a batch never exceeds them.
    return L->ws.nkey_cap;
}

csp_status run_restructure(csp_layer *L, int64_t n_prune, uint64_t seed, uint64_t step, uint32_t regrow_bits,
                           hipStream_t s)
{
    if (n_prune == 0) return CSP_OK;
    if (L->ws.bitmap) return restructure_bitmap(L, n_prune, seed, step, regrow_bits, s);
    if (L->esz == 2) return restructure_v<uint16_t>(L, n_prune, seed, step, (uint16_t)regrow_bits, s);
    return restructure_v<uint32_t>(L, n_prune, seed, step, regrow_bits, s);
}

}  // namespace csp
