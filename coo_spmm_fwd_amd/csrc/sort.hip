// sort.hip -- integer building blocks: stable LSD radix sort of (key, index)
// pairs, device-wide exclusive scans, and segment offsets by binary search.
//
// These serve the canonical (row, col) ordering and the transposed (col, row)
// view of the COO layer ("Beyond Masked Sparsity: SNACK ...", Abstract: COO
// storage of the non-zero connections only) and the re-sort after a
// restructure.  All work is HBM-bound integer traffic; no host sync here.
#include "common.h"
#include "device_util.h"

namespace csp {
namespace {

constexpr int kSortThreads = 256;             // 4 waves
constexpr int kSortItemsPerLane = 16;
constexpr int kSortWaveItems = kWave * kSortItemsPerLane;          // 1024
constexpr int kSortTile = kSortThreads * kSortItemsPerLane;         // 4096
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanThreads * kScanItems;                // 4096
constexpr int kMaxScanPartials = kScanThreads * 64;

int64_t sort_tiles(int64_t n) { return ceil_div(n, kSortTile); }

// The scans read either the items themselves or the number of set bits of
// each item (kPopc: positions of the set bits of a bitmap in order).
template <bool kPopc>
__device__ __forceinline__ uint32_t scan_item(uint32_t v) { return kPopc ? (uint32_t)__popc(v) : v; }

template <bool kPopc>
__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const uint32_t *__restrict__ in, int64_t n,
                                                              uint32_t *__restrict__ partials)
{
    __shared__ uint32_t lds[17];
    int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        s += base + i < n ? scan_item<kPopc>(load_or_first(in, base + i, n)) : 0u;
    uint32_t total;
    block_exclusive_scan(s, lds, &total);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

// One block: exclusive scan of nb partials in place; total -> partials[nb].
__global__ __launch_bounds__(kScanThreads) void k_scan_partials(uint32_t *__restrict__ partials, int64_t nb)
{
    __shared__ uint32_t lds[17];
    int64_t per = ceil_div(nb, kScanThreads);
    int64_t b0 = (int64_t)threadIdx.x * per;
    uint32_t s = 0;
    for (int64_t i = b0; i < b0 + per && i < nb; ++i) s += partials[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan(s, lds, &total);
    for (int64_t i = b0; i < b0 + per && i < nb; ++i) {
        uint32_t v = partials[i];
        partials[i] = run;
        run += v;
    }
    if (threadIdx.x == 0) partials[nb] = total;
}

// out[i] = exclusive prefix of the items; with `total_at` set the last block
// also writes the grand total to out[n].
template <bool kPopc>
__global__ __launch_bounds__(kScanThreads) void k_scan_apply(const uint32_t *in, uint32_t *out, int64_t n,
                                                             const uint32_t *__restrict__ partials, bool total_at)
{
    __shared__ uint32_t lds[17];
    int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    uint32_t v[kScanItems], s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = base + i < n ? scan_item<kPopc>(load_or_first(in, base + i, n)) : 0u;
        s += v[i];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan(s, lds, &total) + partials[blockIdx.x];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        if (base + i < n) {
            out[base + i] = run;
            run += v[i];
        }
    if (total_at && blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = partials[gridDim.x];
}

// k_scan_partials and k_scan_apply in one launch for up to kFusedScanBlocks
// blocks: each block first adds up the reduce sums of the blocks before it.
// The last block writes the grand total to out[n] (total_at) and to *total.
constexpr int64_t kFusedScanBlocks = 1024;
template <bool kPopc>
__global__ __launch_bounds__(kScanThreads) void k_scan_apply_prefix(const uint32_t *in, uint32_t *out, int64_t n,
                                                                    const uint32_t *__restrict__ partials,
                                                                    bool total_at, uint32_t *total_out)
{
    __shared__ uint32_t lds[17];
    const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    uint32_t v[kScanItems], s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = base + i < n ? scan_item<kPopc>(load_or_first(in, base + i, n)) : 0u;
        s += v[i];
    }
    uint32_t before = 0, total;
    for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kScanThreads) before += partials[j];
    block_exclusive_scan(before, lds, &before);
    uint32_t run = block_exclusive_scan(s, lds, &total) + before;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        if (base + i < n) {
            out[base + i] = run;
            run += v[i];
        }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        if (total_at) out[n] = before + total;
        if (total_out) *total_out = before + total;
    }
}

__global__ void k_copy_total(const uint32_t *src, uint32_t *dst)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) *dst = *src;
}

// ---------------------------------------------------------------- radix sort
template <typename K>
__global__ __launch_bounds__(kSortThreads) void k_radix_hist(const K *__restrict__ keys, int64_t n, int shift,
                                                             uint32_t *__restrict__ hist, int64_t ntiles)
{
    __shared__ uint32_t h[256];
    const int t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    // One LDS atomic per distinct digit per wave (its lowest lane adds the
    // count), so runs of equal digits (presorted keys) do not serialize.
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    const int lane = t & 63;
#pragma unroll 4
    for (int j = 0; j < kSortItemsPerLane; ++j) {
        const int64_t idx = base + (int64_t)j * kSortThreads + t;
        const bool ok = idx < n;
        const uint32_t d = ok ? (uint32_t)(load_or_first(keys, idx, n) >> shift) & 255u : 0u;
        uint64_t m = __ballot(ok);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t bb = __ballot(on);
            m &= on ? bb : ~bb;
        }
        if (ok && (m & ((1ull << lane) - 1)) == 0) atomicAdd(&h[d], (uint32_t)__popcll(m));
    }
    __syncthreads();
    hist[(int64_t)t * ntiles + blockIdx.x] = h[t];
}

// Stable scatter of one digit pass.  Wave w of a tile owns items
// [w*1024, (w+1)*1024) of the tile, walked in 16 rounds of 64 consecutive
// items, so the processing order equals the item order.  Within a round the
// lanes sharing a digit are found with eight ballots (one per digit bit);
// their leader reserves space with one LDS atomic and broadcasts the base.
template <typename K>
__global__ __launch_bounds__(kSortThreads) void k_radix_scatter(const K *__restrict__ keys_in,
                                                                const int32_t *__restrict__ vals_in,
                                                                K *__restrict__ keys_out,
                                                                int32_t *__restrict__ vals_out, int64_t n,
                                                                int shift, const uint32_t *__restrict__ scanned,
                                                                int64_t ntiles)
{
    __shared__ uint32_t cnt[4][256];
    __shared__ uint32_t gbase[256];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt[i][t] = 0;
    gbase[t] = scanned[(int64_t)t * ntiles + blockIdx.x];
    __syncthreads();

    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t base = (int64_t)blockIdx.x * kSortTile + (int64_t)w * kSortWaveItems;
    K key[kSortItemsPerLane];
    int32_t val[kSortItemsPerLane];
    uint32_t rank[kSortItemsPerLane];
#pragma unroll
    for (int j = 0; j < kSortItemsPerLane; ++j) {
        int64_t idx = base + (int64_t)j * kWave + lane;
        bool valid = idx < n;
        K k = load_or_first(keys_in, idx, n);
        int32_t v = load_or_first(vals_in, idx, n);
        if (!valid) {
            k = K(0);
            v = 0;
        }
        uint32_t d = (uint32_t)(k >> shift) & 255u;
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            bool on = (d >> bit) & 1u;
            uint64_t bb = __ballot(on);
            m &= on ? bb : ~bb;
        }
        uint32_t r = (uint32_t)__popcll(m & lt);
        int leader = valid ? (__ffsll((unsigned long long)m) - 1) : lane;
        uint32_t before = 0;
        if (valid && r == 0) before = atomicAdd(&cnt[w][d], (uint32_t)__popcll(m));
        before = __shfl(before, leader, 64);
        key[j] = k;
        val[j] = v;
        rank[j] = before + r;
    }
    __syncthreads();
    {
        uint32_t run = gbase[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t c = cnt[i][t];
            cnt[i][t] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortItemsPerLane; ++j) {
        int64_t idx = base + (int64_t)j * kWave + lane;
        if (idx < n) {
            uint32_t d = (uint32_t)(key[j] >> shift) & 255u;
            uint32_t dst = cnt[w][d] + rank[j];
            keys_out[dst] = key[j];
            vals_out[dst] = val[j];
        }
    }
}

template <typename K>
__global__ void k_copy_pairs(const K *ki, const int32_t *vi, K *ko, int32_t *vo, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        ko[i] = ki[i];
        vo[i] = vi[i];
    }
}

template <typename K>
csp_status sort_impl(K *ka, int32_t *va, K *kb, int32_t *vb, int64_t n, int end_bit, uint32_t *hist,
                     int *result_in_b, hipStream_t s)
{
    *result_in_b = 0;
    if (n <= 1 || end_bit <= 0) return CSP_OK;
    const int passes = (end_bit + 7) / 8;
    const int64_t ntiles = sort_tiles(n);
    const int64_t nh = 256 * ntiles;
    uint32_t *partials = hist + nh;
    K *src_k = ka, *dst_k = kb;
    int32_t *src_v = va, *dst_v = vb;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        k_radix_hist<K><<<dim3((unsigned)ntiles), dim3(kSortThreads), 0, s>>>(src_k, n, shift, hist, ntiles);
        CSP_LAUNCHED("k_radix_hist");
        csp_status st = exclusive_scan_u32(hist, hist, nh, partials, nullptr, s);
        if (st != CSP_OK) return st;
        k_radix_scatter<K><<<dim3((unsigned)ntiles), dim3(kSortThreads), 0, s>>>(src_k, src_v, dst_k, dst_v, n,
                                                                                shift, hist, ntiles);
        CSP_LAUNCHED("k_radix_scatter");
        K *tk = src_k; src_k = dst_k; dst_k = tk;
        int32_t *tv = src_v; src_v = dst_v; dst_v = tv;
    }
    *result_in_b = (passes & 1);
    return CSP_OK;
}

__global__ void k_offsets(const int32_t *__restrict__ sorted, int64_t n, int32_t *__restrict__ ptr, int64_t nseg)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i > nseg) return;
    int64_t lo = 0, hi = n;  // first j with sorted[j] >= i
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if ((int64_t)sorted[mid] < i) lo = mid + 1; else hi = mid;
    }
    ptr[i] = (int32_t)lo;
}

__global__ void k_fill_u32(uint32_t *p, uint32_t v, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

size_t sort_hist_words(int64_t n)
{
    int64_t nh = 256 * sort_tiles(n > 0 ? n : 1);
    int64_t scan_n = nh > n ? nh : n;
    return (size_t)(nh + ceil_div(scan_n, kScanTile) + 64);
}

namespace {
// Block sums, then either (up to kFusedScanBlocks blocks) one launch that
// scans with each block's prefix summed in place, or a one-block scan of the
// sums and the apply launch.  The grand total goes to out[n] (total_at) and
// to *total (optional).
template <bool kPopc>
csp_status scan_impl(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *partials, bool total_at,
                     uint32_t *total, hipStream_t s)
{
    const int64_t nb = ceil_div(n, kScanTile);
    if (nb > kMaxScanPartials) return set_error(CSP_ERR_INVALID_ARG, "scan of %lld items exceeds the limit", (long long)n);
    k_scan_reduce<kPopc><<<dim3((unsigned)nb), dim3(kScanThreads), 0, s>>>(in, n, partials);
    CSP_LAUNCHED("k_scan_reduce");
    if (nb <= kFusedScanBlocks) {
        k_scan_apply_prefix<kPopc><<<dim3((unsigned)nb), dim3(kScanThreads), 0, s>>>(in, out, n, partials, total_at,
                                                                                      total);
        CSP_LAUNCHED("k_scan_apply_prefix");
        return CSP_OK;
    }
    k_scan_partials<<<1, kScanThreads, 0, s>>>(partials, nb);
    CSP_LAUNCHED("k_scan_partials");
    k_scan_apply<kPopc><<<dim3((unsigned)nb), dim3(kScanThreads), 0, s>>>(in, out, n, partials, total_at);
    CSP_LAUNCHED("k_scan_apply");
    if (total) {
        k_copy_total<<<1, 64, 0, s>>>(partials + nb, total);
        CSP_LAUNCHED("k_copy_total");
    }
    return CSP_OK;
}
}  // namespace

csp_status exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *partials, uint32_t *total,
                              hipStream_t s)
{
    if (n <= 0) {
        if (total) {
            k_fill_u32<<<1, 64, 0, s>>>(total, 0u, 1);
            CSP_LAUNCHED("k_fill_u32");
        }
        return CSP_OK;
    }
    return scan_impl<false>(in, out, n, partials, false, total, s);
}

csp_status exclusive_scan_popc(const uint32_t *words, uint32_t *pref, int64_t n, uint32_t *partials, hipStream_t s)
{
    if (n <= 0) return fill_u32(pref, 0u, 1, s);
    return scan_impl<true>(words, pref, n, partials, true, nullptr, s);
}

csp_status radix_sort_pairs(int key_bytes, const void *keys_in, const int32_t *vals_in, void *keys_out,
                            int32_t *vals_out, void *keys_tmp, int32_t *vals_tmp, int64_t n, int end_bit,
                            uint32_t *hist, hipStream_t s)
{
    // Sorting ping-pongs between `tmp` and `out`; the input is first copied
    // into whichever of the two makes the final pass land in `out`.
    if (n <= 0) return CSP_OK;
    const int passes = (n <= 1 || end_bit <= 0) ? 0 : (end_bit + 7) / 8;
    const bool start_in_out = (passes % 2) == 0;
    void *ka = start_in_out ? keys_out : keys_tmp;
    int32_t *va = start_in_out ? vals_out : vals_tmp;
    void *kb = start_in_out ? keys_tmp : keys_out;
    int32_t *vb = start_in_out ? vals_tmp : vals_out;
    const unsigned grid = (unsigned)ceil_div(n, 256);
    if (keys_in != ka || vals_in != va) {
        if (key_bytes == 8)
            k_copy_pairs<uint64_t><<<grid, 256, 0, s>>>((const uint64_t *)keys_in, vals_in, (uint64_t *)ka, va, n);
        else
            k_copy_pairs<uint32_t><<<grid, 256, 0, s>>>((const uint32_t *)keys_in, vals_in, (uint32_t *)ka, va, n);
        CSP_LAUNCHED("k_copy_pairs");
    }
    int in_b = 0;
    csp_status st = key_bytes == 8
                        ? sort_impl<uint64_t>((uint64_t *)ka, va, (uint64_t *)kb, vb, n, end_bit, hist, &in_b, s)
                        : sort_impl<uint32_t>((uint32_t *)ka, va, (uint32_t *)kb, vb, n, end_bit, hist, &in_b, s);
    return st;
}

csp_status segment_offsets(const int32_t *sorted, int64_t n, int32_t *ptr, int64_t nseg, hipStream_t s)
{
    k_offsets<<<dim3((unsigned)ceil_div(nseg + 1, 256)), 256, 0, s>>>(sorted, n, ptr, nseg);
    CSP_LAUNCHED("k_offsets");
    return CSP_OK;
}

csp_status fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s)
{
    if (n <= 0) return CSP_OK;
    k_fill_u32<<<dim3((unsigned)ceil_div(n, 256)), 256, 0, s>>>(p, v, n);
    CSP_LAUNCHED("k_fill_u32");
    return CSP_OK;
}

}  // namespace csp
