// occupancy.hip -- prune-and-regrow through position bitmaps ("Beyond Masked
// Sparsity: SNACK ...", Abstract: connections of the truly sparse layer are
// restructured during dynamic sparse training while only the stored entries
// are kept).
//
// The layer keeps one bit per weight position, row-major with rows padded to
// a multiple of 8 words, plus the exclusive rank of every word (set bits
// before it), as long as that costs at most 1 GiB and out*in < 2^32.  The
// rule is the one of the sorted path (prune order and regrow stream in
// regrow.h); what changes is how it is evaluated:
//  1. prune threshold: a radix select over the magnitude keys, 8 bits per
//     pass; each pass's blocks redo the digit choice of the earlier passes
//     from their histograms (eight spread copies, so the hot bins of the top
//     digit do not serialize the global atomics);
//  2. prune: per 4096-entry tile, counts of keys below / equal to the
//     threshold, one block scans them, then every entry knows whether it goes
//     (a bit per canonical index); the next bitmap is the current one without
//     those bits (one thread per word: its bits are consecutive entries);
//  3. regrow: a batch of the stream's candidates is tested against the next
//     bitmap; a hash table keyed by position keeps the smallest candidate
//     index per position, so "first occurrence and empty" is a flag per
//     candidate; a scan over the flags in stream order ranks them and the
//     first n_prune (minus those taken by earlier batches) set their bit;
//  4. rebuild: a scan of the next bitmap's bit counts gives every position
//     its canonical index; one thread per word writes its entries in order,
//     a kept one with the value at its old index (old bitmap and ranks), a
//     new one with the regrow value.  The transposed view comes from tiles
//     of 256 x 256 positions, one wave each: a ballot per column over the
//     tile's rows gives that column's entries in row order, so with the
//     scanned per-tile column counts every entry knows its transposed rank;
//     the task lists follow.
// Every pass reads or writes whole arrays in order; the only scattered
// traffic is the candidates' bitmap and hash probes.  The host reads back
// once at the end (taken count and task counts); only if the first batch fell
// short does it run further batches and rebuild again.
#include <cstdlib>
#include <cstring>
#include <utility>

#include "common.h"
#include "device_util.h"
#include "regrow.h"

namespace csp {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 4096;            // entries per block in the ranked passes
constexpr int kWaveItems = kTile / 4;  // 1024 consecutive entries per wave, 16 rounds of 64
constexpr int kCopies = 8;             // spread copies of each select histogram
constexpr int kHistWords = 256 * kCopies;
constexpr int kMaxPasses = 4;
constexpr int kSelT = kMaxPasses * kHistWords;  // threshold key
constexpr int kSelNeedEq = kSelT + 1;           // entries equal to the threshold that go
constexpr uint32_t kNoPos = 0xFFFFFFFFu;
constexpr uint64_t kEmptySlot = ~0ull;
constexpr int64_t kBatchLimit = int64_t(1) << 21;  // candidates per regrow batch
constexpr size_t kBitmapBytesLimit = size_t(1) << 30;

static_assert(kSelNeedEq < kSelCounts, "select state overlaps the counts");

// ------------------------------------------------------------ prune threshold
// One full wave: the digit whose bin holds the need-th entry (1-based) of the
// histogram h (kCopies copies of 256 bins), and how many entries precede it.
__device__ inline void pick_digit(const uint32_t *h, uint32_t need, uint32_t &digit, uint32_t &before)
{
    const int lane = threadIdx.x & 63;
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
        const uint4 v = *(const uint4 *)(h + k * 256 + lane * 4);
        c0 += v.x;
        c1 += v.y;
        c2 += v.z;
        c3 += v.w;
    }
    const uint32_t own = c0 + c1 + c2 + c3;
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    const uint64_t hit = __ballot(incl >= need);
    const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 63;
    uint32_t run = __shfl(incl - own, L, 64);
    const uint32_t b0 = __shfl(c0, L, 64), b1 = __shfl(c1, L, 64), b2 = __shfl(c2, L, 64);
    uint32_t d = 4 * L + 3;
    if (run + b0 >= need) {
        d = 4 * L;
    } else {
        run += b0;
        if (run + b1 >= need) {
            d = 4 * L + 1;
        } else {
            run += b1;
            if (run + b2 >= need) d = 4 * L + 2;
            else run += b2;
        }
    }
    digit = d;
    before = run;
}

// One full wave: prefix and mask of the digits fixed by passes [0, npass).
__device__ inline void select_state(const uint32_t *sel, int npass, int top, uint32_t n_prune, uint32_t &prefix,
                                    uint32_t &mask, uint32_t &need)
{
    prefix = 0;
    mask = 0;
    need = n_prune;
    for (int p = 0; p < npass; ++p) {
        uint32_t d, before;
        pick_digit(sel + p * kHistWords, need, d, before);
        const int shift = top - 8 * p;
        prefix |= d << shift;
        mask |= 255u << shift;
        need -= before;
    }
}

// Key sources of the radix select: the prune order reads the magnitude keys
// of the values (smallest first); the gradient-informed regrow reads score
// keys and wants the largest first, so it selects on their complement.
template <typename V>
struct MagKeys {
    const V *v;
    __device__ __forceinline__ uint32_t operator()(int64_t k, int64_t n) const
    {
        return mag_key<V>(load_or_first(v, k, n));
    }
};
struct InvKeys {
    const uint32_t *w;
    __device__ __forceinline__ uint32_t operator()(int64_t k, int64_t n) const { return ~load_or_first(w, k, n); }
};

// Histogram pass `pass` of the radix select; pass 0 also fills `clear`
// (the regrow hash table) with empty slots.  Few fat blocks: every block adds
// its nonzero bins to the global histogram with one atomic each.  Lanes that
// hit the same bin serialize on the LDS atomic (four copies, by lane, cut
// that by four), which costs less than matching digits across the wave.
constexpr int kHistThreads = 1024;

template <class K>
__global__ __launch_bounds__(kHistThreads) void k_bm_hist(K keyof, int64_t n, int pass, int top,
                                                          uint32_t n_prune, uint32_t *sel,
                                                          uint64_t *__restrict__ clear, int64_t nclear)
{
    __shared__ uint32_t h[4][256];  // lane & 3 picks the copy: a quarter of the lanes per address
    __shared__ uint32_t state[2];
    const int t = threadIdx.x;
    h[t >> 8][t & 255] = 0;
    if (t < 64) {
        uint32_t prefix, mask, need;
        select_state(sel, pass, top, n_prune, prefix, mask, need);
        if (t == 0) {
            state[0] = prefix;
            state[1] = mask;
        }
    }
    const int64_t stride = (int64_t)gridDim.x * kHistThreads;
    for (int64_t i = (int64_t)blockIdx.x * kHistThreads + t; i < nclear; i += stride) clear[i] = kEmptySlot;
    __syncthreads();
    const uint32_t prefix = state[0], mask = state[1];
    const int shift = top - 8 * pass;
    constexpr int U = 8;
    for (int64_t base = (int64_t)blockIdx.x * (kHistThreads * U); base < n; base += stride * U) {
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + u * kHistThreads + t;
            key[u] = keyof(k, n);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * kHistThreads + t < n && (key[u] & mask) == prefix)
                atomicAdd(&h[t & 3][(key[u] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t < 256) {
        const uint32_t c = h[0][t] + h[1][t] + h[2][t] + h[3][t];
        if (c) atomicAdd(&sel[pass * kHistWords + (blockIdx.x & (kCopies - 1)) * 256 + t], c);
    }
}

__global__ __launch_bounds__(64) void k_bm_sel_final(uint32_t *sel, uint32_t n_prune, int passes, int top)
{
    uint32_t prefix, mask, need;
    select_state(sel, passes, top, n_prune, prefix, mask, need);
    if (threadIdx.x == 0) {
        sel[kSelT] = prefix;
        sel[kSelNeedEq] = need;
    }
}

// ---------------------------------------------------------------------- prune
// Per tile: entries with key below the threshold, and equal to it.
template <class K>
__global__ __launch_bounds__(kThreads) void k_bm_prune_count(K keyof, int64_t n,
                                                             const uint32_t *__restrict__ sel,
                                                             uint32_t *__restrict__ tiles)
{
    __shared__ uint32_t part[2][4];
    const uint32_t T = sel[kSelT];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int64_t base = (int64_t)blockIdx.x * kTile;
    uint32_t lt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < kTile / kThreads; ++u) {
        const int64_t k = base + u * kThreads + t;
        const uint32_t key = keyof(k, n);
        lt += k < n && key < T;
        eq += k < n && key == T;
    }
    lt = wave_sum(lt);
    eq = wave_sum(eq);
    if (lane == 0) {
        part[0][w] = lt;
        part[1][w] = eq;
    }
    __syncthreads();
    if (t == 0) {
        tiles[2 * blockIdx.x] = part[0][0] + part[0][1] + part[0][2] + part[0][3];
        tiles[2 * blockIdx.x + 1] = part[1][0] + part[1][1] + part[1][2] + part[1][3];
    }
}

// One block of 1024: exclusive scans (in place) of the interleaved per-tile
// counts; clears the regrow counters and the select histograms.  The pairs
// are read and written coalesced: in each round wave w takes kScanRows rows
// of 64 consecutive pairs (lane l holds pair 64 g + l of its run), scans them
// row by row across the lanes with a running carry, and the waves' totals are
// added in order through LDS.  (A thread reading its own run of consecutive
// pairs touched a cache line per lane per load: 27 us for the 16 K tiles of
// the gradient-informed select.)
constexpr int kScanRows = 8;
__global__ __launch_bounds__(1024) void k_bm_prune_scan(uint32_t *tiles, int64_t nt, uint32_t *sel)
{
    constexpr int kWaves = 1024 / 64;
    constexpr int64_t kRound = (int64_t)kWaves * 64 * kScanRows;  // pairs per round
    __shared__ uint32_t wt[2][kWaves];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    uint2 *pairs = reinterpret_cast<uint2 *>(tiles);  // (below, equal) of tile i
    uint32_t carry0 = 0, carry1 = 0;                  // totals of the earlier rounds
    for (int64_t r0 = 0; r0 < nt; r0 += kRound) {
        const int64_t base = r0 + (int64_t)w * 64 * kScanRows + lane;
        uint2 v[kScanRows];
#pragma unroll
        for (int g = 0; g < kScanRows; ++g) {
            const int64_t i = base + 64 * g;
            const uint2 x = pairs[i < nt ? i : 0];
            v[g] = i < nt ? x : make_uint2(0u, 0u);
        }
        uint32_t run0 = 0, run1 = 0;  // the wave's pairs before row g
#pragma unroll
        for (int g = 0; g < kScanRows; ++g) {
            uint32_t a0 = v[g].x, a1 = v[g].y;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y0 = __shfl_up(a0, off, 64), y1 = __shfl_up(a1, off, 64);
                if (lane >= off) {
                    a0 += y0;
                    a1 += y1;
                }
            }
            const uint32_t own0 = v[g].x, own1 = v[g].y;
            v[g] = make_uint2(run0 + a0 - own0, run1 + a1 - own1);  // exclusive, within the wave's run
            run0 += __shfl(a0, 63, 64);
            run1 += __shfl(a1, 63, 64);
        }
        if (lane == 0) {
            wt[0][w] = run0;
            wt[1][w] = run1;
        }
        __syncthreads();
        uint32_t off0 = carry0, off1 = carry1, tot0 = 0, tot1 = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            if (k < w) {
                off0 += wt[0][k];
                off1 += wt[1][k];
            }
            tot0 += wt[0][k];
            tot1 += wt[1][k];
        }
#pragma unroll
        for (int g = 0; g < kScanRows; ++g) {
            const int64_t i = base + 64 * g;
            if (i < nt) pairs[i] = make_uint2(off0 + v[g].x, off1 + v[g].y);
        }
        carry0 += tot0;
        carry1 += tot1;
        __syncthreads();  // wt is written again in the next round
    }
    if (threadIdx.x == 0) {
        sel[kSelCounts + 4] = 0;
        sel[kSelCounts + 5] = 0;
    }
    // the select is done: clear its histograms for the next one
    for (int i = threadIdx.x; i < kMaxPasses * kHistWords; i += 1024) sel[i] = 0;
}

// Entry k goes if its key is below the threshold, or equal to it and fewer
// than need_eq equal keys precede it; the pruned ones are marked in a bit
// mask, one bit per canonical index.
// kPrefix: tiles holds the raw per-tile counts (k_bm_prune_scan skipped) and
// each block adds up the equal counts of the tiles before it; block 0 then
// also does the scan kernel's clean-up.  Used up to kPrefixTiles tiles.
constexpr int64_t kPrefixTiles = 2048;
template <class K, bool kPrefix>
__global__ __launch_bounds__(kThreads) void k_bm_prune_mark(K keyof, int64_t n,
                                                            uint32_t *__restrict__ sel,
                                                            const uint32_t *__restrict__ tiles,
                                                            uint64_t *__restrict__ pruned)
{
    constexpr int R = kWaveItems / kWave;
    __shared__ uint32_t we[4];
    __shared__ uint32_t wb[4];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const uint32_t T = sel[kSelT], need_eq = sel[kSelNeedEq];
    uint32_t eq_before = 0;
    if constexpr (kPrefix) {
        uint32_t v = 0;
        for (int64_t j = t; j < (int64_t)blockIdx.x; j += kThreads) v += tiles[2 * j + 1];
        v = wave_sum(v);
        if (lane == 0) wb[w] = v;
        __syncthreads();
        eq_before = wb[0] + wb[1] + wb[2] + wb[3];
        if (blockIdx.x == 0) {  // what k_bm_prune_scan does after its scan
            if (t == 0) {
                sel[kSelCounts + 4] = 0;
                sel[kSelCounts + 5] = 0;
            }
            for (int i = t; i < kMaxPasses * kHistWords; i += kThreads) sel[i] = 0;
        }
    }
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)w * kWaveItems;
    uint32_t key[R];
    uint32_t eq_w = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t k = base + j * kWave + lane;
        key[j] = keyof(k, n);
        eq_w += (uint32_t)__popcll(__ballot(k < n && key[j] == T));
    }
    if (lane == 0) we[w] = eq_w;
    __syncthreads();
    uint32_t eq_run = kPrefix ? eq_before : tiles[2 * blockIdx.x + 1];
    for (int i = 0; i < w; ++i) eq_run += we[i];
    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t k = base + j * kWave + lane;
        const bool valid = k < n;
        const bool eq = valid && key[j] == T;
        const uint64_t eqm = __ballot(eq);
        const uint32_t eqb = eq_run + (uint32_t)__popcll(eqm & below);
        const uint64_t gm = __ballot((valid && key[j] < T) || (eq && eqb < need_eq));
        if (lane == 0 && base + j * kWave < n) pruned[(base + j * kWave) >> 6] = gm;
        eq_run += (uint32_t)__popcll(eqm);
    }
}

// One thread per row-major bitmap word: its set bits are canonical entries
// pref[w], pref[w] + 1, ...; the next bitmap keeps the ones not pruned.
__global__ __launch_bounds__(kThreads) void k_bm_occ_prune(const uint32_t *__restrict__ occ,
                                                           const uint32_t *__restrict__ pref, int64_t nw,
                                                           const uint64_t *__restrict__ pruned,
                                                           uint32_t *__restrict__ occ_next)
{
    // Four consecutive words per thread (nw is a multiple of 8): 16-byte loads
    // and store, and one round of dependent loads for the whole bitmap.
    const int64_t w4 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (4 * w4 >= nw) return;
    const uint4 o4 = reinterpret_cast<const uint4 *>(occ)[w4], k4 = reinterpret_cast<const uint4 *>(pref)[w4];
    const uint32_t o[4] = {o4.x, o4.y, o4.z, o4.w}, k0[4] = {k4.x, k4.y, k4.z, k4.w};
    const uint32_t n = (uint32_t)(__popc(o4.x) + __popc(o4.y) + __popc(o4.z) + __popc(o4.w));
    // the words' entries k4.x .. k4.x + n - 1 (n <= 128) span at most three mask words
    const uint32_t base = k4.x >> 6;
    uint64_t m[3] = {0, 0, 0};
    if (n) {
        const uint32_t last = (k4.x + n - 1u) >> 6;
        m[0] = pruned[base];
        m[1] = pruned[base + 1 < last ? base + 1 : last];
        m[2] = pruned[last];
    }
    uint32_t keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        keep[i] = o[i];
        uint32_t k = k0[i];
        for (uint32_t b = o[i]; b; b &= b - 1, ++k) {
            const uint32_t d = (k >> 6) - base;  // 0, 1 or 2
            const uint64_t pw = d == 0 ? m[0] : (d == 1 ? m[1] : m[2]);
            if ((pw >> (k & 63)) & 1ull) keep[i] &= ~(b & (0u - b));
        }
    }
    reinterpret_cast<uint4 *>(occ_next)[w4] = make_uint4(keep[0], keep[1], keep[2], keep[3]);
}

// --------------------------------------------------------------------- regrow
__device__ __forceinline__ uint64_t hash_home(uint32_t p, int hbits)
{
    return ((uint64_t)p * 0x9E3779B97F4A7C15ull) >> (64 - hbits);
}

// Slot entry: position in the high word, candidate index in the low word; a
// slot keeps the smallest index seen for its position (same high word, so
// the 64-bit minimum is the minimum index).  Linear probing; the table has at
// least twice as many slots as candidates, so a free slot always exists.
// Finishes an insertion whose attempt at slot s found `old` there.
__device__ inline void hash_insert_from(uint64_t *tab, int hbits, uint32_t p, uint32_t j, uint64_t s, uint64_t old)
{
    const uint64_t mask = (1ull << hbits) - 1, entry = ((uint64_t)p << 32) | j;
    for (uint64_t probe = 0; probe <= mask; ++probe) {
        if (old == kEmptySlot) return;
        if ((uint32_t)(old >> 32) == p) {
            atomicMin((unsigned long long *)&tab[s], (unsigned long long)entry);
            return;
        }
        s = (s + 1) & mask;
        old = atomicCAS((unsigned long long *)&tab[s], kEmptySlot, entry);
    }
}

__device__ inline uint32_t hash_first(const uint64_t *tab, int hbits, uint32_t p)
{
    const uint64_t mask = (1ull << hbits) - 1;
    uint64_t s = hash_home(p, hbits);
    for (uint64_t probe = 0; probe <= mask; ++probe, s = (s + 1) & mask) {
        const uint64_t e = tab[s];
        if (e == kEmptySlot) return kNoPos;
        if ((uint32_t)(e >> 32) == p) return (uint32_t)e;
    }
    return kNoPos;
}

// Candidates [i0, i0 + M) of the stream (i0 a multiple of 4), one per
// thread: each thread computes its candidate's Philox block (four threads
// share one; recomputing it is cheaper than waiting on fewer, longer chains)
// and keeps its word.  Occupied positions drop out, the others enter the
// hash table.
// step_dev (restructure_async): the step is read from device memory instead.
__global__ __launch_bounds__(kThreads) void k_bm_cand_insert(uint64_t seed, uint64_t step,
                                                             const uint64_t *__restrict__ step_dev, uint64_t i0,
                                                             int64_t M, int64_t in, uint64_t npos, const uint32_t *occ,
                                                             int64_t inw, uint32_t *__restrict__ cand, uint64_t *tab,
                                                             int hbits)
{
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= M) return;
    uint64_t u[4];
    Philox4x64::block(seed, step_dev ? *step_dev : step, (i0 >> 2) + (uint64_t)(j >> 2), u);
    const int q = (int)(j & 3);
    const uint64_t uq = q == 0 ? u[0] : q == 1 ? u[1] : q == 2 ? u[2] : u[3];
    const uint64_t pq = __umul64hi(uq, npos);
    const uint32_t p = (uint32_t)pq;  // npos < 2^32 on the bitmap path: 32-bit division suffices
    const int64_t r = (int64_t)(p / (uint32_t)in), c = (int64_t)p - r * in;
    const bool free_ = !((occ[r * inw + (c >> 5)] >> (c & 31)) & 1u);
    cand[j] = free_ ? p : kNoPos;
    if (!free_) return;
    const uint64_t home = hash_home(p, hbits);
    const uint64_t old = atomicCAS((unsigned long long *)&tab[home], kEmptySlot, ((uint64_t)p << 32) | (uint64_t)j);
    hash_insert_from(tab, hbits, p, (uint32_t)j, home, old);
}

// flag[j] = candidate j is empty and the first of its position in the batch;
// one bit per candidate (a word per wave), and the count per block.
__global__ __launch_bounds__(kThreads) void k_bm_cand_count(const uint32_t *__restrict__ cand, int64_t M,
                                                            const uint64_t *__restrict__ tab, int hbits,
                                                            uint64_t *__restrict__ flags,
                                                            uint32_t *__restrict__ tile_cnt)
{
    __shared__ uint32_t part[4];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int64_t j = (int64_t)blockIdx.x * kThreads + t;
    bool f = false;
    if (j < M) {
        const uint32_t p = cand[j];
        f = p != kNoPos && hash_first(tab, hbits, p) == (uint32_t)j;
    }
    const uint64_t m = __ballot(f);
    if (lane == 0) {
        if (j < M) flags[j >> 6] = m;
        part[w] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (t == 0) tile_cnt[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

// One block of 1024: exclusive scan of the block counts; the batch takes
// min(flags, still needed) and the running total advances.  step_dev
// (restructure_async, one batch): the step counter moves on, and a batch that
// took fewer than n_prune positions sets a sticky flag (read back by the next
// synchronizing call, which then refuses the layer).
__global__ __launch_bounds__(1024) void k_bm_cand_scan(uint32_t *tile_cnt, int64_t nt, uint32_t n_prune,
                                                       uint32_t *sel, uint64_t *step_dev)
{
    __shared__ uint32_t lds[17];
    const int64_t per = ceil_div(nt, 1024), b0 = (int64_t)threadIdx.x * per;
    uint32_t sum = 0;
    for (int64_t i = b0; i < b0 + per && i < nt; ++i) sum += tile_cnt[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan(sum, lds, &total);
    for (int64_t i = b0; i < b0 + per && i < nt; ++i) {
        const uint32_t v = tile_cnt[i];
        tile_cnt[i] = run;
        run += v;
    }
    if (threadIdx.x == 0) {
        const uint32_t nacc = sel[kSelCounts + 4], need = n_prune - nacc;
        const uint32_t now = nacc + (total < need ? total : need);
        sel[kSelCounts + 5] = nacc;
        sel[kSelCounts + 4] = now;
        if (step_dev) {
            *step_dev += 1;
            if (now != n_prune) sel[kSelAsyncShort] = 1u;
        }
    }
}

// Flagged candidates ranked in stream order; those below the still-needed
// count are taken: their bit is set in the next bitmap.
__global__ __launch_bounds__(kThreads) void k_bm_cand_take(const uint32_t *__restrict__ cand, int64_t M,
                                                           const uint64_t *__restrict__ flags,
                                                           const uint32_t *__restrict__ tile_pre,
                                                           const uint32_t *__restrict__ sel, uint32_t n_prune,
                                                           int64_t in, uint32_t *occ, int64_t inw)
{
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int64_t j = (int64_t)blockIdx.x * kThreads + t;
    if (j >= M) return;
    const int64_t q0 = (int64_t)blockIdx.x * (kThreads / 64);
    uint32_t rank = tile_pre[blockIdx.x];
    for (int i = 0; i < w; ++i) rank += (uint32_t)__popcll(flags[q0 + i]);
    const uint64_t fw = flags[j >> 6];
    if (!((fw >> lane) & 1ull)) return;
    rank += (uint32_t)__popcll(fw & lanes_below());
    const uint32_t prev = sel[kSelCounts + 5];
    if (rank >= n_prune - prev) return;
    const uint32_t p = cand[j];
    const int64_t r = (int64_t)(p / (uint64_t)in), c = (int64_t)p - r * in;
    atomicOr(&occ[r * inw + (c >> 5)], 1u << (c & 31));
}

// ------------------------------------------------- gradient-informed regrow
// Score key of every padded bitmap position: 0 unless the position is inside
// the layer and empty after the prune, else 1 + bit pattern of |s| with
//     s = 0; for b = 0..B-1: s = fma(dY[b, r], X[b, c], s)     (fp32)
// -- the fused-multiply-add chain in batch order, so the integer decision
// "which positions come back" is the same on any implementation that keeps
// this order.  Block = 128 rows x 128 columns; thread = 8 rows x 8 columns
// (64 independent chains in registers, one LDS word per four FMAs); dY and X
// tiles of kScoreB batch rows at a time in LDS.
constexpr int kScoreTile = 128;
constexpr int kScoreB = 32;
// The block also adds its keys to the first histogram pass of the select
// that follows (hist0: pass 0's kCopies x 256 bins, digit (~key >> shift0) &
// 255, in the select's order of InvKeys), so that pass needs no launch of
// its own: per-block counts in LDS (4 copies by lane), then one atomic per
// nonzero bin into copy blockIdx % kCopies.
template <class D>
__global__ __launch_bounds__(kThreads) void k_bm_scores(const typename D::T *__restrict__ dY,
                                                        const typename D::T *__restrict__ X, int64_t B, int64_t out,
                                                        int64_t in, const uint32_t *__restrict__ occ, int64_t inw,
                                                        int64_t rows_alloc, uint32_t *__restrict__ keys,
                                                        uint32_t *__restrict__ hist0, int shift0)
{
    __shared__ __align__(16) float ty[kScoreB][kScoreTile + 4];  // [b][row]
    __shared__ __align__(16) float tx[kScoreB][kScoreTile + 4];  // [b][col]
    constexpr int kHistCopies = 4;  // keeps four blocks' LDS within a CU
    __shared__ uint32_t hh[kHistCopies][256];
    const int t = threadIdx.x, tr = t >> 4, tc = t & 15;         // 16 x 16 threads, 8 x 8 each
    for (int i = t; i < kHistCopies * 256; i += kThreads) (&hh[0][0])[i] = 0u;  // ordered by the first barrier below
    const int64_t ncb = inw * 32 / kScoreTile;                    // column blocks
    const int64_t r0 = (int64_t)(blockIdx.x / ncb) * kScoreTile, c0 = (int64_t)(blockIdx.x % ncb) * kScoreTile;
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int64_t b0 = 0; b0 < B; b0 += kScoreB) {
        const int nb = B - b0 < kScoreB ? (int)(B - b0) : kScoreB;
        __syncthreads();
        for (int e = t; e < kScoreB * kScoreTile; e += kThreads) {
            const int bb = e / kScoreTile, k = e % kScoreTile;
            const bool okb = bb < nb;
            const int64_t r = r0 + k, c = c0 + k;
            ty[bb][k] = okb && r < out ? D::load(dY, (b0 + bb) * out + r) : 0.f;
            tx[bb][k] = okb && c < in ? D::load(X, (b0 + bb) * in + c) : 0.f;
        }
        __syncthreads();
        for (int bb = 0; bb < nb; ++bb) {
            const float4 y0 = *reinterpret_cast<const float4 *>(&ty[bb][tr * 8]);
            const float4 y1 = *reinterpret_cast<const float4 *>(&ty[bb][tr * 8 + 4]);
            const float4 x0 = *reinterpret_cast<const float4 *>(&tx[bb][tc * 8]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&tx[bb][tc * 8 + 4]);
            const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __fmaf_rn(y[i], x[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + tr * 8 + i;
        if (r >= rows_alloc) break;
        const int64_t c = c0 + tc * 8;  // eight consecutive columns in one bitmap word
        const uint32_t w = occ[r * inw + (c >> 5)];
        uint32_t kv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool live = r < out && c + j < in && !((w >> ((c + j) & 31)) & 1u);
            kv[j] = live ? (__float_as_uint(fabsf(acc[i][j])) + 1u) : 0u;
        }
        uint4 *dst = reinterpret_cast<uint4 *>(keys + r * inw * 32 + c);
        dst[0] = make_uint4(kv[0], kv[1], kv[2], kv[3]);
        dst[1] = make_uint4(kv[4], kv[5], kv[6], kv[7]);
#pragma unroll
        for (int j = 0; j < 8; ++j) atomicAdd(&hh[t & (kHistCopies - 1)][(~kv[j] >> shift0) & 255u], 1u);
    }
    __syncthreads();
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kHistCopies; ++k) cnt += hh[k][t];
    if (cnt) atomicAdd(&hist0[(blockIdx.x & (kCopies - 1)) * 256 + t], cnt);
}
static_assert(kThreads == 256, "one thread per bin of the scores' histogram");

// Adds the chosen positions (bit mask in bitmap word order) to the next
// bitmap; records that all n_prune are taken.
__global__ __launch_bounds__(kThreads) void k_bm_or(uint32_t *__restrict__ occ, const uint32_t *__restrict__ chosen,
                                                    int64_t nw, uint32_t *sel, uint32_t n_prune)
{
    const int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (w < nw) occ[w] |= chosen[w];
    if (w == 0) sel[kSelCounts + 4] = n_prune;
}

// -------------------------------------------------------------------- rebuild
// Canonical arrays from the next bitmap, one thread per word (its set bits
// are consecutive canonical indices from pref[w] on).  A position that was
// occupied before and not pruned keeps its value, read at its old canonical
// index; any other (regrown, also a just-pruned one) gets the regrow value.
// The thread of a row's first word also writes row_ptr.
template <typename V>
struct CanonArgs {
    const uint32_t *occ, *pref, *occ_old, *pref_old;
    const uint64_t *pruned;
    const V *vals_old;
    V regrow;
    uint32_t nw, inw;
    int64_t out;
    int32_t *rows, *cols;
    V *vals;
    int32_t *row_ptr, *tptr;
    int64_t ncb;
};

template <typename V>
__device__ __forceinline__ void bm_canon(uint32_t w, const CanonArgs<V> &A)
{
    const uint32_t *__restrict__ occ = A.occ, *__restrict__ pref = A.pref, *__restrict__ occ_old = A.occ_old,
                                 *__restrict__ pref_old = A.pref_old;
    const uint64_t *__restrict__ pruned = A.pruned;
    const V *__restrict__ vals_old = A.vals_old;
    const V regrow = A.regrow;
    const uint32_t nw = A.nw, inw = A.inw;
    const int64_t out = A.out, ncb = A.ncb;
    int32_t *__restrict__ rows = A.rows, *__restrict__ cols = A.cols, *__restrict__ row_ptr = A.row_ptr,
            *__restrict__ tptr = A.tptr;
    V *__restrict__ vals = A.vals;
    if (w > nw) return;
    const uint32_t r = w / inw, cw = w - r * inw;
    uint32_t pos = pref[w];
    if (cw == 0 && r <= out) row_ptr[r] = (int32_t)pos;
    // Tile offsets of the row view (when the layer has tiles): the first entry
    // of row r at column 512 k or later is the rank of the row's word 16 k,
    // and the row's end is the next row's start.
    if (tptr) {
        if (cw == 0 && r >= 1 && r - 1 < out) tptr[(int64_t)(r - 1) * (ncb + 1) + ncb] = (int32_t)pos;
        if (r < out && (cw & 15u) == 0 && (int64_t)(cw >> 4) < ncb) tptr[(int64_t)r * (ncb + 1) + (cw >> 4)] = (int32_t)pos;
    }
    if (w == nw) return;
    const uint32_t o = occ[w], oo = occ_old[w], ko = pref_old[w];
    // The word's old entries are canonical indices ko .. ko + nold - 1: their
    // prune bits lie in at most two mask words, loaded once.
    const uint32_t nold = (uint32_t)__popc(oo), k0 = ko & ~63u;
    uint64_t p0 = 0, p1 = 0;
    if (nold) {
        p0 = pruned[ko >> 6];
        if (((ko + nold - 1) >> 6) != (ko >> 6)) p1 = pruned[(ko >> 6) + 1];
    }
    // Four set bits per pass, so their value loads are in flight together.
    constexpr int P = 4;
    for (uint32_t m = o; m;) {
        int b[P];
        uint32_t k[P];
        bool has[P], keep[P];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            has[j] = m != 0;
            b[j] = has[j] ? __ffs(m) - 1 : 0;
            m &= m - 1;
            k[j] = ko + (uint32_t)__popc(oo & ((1u << b[j]) - 1u));
            const uint32_t off = k[j] - k0;
            const bool gone = off < 64 ? (p0 >> off) & 1ull : (p1 >> ((off - 64) & 63)) & 1ull;
            keep[j] = has[j] && ((oo >> b[j]) & 1u) && !gone;
        }
        V v[P];
#pragma unroll
        for (int j = 0; j < P; ++j) v[j] = keep[j] ? vals_old[k[j]] : regrow;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (has[j]) {
                rows[pos + j] = (int32_t)r;
                cols[pos + j] = (int32_t)(cw * 32 + b[j]);
                vals[pos + j] = v[j];
            }
        pos += P;  // only read again when the word had P more bits
    }
}

// The transposed view is built in tiles of 1024 rows x 64 columns (two
// bitmap words per row), one block each.  Each 64-row slice of a tile's words
// is turned into column words by 32 x 32 bit transposes across the lanes, so
// a column's entries in row order are the set bits of its 32 column words.
constexpr int kTR = 1024, kTC = 64, kTSlices = kTR / 64;
static_assert(kTR == 2 * kTileCols && kTileCols == 16 * 32, "a transposition chunk holds two tile blocks of 16 column words");

__device__ __forceinline__ uint2 tile_row_words(const uint32_t *__restrict__ occ, int64_t r, int64_t rows_alloc,
                                                int64_t inw, int64_t cg)
{
    const bool ok = r < rows_alloc;
    const uint2 w = *(const uint2 *)(occ + (ok ? r : 0) * inw + 2 * cg);
    return ok ? w : make_uint2(0u, 0u);
}

// Entries per column within each 1024-row chunk: tcnt[c * nrc + chunk], and
// their sum over the tile's 64 columns: gsum[column group * nrc + chunk].
// One block per tile (block index bid), wave w takes slices w, w + 4, ...
__device__ __forceinline__ void bm_tcount(int64_t bid, const uint32_t *__restrict__ occ, int64_t inw,
                                          int64_t rows_alloc, int64_t nrc, uint32_t *__restrict__ tcnt,
                                          uint32_t *__restrict__ gsum)
{
    __shared__ uint32_t part[4][kTC];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t rc = bid % nrc, cg = bid / nrc;
    uint2 wd[kTSlices / 4];
#pragma unroll
    for (int i = 0; i < kTSlices / 4; ++i)
        wd[i] = tile_row_words(occ, rc * kTR + (4 * i + w) * 64 + lane, rows_alloc, inw, cg);
    uint32_t c0 = 0, c1 = 0;  // lane i: columns i & 31 and 32 + (i & 31), rows of its half-slice
#pragma unroll
    for (int i = 0; i < kTSlices / 4; ++i) {
        if (__ballot((wd[i].x | wd[i].y) != 0u) == 0) continue;
        c0 += (uint32_t)__popc(transpose32(wd[i].x));
        c1 += (uint32_t)__popc(transpose32(wd[i].y));
    }
    c0 += __shfl_xor(c0, 32, 64);
    c1 += __shfl_xor(c1, 32, 64);
    if (lane < 32) {
        part[w][lane] = c0;
        part[w][32 + lane] = c1;
    }
    __syncthreads();
    static_assert(kTC == kWave, "the tile's columns are the lanes of wave 0");
    if (threadIdx.x < kTC) {
        const int c = threadIdx.x;
        const uint32_t n = part[0][c] + part[1][c] + part[2][c] + part[3][c];
        tcnt[(cg * kTC + c) * nrc + rc] = n;
        const uint32_t g = wave_sum(n);
        if (c == 0) gsum[cg * nrc + rc] = g;
    }
}

// The canonical arrays and the per-chunk column counts read only the next
// bitmap and its ranks, so one launch does both: the ntc count blocks
// first, then one thread per bitmap word.
template <typename V>
__global__ __launch_bounds__(kThreads) void k_bm_canon_tcount(CanonArgs<V> A, int64_t rows_alloc, int64_t nrc,
                                                              uint32_t *__restrict__ tcnt, uint32_t *__restrict__ gsum,
                                                              uint32_t ntc)
{
    if (blockIdx.x < ntc) {
        bm_tcount(blockIdx.x, A.occ, A.inw, rows_alloc, nrc, tcnt, gsum);
        return;
    }
    bm_canon<V>((blockIdx.x - ntc) * kThreads + threadIdx.x, A);
}

// Plain copies of three arrays of 32-bit words (16-byte aligned): piece i of
// their concatenation is 16 bytes, copied word by word at an array's end.
struct CopySeg {
    const uint32_t *src;
    uint32_t *dst;
    int64_t n;
};
__device__ __forceinline__ void copy3_piece(int64_t i, const CopySeg &a, const CopySeg &b, const CopySeg &c)
{
    const int64_t na = ceil_div(a.n, 4), nb = ceil_div(b.n, 4);
    const CopySeg &g = i < na ? a : (i < na + nb ? b : c);
    const int64_t j = i < na ? i : (i < na + nb ? i - na : i - na - nb), w = 4 * j;
    if (w + 4 <= g.n) reinterpret_cast<uint4 *>(g.dst)[j] = reinterpret_cast<const uint4 *>(g.src)[j];
    else
        for (int64_t k = w; k < g.n; ++k) g.dst[k] = g.src[k];
}
__host__ __device__ inline int64_t copy3_pieces(const CopySeg &a, const CopySeg &b, const CopySeg &c)
{
    return ceil_div(a.n, 4) + ceil_div(b.n, 4) + ceil_div(c.n, 4);
}

// Transposed view, one block per tile: the tile's output is, per column, a
// run of consecutive transposed ranks, starting after the entries of all
// earlier column groups (gsum), of the group's earlier columns and of the
// column's earlier row chunks (tcnt); wave 0 adds these up while the tile's
// bitmap words load, so no scan pass runs in between.  Lanes walk the tile's
// entries in that order, so stores are
// coalesced: output o -> column (search in the column starts) -> row (search
// in the column's cumulative word counts, then the bit) -> canonical index
// (the row's first entry in the tile plus its entries to the left).  rc = 0
// also writes col_ptr.  Blocks from ntiles on copy the pieces of (ca, cb, cc)
// instead (restructure_async's write-back, which reads nothing the tiles
// write and writes nothing they read).
template <typename V>
__global__ __launch_bounds__(kThreads) void k_bm_tgather(const uint32_t *__restrict__ occ,
                                                   const uint32_t *__restrict__ pref, int64_t inw, int64_t rows_alloc,
                                                   int64_t nrc, int64_t in, const uint32_t *__restrict__ tcnt,
                                                   const uint32_t *__restrict__ gsum,
                                                   const V *__restrict__ vals, int32_t *__restrict__ perm_c,
                                                   int32_t *__restrict__ rows_by_col, V *__restrict__ vals_c,
                                                   int32_t *__restrict__ col_ptr, int32_t *__restrict__ tptr,
                                                   int64_t nrb, int64_t ntiles, CopySeg ca, CopySeg cb, CopySeg cc)
{
    if ((int64_t)blockIdx.x >= ntiles) {
        const int64_t i = ((int64_t)blockIdx.x - ntiles) * kThreads + threadIdx.x;
        if (i < copy3_pieces(ca, cb, cc)) copy3_piece(i, ca, cb, cc);
        return;
    }
    __shared__ uint2 rw[kTR];                     // row words
    __shared__ uint32_t seg[kTR];                 // canonical index of the row's first entry in the tile
    __shared__ uint32_t cw[kTC][kTR / 32 + 1];    // column words (padded against bank conflicts)
    __shared__ uint16_t ccum[kTC][kTR / 32 + 1];  // set bits in the column's earlier words
    __shared__ uint32_t cstart[kTC + 1];          // tile-local start of each column's run
    __shared__ uint32_t gout[kTC];                // transposed rank of each run's first entry
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t rc = blockIdx.x % nrc, cg = blockIdx.x / nrc, r0 = rc * kTR;
    const int64_t c_glob = cg * kTC + lane;
    uint32_t col_start = 0, group_end = 0;  // wave 0: lane's column, and the group's end
    if (wv == 0) {
        constexpr int U = 8;
        const int64_t ng = cg * nrc;  // chunk sums of the earlier column groups
        uint32_t groups = 0;
        for (int64_t k0 = lane; k0 < ng; k0 += U * kWave) {
            uint32_t x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t k = k0 + u * kWave;
                const uint32_t v = gsum[k < ng ? k : 0];
                x[u] = k < ng ? v : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) groups += x[u];
        }
        groups = wave_sum(groups);
        uint32_t col = 0, above = 0;  // the column's entries, and those in chunks before rc
        for (int64_t k0 = 0; k0 < nrc; k0 += U) {
            uint32_t x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t k = k0 + u;
                const uint32_t v = tcnt[c_glob * nrc + (k < nrc ? k : 0)];
                x[u] = k < nrc ? v : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                col += x[u];
                above += k0 + u < rc ? x[u] : 0u;
            }
        }
        uint32_t incl = col;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        col_start = groups + (incl - col) + above;
        group_end = groups + __shfl(incl, 63, 64);
    }
#pragma unroll
    for (int i = 0; i < kTSlices / 4; ++i) {
        const int sl = 4 * i + wv;
        const int64_t r = r0 + sl * 64 + lane;
        const uint2 w = tile_row_words(occ, r, rows_alloc, inw, cg);
        rw[sl * 64 + lane] = w;
        seg[sl * 64 + lane] = pref[(r < rows_alloc ? r : 0) * inw + 2 * cg];
        cw[lane & 31][2 * sl + (lane >> 5)] = transpose32(w.x);
        cw[32 + (lane & 31)][2 * sl + (lane >> 5)] = transpose32(w.y);
    }
    __syncthreads();
    __shared__ uint32_t total_s;
    if (wv == 0) {
        uint32_t run = 0;  // lane = column
        for (int b = 0; b < kTR / 32; ++b) {
            ccum[lane][b] = (uint16_t)run;
            run += (uint32_t)__popc(cw[lane][b]);
        }
        uint32_t incl = run;  // scan of the column counts over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        cstart[lane] = incl - run;
        if (lane == 63) {
            cstart[kTC] = incl;
            total_s = incl;
        }
        gout[lane] = col_start;
        if (rc == 0 && c_glob < in) col_ptr[c_glob] = (int32_t)gout[lane];
        if (rc == 0 && cg == inw / 2 - 1 && lane == 63) col_ptr[in] = (int32_t)group_end;  // every entry
        // Tile offsets of the column view (when the layer has tiles), in
        // 512-row blocks: this chunk's two blocks start at the column's first
        // entry in the chunk and after its entries in the chunk's first 512
        // rows (its first 16 column words); the last chunk also writes the
        // column's end.
        if (tptr && c_glob < in) {
            int32_t *tp = tptr + c_glob * (nrb + 1);
            const int64_t k0 = 2 * rc;
            if (k0 < nrb) tp[k0] = (int32_t)gout[lane];
            if (k0 + 1 < nrb) tp[k0 + 1] = (int32_t)(gout[lane] + ccum[lane][16]);
            if (rc == nrc - 1) tp[nrb] = (int32_t)(gout[lane] + run);
        }
    }
    __syncthreads();
    const uint32_t total = total_s;
    // Outputs in flight per thread.  Each search step is taken for all of
    // them together, without branches, so their LDS reads issue back to back
    // instead of as U dependent chains.
    constexpr int U = 4;
    for (uint32_t o0 = 0; o0 < total; o0 += kThreads * U) {
        uint32_t o[U], q[U];
        int c[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            o[u] = o0 + u * kThreads + t;
            c[u] = 0;  // last column whose run starts at or before o
            b[u] = 0;  // column word holding the q-th entry of that column
        }
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1)
#pragma unroll
            for (int u = 0; u < U; ++u) c[u] += cstart[c[u] + step] <= o[u] ? step : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) q[u] = o[u] < total ? o[u] - cstart[c[u]] : 0u;
#pragma unroll
        for (int step = 16; step >= 1; step >>= 1)
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] += ccum[c[u]][b[u] + step] <= q[u] ? step : 0;
        int32_t kk[U], rr[U];
        uint32_t jj[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ro = b[u] * 32 + nth_set_bit(cw[c[u]][b[u]], q[u] - ccum[c[u]][b[u]]);
            const uint2 w = rw[ro];
            // entries of the row left of column c within the tile's two words
            const uint32_t below = (1u << (c[u] & 31)) - 1u;
            const uint32_t mx = c[u] < 32 ? below : ~0u, my = c[u] < 32 ? 0u : below;
            const uint32_t left = (uint32_t)__popc(w.x & mx) + (uint32_t)__popc(w.y & my);
            kk[u] = o[u] < total ? (int32_t)(seg[ro] + left) : -1;
            rr[u] = (int32_t)(r0 + ro);
            jj[u] = gout[c[u]] + q[u];
        }
        V vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) vv[u] = vals[kk[u] >= 0 ? kk[u] : 0];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (kk[u] >= 0) {
                perm_c[jj[u]] = kk[u];
                rows_by_col[jj[u]] = rr[u];
                vals_c[jj[u]] = vv[u];
            }
    }
}

__global__ void k_bm_occ_set(const int32_t *__restrict__ rows, const int32_t *__restrict__ cols, int64_t n,
                             uint32_t *occ, int64_t inw)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const int32_t r = rows[k], c = cols[k];
    atomicOr(&occ[(int64_t)r * inw + (c >> 5)], 1u << (c & 31));
}

inline unsigned blocks_for(int64_t items, int64_t per_block) { return (unsigned)ceil_div(items, per_block); }

int hash_bits_for(int64_t M)  // smallest b with 2^b >= 2M
{
    const int b = bits_for((uint64_t)(2 * M - 1));
    return b < 1 ? 1 : b;
}

template <typename V>
struct BitmapRun {
    csp_layer *L;
    int64_t n_prune;
    uint64_t seed, step, npos;
    V regrow;
    hipStream_t s;
    uint64_t i0 = 0;
    int64_t nacc = 0;
    const uint64_t *step_dev = nullptr;  // restructure_async: the step lives on the device

    int64_t batch_size(int64_t cap) const
    {
        const int64_t need = n_prune - nacc, nkept = L->nnz - n_prune;
        const double free_frac = (double)(npos - (uint64_t)nkept - (uint64_t)nacc) / (double)npos;
        const double want = (double)need / free_frac * 1.1 + 1024.0;
        int64_t M = want > (double)cap ? cap : (int64_t)want;
        M -= M % 4;  // whole Philox blocks, so every batch starts at a multiple of 4
        return M < 4 ? 4 : M;
    }

    csp_status batch(int64_t M, int hb)
    {
        Workspace &W = L->ws;
        const unsigned nt = blocks_for(M, kThreads);
        k_bm_cand_insert<<<blocks_for(M, kThreads), kThreads, 0, s>>>(seed, step, step_dev, i0, M, L->in, npos,
                                                                      W.occ_next, W.occ_row_words, W.u_a, W.hash, hb);
        CSP_LAUNCHED("k_bm_cand_insert");
        k_bm_cand_count<<<nt, kThreads, 0, s>>>(W.u_a, M, W.hash, hb, (uint64_t *)W.u_b, W.hist);
        CSP_LAUNCHED("k_bm_cand_count");
        k_bm_cand_scan<<<1, 1024, 0, s>>>(W.hist, nt, (uint32_t)n_prune, W.sel, const_cast<uint64_t *>(step_dev));
        CSP_LAUNCHED("k_bm_cand_scan");
        k_bm_cand_take<<<nt, kThreads, 0, s>>>(W.u_a, M, (const uint64_t *)W.u_b, W.hist, W.sel, (uint32_t)n_prune,
                                               L->in, W.occ_next, W.occ_row_words);
        CSP_LAUNCHED("k_bm_cand_take");
        i0 += (uint64_t)M;
        return CSP_OK;
    }

    // Canonical arrays, transposed view and offsets from the next bitmap, task
    // lists.  rows_out and cols_out take the canonical rows and columns (the
    // staged arrays, or the layer's own: nothing of the old ones is read);
    // the values always go to the staged array (the old ones are read).
    csp_status rebuild_device(int32_t *rows_out, int32_t *cols_out, const CopySeg *copy = nullptr)
    {
        Workspace &W = L->ws;
        const int64_t nw = W.occ_words, inw = W.occ_row_words, rows_alloc = W.occ_rows;
        const int64_t nrc = ceil_div(rows_alloc, kTR), ncg = inw / 2, ntiles = nrc * ncg;
        csp_status st = exclusive_scan_popc(W.occ_next, W.occ_pref_next, nw, W.hist, s);
        if (st != CSP_OK) return st;
        const CanonArgs<V> ca{W.occ_next, W.occ_pref_next, W.occ, W.occ_pref, (const uint64_t *)W.acc_b,
                              (const V *)L->vals, regrow, (uint32_t)nw, (uint32_t)inw, L->out, rows_out, cols_out,
                              (V *)W.vals_k, L->row_ptr, L->tiles_r.ptr, L->tiles_r.ncb};
        uint32_t *gsum = W.tcnt + ncg * kTC * nrc;  // after the per-column counts
        k_bm_canon_tcount<V><<<(unsigned)ntiles + blocks_for(nw + 1, kThreads), kThreads, 0, s>>>(
            ca, rows_alloc, nrc, W.tcnt, gsum, (uint32_t)ntiles);
        CSP_LAUNCHED("k_bm_canon_tcount");
        const CopySeg none{nullptr, nullptr, 0};
        const CopySeg c0 = copy ? copy[0] : none, c1 = copy ? copy[1] : none, c2 = copy ? copy[2] : none;
        const unsigned cblocks = blocks_for(copy3_pieces(c0, c1, c2), kThreads);
        k_bm_tgather<V><<<(unsigned)ntiles + cblocks, kThreads, 0, s>>>(
            W.occ_next, W.occ_pref_next, inw, rows_alloc, nrc, L->in, W.tcnt, gsum, (const V *)W.vals_k, L->perm_c,
            L->rows_by_col, (V *)L->vals_c, L->col_ptr, L->tiles_c.ptr, L->tiles_c.ncb, ntiles, c0, c1, c2);
        CSP_LAUNCHED("k_bm_tgather");
        L->tile_ptr_ready = L->tiles_r.ptr != nullptr;  // build_tiles then only orders the tiles' rows
        if (step_dev && L->tile_partial) {
            // restructure_async on a layer with tiles: the task lists wait for
            // the first call that reads them (tasks_ready).
            L->tasks_pending = true;
            return CSP_OK;
        }
        return build_task_lists(L, s, L->narrow_seen);
    }

    // Eager rebuild: staged arrays, then the read-back of the taken count and
    // the task counts; the staged arrays and bitmap become the layer's by
    // pointer swaps.
    csp_status rebuild()
    {
        Workspace &W = L->ws;
        csp_status st = rebuild_device(W.rows_k, W.cols_k);
        if (st != CSP_OK) return st;
        uint32_t counts[kSelCountWords] = {};
        CSP_HIP(hipMemcpyAsync(counts, W.sel + kSelCounts, sizeof counts, hipMemcpyDeviceToHost, s));
        CSP_HIP(hipStreamSynchronize(s));
        nacc = counts[4];
        if (nacc != n_prune) return CSP_OK;  // short: another batch, then rebuild again
        st = set_task_counts(L, counts);
        if (st != CSP_OK) return st;
        // The staged canonical arrays and the next bitmap become the layer's.
        std::swap(L->rows, W.rows_k);
        std::swap(L->cols, W.cols_k);
        std::swap(L->vals, W.vals_k);
        std::swap(W.occ, W.occ_next);
        std::swap(W.occ_pref, W.occ_pref_next);
        return CSP_OK;
    }

    // Radix select of the `count` smallest keys of keyof over [0, n), then a
    // bit per index of the chosen ones (ties go to the smaller index) in mask;
    // `clear` (optional) is filled with empty hash slots by the first pass.
    template <class K>
    // first = 1: pass 0's histogram is already in place (the producer of the
    // keys counted them), and there is nothing to clear.
    csp_status select(K keyof, int64_t n, int64_t count, int passes, int top, uint64_t *mask, uint64_t *clear,
                      int64_t nclear, int first = 0)
    {
        Workspace &W = L->ws;
        const int64_t hgrid = ceil_div(n, kHistThreads * 8) < 256 ? ceil_div(n, kHistThreads * 8) : 256;
        for (int p = first; p < passes; ++p) {
            k_bm_hist<K><<<(unsigned)hgrid, kHistThreads, 0, s>>>(keyof, n, p, top, (uint32_t)count, W.sel,
                                                                   p == 0 ? clear : nullptr, p == 0 ? nclear : 0);
            CSP_LAUNCHED("k_bm_hist");
        }
        k_bm_sel_final<<<1, 64, 0, s>>>(W.sel, (uint32_t)count, passes, top);
        CSP_LAUNCHED("k_bm_sel_final");
        const int64_t nt = ceil_div(n, kTile);
        k_bm_prune_count<K><<<(unsigned)nt, kThreads, 0, s>>>(keyof, n, W.sel, W.hist);
        CSP_LAUNCHED("k_bm_prune_count");
        if (nt <= kPrefixTiles) {
            k_bm_prune_mark<K, true><<<(unsigned)nt, kThreads, 0, s>>>(keyof, n, W.sel, W.hist, mask);
        } else {
            k_bm_prune_scan<<<1, 1024, 0, s>>>(W.hist, nt, W.sel);
            CSP_LAUNCHED("k_bm_prune_scan");
            k_bm_prune_mark<K, false><<<(unsigned)nt, kThreads, 0, s>>>(keyof, n, W.sel, W.hist, mask);
        }
        CSP_LAUNCHED("k_bm_prune_mark");
        return CSP_OK;
    }

    // Prune: mark the n_prune entries first in the prune order, and start the
    // next bitmap as the current one without them.
    csp_status prune(uint64_t *clear, int64_t nclear)
    {
        Workspace &W = L->ws;
        const int passes = sizeof(V) == 4 ? 4 : 2, top = sizeof(V) == 4 ? 24 : 8;
        csp_status st = select(MagKeys<V>{(const V *)L->vals}, L->nnz, n_prune, passes, top, (uint64_t *)W.acc_b,
                               clear, nclear);
        if (st != CSP_OK) return st;
        k_bm_occ_prune<<<blocks_for(W.occ_words / 4, kThreads), kThreads, 0, s>>>(W.occ, W.occ_pref, W.occ_words,
                                                                              (const uint64_t *)W.acc_b, W.occ_next);
        CSP_LAUNCHED("k_bm_occ_prune");
        return CSP_OK;
    }

    // Gradient-informed regrow: the n_prune empty positions with the largest
    // score keys (ties to the smaller position) join the next bitmap.
    template <class D>
    csp_status regrow_by_gradient(const void *dY, const void *X, int64_t B)
    {
        Workspace &W = L->ws;
        const int64_t npad = W.occ_words * 32;  // padded positions, bitmap order
        const int64_t rblk = ceil_div(W.occ_rows, kScoreTile), cblk = W.occ_row_words * 32 / kScoreTile;
        k_bm_scores<D><<<(unsigned)(rblk * cblk), kThreads, 0, s>>>((const typename D::T *)dY,
                                                                     (const typename D::T *)X, B, L->out, L->in,
                                                                     W.occ_next, W.occ_row_words, W.occ_rows,
                                                                     W.score, W.sel, 24);
        CSP_LAUNCHED("k_bm_scores");
        uint64_t *chosen = (uint64_t *)W.occ_pref_next;  // scratch until the rebuild
        csp_status st = select(InvKeys{W.score}, npad, n_prune, 4, 24, chosen, nullptr, 0, 1);
        if (st != CSP_OK) return st;
        k_bm_or<<<blocks_for(W.occ_words, kThreads), kThreads, 0, s>>>(W.occ_next, (const uint32_t *)chosen,
                                                                       W.occ_words, W.sel, (uint32_t)n_prune);
        CSP_LAUNCHED("k_bm_or");
        return rebuild();
    }

    // restructure_async: one batch of candidates sized with a wide margin,
    // the rebuild writing the layer's own arrays (values and bitmaps copied
    // back from their staged halves instead of swapped, so the buffers a
    // captured graph holds stay the layer's), no read-back.
    csp_status run_async(int64_t M)
    {
        Workspace &W = L->ws;
        const int hb = hash_bits_for(M);
        csp_status st = prune(W.hash, int64_t(1) << hb);
        if (st == CSP_OK) st = batch(M, hb);
        if (st != CSP_OK) return st;
        // the staged values and bitmaps written back by the transposing launch
        const CopySeg copy[3] = {
            {(const uint32_t *)W.vals_k, (uint32_t *)L->vals, ceil_div(L->nnz * (int64_t)sizeof(V), 4)},
            {W.occ_next, W.occ, W.occ_words},
            {W.occ_pref_next, W.occ_pref, W.occ_words + 1}};
        return rebuild_device(L->rows, L->cols, copy);
    }

    csp_status run()
    {
        Workspace &W = L->ws;
        int64_t cap = W.bm_batch_cap;
        if (const char *e = std::getenv("COOSPMM_REGROW_BATCH")) {  // test hook: smaller batches
            long long v = std::atoll(e);
            if (v >= 1 && v < cap) cap = v;
        }
        int64_t M = batch_size(cap);
        int hb = hash_bits_for(M);
        csp_status st = prune(W.hash, int64_t(1) << hb);
        if (st != CSP_OK) return st;
        st = batch(M, hb);
        if (st != CSP_OK) return st;
        st = rebuild();
        if (st != CSP_OK) return st;
        for (int64_t batches = 1; nacc < n_prune; ++batches) {
            if (batches >= 4096)
                return set_error(CSP_ERR_INVALID_ARG, "regrow found only %lld of %lld empty positions in %llu draws",
                                 (long long)nacc, (long long)n_prune, (unsigned long long)i0);
            M = batch_size(cap);
            hb = hash_bits_for(M);
            st = fill_u32((uint32_t *)W.hash, 0xFFFFFFFFu, int64_t(2) << hb, s);
            if (st != CSP_OK) return st;
            st = batch(M, hb);
            if (st != CSP_OK) return st;
            st = rebuild();
            if (st != CSP_OK) return st;
        }
        return CSP_OK;
    }
};

}  // namespace

bool plan_bitmap(csp_layer *L)
{
    Workspace &W = L->ws;
    W.bitmap = false;
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    if (npos >= (uint64_t(1) << 32)) return false;
    if (const char *e = std::getenv("COOSPMM_RESTRUCTURE"))  // test hook: force the sorted path
        if (std::strcmp(e, "sorted") == 0) return false;
    const int64_t inw = ceil_div(L->in, 256) * 8, rows_alloc = ceil_div(L->out, 64) * 64;
    const int64_t nw = rows_alloc * inw, tcnt = (inw * 32 + inw / 2) * ceil_div(rows_alloc, kTR);
    // two bitmaps and their ranks, the transposition counts and their sums per tile
    const size_t bytes = (size_t)nw * 16 + 8 + (size_t)tcnt * 4;
    if (bytes > kBitmapBytesLimit) return false;
    W.bitmap = true;
    W.occ_words = nw;
    W.occ_row_words = inw;
    W.occ_rows = rows_alloc;
    W.tcnt_words = tcnt;
    W.bm_batch_cap = W.nkey_cap < kBatchLimit ? W.nkey_cap : kBatchLimit;
    W.hash_slots = int64_t(1) << hash_bits_for(W.bm_batch_cap);
    return true;
}

size_t bitmap_hist_words(const csp_layer *L)
{
    const Workspace &W = L->ws;
    if (!W.bitmap) return 0;
    const int64_t a = 2 * ceil_div(L->nnz, kTile) + 2, b = ceil_div(W.bm_batch_cap, kThreads) + 2,
                  c = ceil_div(W.occ_words, 4096) + 2, d = ceil_div(W.tcnt_words, 4096) + 2,
                  e = 2 * ceil_div(W.occ_words * 32, kTile) + 2;  // tiles of the gradient regrow select
    int64_t m = a > b ? a : b;
    m = m > c ? m : c;
    m = m > d ? m : d;
    return (size_t)(m > e ? m : e);
}

csp_status occupancy_init(csp_layer *L, hipStream_t s)
{
    Workspace &W = L->ws;
    if (!W.bitmap) return CSP_OK;
    csp_status st = fill_u32(W.occ, 0u, W.occ_words, s);
    if (st != CSP_OK) return st;
    if (L->nnz > 0) {
        k_bm_occ_set<<<blocks_for(L->nnz, 256), 256, 0, s>>>(L->rows, L->cols, L->nnz, W.occ, W.occ_row_words);
        CSP_LAUNCHED("k_bm_occ_set");
    }
    return exclusive_scan_popc(W.occ, W.occ_pref, W.occ_words, W.hist, s);  // ranks of the set bits
}

csp_status restructure_gradient(csp_layer *L, int64_t n_prune, const void *dY, const void *X, int64_t B,
                                uint32_t regrow_bits, hipStream_t s)
{
    Workspace &W = L->ws;
    if (!W.bitmap)
        return set_error(CSP_ERR_INVALID_ARG, "gradient-informed restructure needs the position bitmaps "
                                              "(out * in < 2^32 and bitmaps within 1 GiB)");
    if (n_prune == 0) return CSP_OK;
    if (!W.score) {  // score keys of every padded position, allocated at the first call
        if (hipMalloc((void **)&W.score, 4 * (size_t)W.occ_words * 32) != hipSuccess) {
            (void)hipGetLastError();
            W.score = nullptr;
            return set_error(CSP_ERR_NO_MEMORY, "cannot allocate %zu bytes of regrow scores",
                             4 * (size_t)W.occ_words * 32);
        }
    }
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    if (L->esz == 2) {
        BitmapRun<uint16_t> r{L, n_prune, 0, 0, npos, (uint16_t)regrow_bits, s};
        csp_status st = r.prune(nullptr, 0);
        return st != CSP_OK ? st : r.template regrow_by_gradient<BF16>(dY, X, B);
    }
    BitmapRun<uint32_t> r{L, n_prune, 0, 0, npos, regrow_bits, s};
    csp_status st = r.prune(nullptr, 0);
    return st != CSP_OK ? st : r.template regrow_by_gradient<F32>(dY, X, B);
}

// Candidates restructure_async draws in its one batch: the expected need
// (n_prune over the empty fraction) times 1.2, plus 4096.  Falling short
// (fewer empty, first-seen positions than n_prune) then takes a deviation of
// hundreds of standard deviations: at 8192 x 8192 and 95% sparsity the
// batch's expected surplus is ~65,000 positions against a spread of ~150.
// 0 when the batch would exceed the workspace.
int64_t async_batch(const csp_layer *L, int64_t n_prune)
{
    const Workspace &W = L->ws;
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    const double free_frac = (double)(npos - (uint64_t)(L->nnz - n_prune)) / (double)npos;
    const double want = (double)n_prune / free_frac * 1.2 + 4096.0;
    if (want > (double)W.bm_batch_cap) return 0;
    int64_t M = (int64_t)want;
    if (const char *e = std::getenv("COOSPMM_REGROW_BATCH")) {  // test hook: a smaller batch (may come up short)
        const long long v = std::atoll(e);
        if (v >= 4 && v < M) M = v;
    }
    return M + (4 - M % 4) % 4;  // whole Philox blocks
}

csp_status restructure_bitmap_async(csp_layer *L, int64_t n_prune, uint64_t seed, const uint64_t *step_dev,
                                    uint32_t regrow_bits, hipStream_t s)
{
    const int64_t M = async_batch(L, n_prune);
    if (M == 0)
        return set_error(CSP_ERR_INVALID_ARG, "restructure_async: %lld regrow candidates do not fit one batch "
                                              "(%lld); use restructure", (long long)n_prune,
                         (long long)L->ws.bm_batch_cap);
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    if (L->esz == 2) {
        BitmapRun<uint16_t> r{L, n_prune, seed, 0, npos, (uint16_t)regrow_bits, s};
        r.step_dev = step_dev;
        return r.run_async(M);
    }
    BitmapRun<uint32_t> r{L, n_prune, seed, 0, npos, regrow_bits, s};
    r.step_dev = step_dev;
    return r.run_async(M);
}

csp_status restructure_bitmap(csp_layer *L, int64_t n_prune, uint64_t seed, uint64_t step, uint32_t regrow_bits,
                              hipStream_t s)
{
    const uint64_t npos = (uint64_t)L->out * (uint64_t)L->in;
    if (L->esz == 2) {
        BitmapRun<uint16_t> r{L, n_prune, seed, step, npos, (uint16_t)regrow_bits, s};
        return r.run();
    }
    BitmapRun<uint32_t> r{L, n_prune, seed, step, npos, regrow_bits, s};
    return r.run();
}

}  // namespace csp
