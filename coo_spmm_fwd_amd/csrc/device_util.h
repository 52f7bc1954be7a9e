// device_util.h -- small wave- and block-level building blocks shared by the
// integer passes of the library (scans, compaction ranks).  Private header.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csp {

// Bits of the lanes below this one.
__device__ __forceinline__ uint64_t lanes_below()
{
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan of one uint32 per thread over a block of blockDim.x threads
// (a multiple of 64, at most 1024).  Returns the exclusive prefix; *total gets
// the block sum (all threads).  lds16 holds at least 17 words.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *lds16, uint32_t *total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds16[w] = x;
    __syncthreads();
    if (w == 0) {
        uint32_t t = lane < nw ? lds16[lane] : 0u, s = t;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            uint32_t y = __shfl_up(s, off, 64);
            if (lane >= off) s += y;
        }
        if (lane < nw) lds16[lane] = s - t;
        if (lane == nw - 1) lds16[16] = s;
    }
    __syncthreads();
    uint32_t r = x - v + lds16[w];
    *total = lds16[16];
    __syncthreads();  // lds16 may be reused by the caller
    return r;
}

// Element types of the layer: fp32, and bf16 held as its 16-bit pattern
// (widened exactly by a 16-bit shift; narrowed round-to-nearest-even).
struct F32 {
    using T = float;
    __device__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ static float from_f(float v) { return v; }
};
struct BF16 {
    using T = uint16_t;
    __device__ static float load(const uint16_t *p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
    __device__ static uint16_t from_f(float f)  // round to nearest even
    {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};
// Lanes of the wave whose 8-bit value d equals this lane's, among the lanes
// with `take` set (eight ballots, one per bit).
__device__ __forceinline__ uint64_t lanes_with_same_byte(uint32_t d, bool take)
{
    uint64_t m = __ballot(take);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool on = (d >> bit) & 1u;
        const uint64_t bb = __ballot(on);
        m &= on ? bb : ~bb;
    }
    return m;
}

// a[k] for k < n, else a[0] (the buffer has at least one element).  The
// load is unconditional, so an unrolled loop of them issues every load before
// its first wait instead of branching around each one.
template <typename T>
__device__ __forceinline__ T load_or_first(const T *__restrict__ a, int64_t k, int64_t n)
{
    return a[k < n ? k : 0];
}

// x from lane (lane xor OFF), OFF < 32: DPP quad permutes for 1 and 2,
// ds_swizzle in bit-mask mode (within 32 lanes) for 4, 8 and 16.
template <int OFF>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x)
{
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16, "lane distance");
    if constexpr (OFF == 1) return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false);
    else if constexpr (OFF == 2) return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false);
    else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (OFF << 10));
}

template <int J>
__device__ __forceinline__ uint32_t transpose_step(uint32_t x, uint32_t m, bool upper)
{
    const uint32_t y = xor_lane_u32<J>(x);
    return upper ? (x & ~m) | ((y >> J) & m) : (x & m) | ((y & m) << J);
}

// 32 x 32 bit transpose across each half-wave: on entry lane i (of its 32)
// holds row i (bit k = column k); on exit it holds column i (bit k = row k).
// Five rounds swap the off-diagonal blocks of 16, 8, 4, 2 and 1 bits.
__device__ __forceinline__ uint32_t transpose32(uint32_t x)
{
    const int lane = threadIdx.x & 31;
    x = transpose_step<16>(x, 0x0000FFFFu, lane & 16);
    x = transpose_step<8>(x, 0x00FF00FFu, lane & 8);
    x = transpose_step<4>(x, 0x0F0F0F0Fu, lane & 4);
    x = transpose_step<2>(x, 0x33333333u, lane & 2);
    x = transpose_step<1>(x, 0x55555555u, lane & 1);
    return x;
}

// Position of the n-th (0-based) set bit of w (n < popc(w)).
__device__ __forceinline__ int nth_set_bit(uint32_t w, uint32_t n)
{
    int pos = 0;
#pragma unroll
    for (int half = 16; half >= 1; half >>= 1) {
        const uint32_t low = (uint32_t)__popc(w & ((1u << half) - 1u));
        if (n >= low) {
            n -= low;
            w >>= half;
            pos += half;
        }
    }
    return pos;
}

// Sum over the wave (all lanes get it).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace csp
