// regrow.h -- the magnitude key of the prune order and the counter-based
// stream of regrow candidates, shared by both restructure paths.  Private header.
//
// "Beyond Masked Sparsity: SNACK ..." (Abstract) restructures the connections
// of the truly sparse layer during dynamic sparse training; the order in which
// entries are pruned and the stream regrow positions are drawn from are
// defined here once so that every path yields the same layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csp {

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds over a
// 4 x 64-bit counter with a 2 x 64-bit key; each round multiplies two words
// by fixed odd constants (keeping both halves of the 128-bit products) and
// the key is advanced by two Weyl increments between rounds.
struct Philox4x64 {
    static constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
    static constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull, kWeyl1 = 0xBB67AE8584CAA73Bull;
    // The four words of block b (counter (b, step, 0, 0), key (seed, 0)).
    __device__ static void block(uint64_t seed, uint64_t step, uint64_t b, uint64_t out[4])
    {
        uint64_t x0 = b, x1 = step, x2 = 0, x3 = 0;
        uint64_t key0 = seed, key1 = 0;
#pragma unroll
        for (int r = 0; r < 10; ++r) {
            const uint64_t p0_hi = __umul64hi(kMul0, x0), p0_lo = kMul0 * x0;
            const uint64_t p1_hi = __umul64hi(kMul1, x2), p1_lo = kMul1 * x2;
            const uint64_t y0 = p1_hi ^ x1 ^ key0, y2 = p0_hi ^ x3 ^ key1;
            x0 = y0;
            x1 = p1_lo;
            x2 = y2;
            x3 = p0_lo;
            key0 += kWeyl0;
            key1 += kWeyl1;
        }
        out[0] = x0;
        out[1] = x1;
        out[2] = x2;
        out[3] = x3;
    }
    // Word i of the stream: word (i mod 4) of block (i div 4).
    __device__ static uint64_t word(uint64_t seed, uint64_t step, uint64_t i)
    {
        uint64_t w[4];
        block(seed, step, i >> 2, w);
        return w[i & 3];
    }
};

// Candidate i of the regrow stream: a 64-bit word scaled to a position in
// [0, npos) by the high half of the 128-bit product.
__device__ __forceinline__ uint64_t regrow_position(uint64_t seed, uint64_t step, uint64_t i, uint64_t npos)
{
    return __umul64hi(Philox4x64::word(seed, step, i), npos);
}

// Prune order key: the bit pattern of |v| read as an unsigned integer (so
// +0 and -0 tie and NaN sorts above +inf); ties go by canonical index.
template <typename V>
__device__ inline uint32_t mag_key(V v);
template <>
__device__ inline uint32_t mag_key<uint32_t>(uint32_t v) { return v & 0x7FFFFFFFu; }
template <>
__device__ inline uint32_t mag_key<uint16_t>(uint16_t v) { return (uint32_t)v & 0x7FFFu; }

}  // namespace csp
