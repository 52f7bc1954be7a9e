// spmm.hip -- forward product, input gradient and value gradient of the
// truly sparse COO layer ("Beyond Masked Sparsity: SNACK ...", Abstract:
// the layer computes only its stored connections, forward and backward).
//
//   forward      Y[b,r]  = sum_{k in row r} v_k X[b,col_k]
//   input grad   dX[b,c] = sum_{k in col c} v_k dY[b,row_k]
//   value grad   dW_k    = sum_b dY[b,row_k] X[b,col_k]
//
// Layout.  Dense operands arrive row-major ([B, n]).  For B > 1 each call
// first copies the operand it gathers to a batch-minor layout [chunk][n][ld]
// (ld = batch rounded up to a power of two, at most 64; a batch above 64 is cut
// into chunks of 64), so the B values one stored entry needs form one
// contiguous 4*ld-byte run: one coalesced load instead of B scattered ones.
//
// Work split.  One wavefront runs one task: up to kTaskChunk consecutive
// entries of one segment (a row for the forward pass and the value gradient,
// a column for the input gradient).  A lane holds VW = min(4, ld) batch
// values of one entry, LPE = ld/VW lanes cover an entry, and the wave steps
// through S = 64/LPE entries at a time (see Map).  A pass first loads 256 of
// the task's index/value words with coalesced loads (4 per lane), then hands
// them to the entry slots with ds_bpermute, so a run of the pass's operand
// gathers can be in flight together.  Slots are summed at the end of the task
// with cross-lane adds; per-entry sums over the batch (value gradient) use
// DPP row operations.  At ld <= 4 the forward runs from a packed row list
// whose tasks may hold several whole short rows (packed_task_body: a
// segmented scan over the lanes).  No MFMA: an unstructured gather is not a
// dense contraction; the bound is HBM for the COO stream and L1/L2 for the
// operand gathers (one L2 request per stored entry and gathered table).
#include <cstdlib>

#include <hip/hip_ext.h>

#include "common.h"
#include "device_util.h"

namespace csp {
namespace {



inline int pow2_ld(int64_t B)
{
    int ld = 1;
    while (ld < B && ld < 64) ld <<= 1;
    return ld;
}

__device__ inline int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

template <int CTRL>
__device__ inline float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v from lane (lane xor OFF): DPP for 1 and 2, ds_swizzle (bit-mask mode,
// within 32 lanes) for 4, 8, 16, ds_bpermute for 32.
template <int OFF>
__device__ inline float xor_lane(float v)
{
    if constexpr (OFF == 1) return dpp<0xB1>(v);
    else if constexpr (OFF == 2) return dpp<0x4E>(v);
    else if constexpr (OFF < 32) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (OFF << 10)));
    else return __shfl_xor(v, 32, 64);
}

// Sum over each aligned group of LD lanes; every lane of the group gets it.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes inside a quad, row_half_mirror
// and row_mirror pair the two halves of 8- and 16-lane groups (all lanes of a
// half already agree), ds_swizzle xor-16 and a bpermute xor-32 finish.
template <int LD>
__device__ inline float group_sum(float v)
{
    if constexpr (LD >= 2) v += dpp<0xB1>(v);
    if constexpr (LD >= 4) v += dpp<0x4E>(v);
    if constexpr (LD >= 8) v += dpp<0x141>(v);
    if constexpr (LD >= 16) v += dpp<0x140>(v);
    if constexpr (LD >= 32) v += xor_lane<16>(v);
    if constexpr (LD >= 64) v += xor_lane<32>(v);
    return v;
}

// Sum over the S slots (lanes b, b+LD, b+2LD, ...): xor exchanges keep lane mod LD.
template <int LD>
__device__ inline float slot_sum(float v)
{
    if constexpr (LD <= 1) v += xor_lane<1>(v);
    if constexpr (LD <= 2) v += xor_lane<2>(v);
    if constexpr (LD <= 4) v += xor_lane<4>(v);
    if constexpr (LD <= 8) v += xor_lane<8>(v);
    if constexpr (LD <= 16) v += xor_lane<16>(v);
    if constexpr (LD <= 32) v += xor_lane<32>(v);
    return v;
}

// ------------------------------------------------------- batch-minor copy
// One or two operands [B, n] -> [n][LD] (B <= LD <= 64, pad slots b >= B
// written as zeros, so consumers never mask them).  A workgroup transposes a
// tile of kBmCols columns through LDS: reads go along the operand's rows
// (coalesced, all of a thread's loads in flight together), and the tile's
// output [kBmCols][LD] is one contiguous run (coalesced writes).  The LDS rows
// are LD + 1 elements long, so the column-wise writes spread over the banks.
constexpr int kBmCols = 32;
constexpr int kBmThreads = 256;

template <typename T, int LD>
__global__ __launch_bounds__(kBmThreads) void k_batch_minor(const T *__restrict__ X1, int64_t n1, T *__restrict__ O1,
                                                          const T *__restrict__ X2, int64_t n2, T *__restrict__ O2,
                                                          int64_t B)
{
    constexpr int N = LD * kBmCols;                         // elements of a tile
    constexpr int E = (N + kBmThreads - 1) / kBmThreads;    // per thread
    __shared__ T tile[kBmCols * (LD + 1)];
    const int64_t tiles1 = (n1 + kBmCols - 1) / kBmCols;
    const bool first = blockIdx.x < tiles1;
    const T *__restrict__ X = first ? X1 : X2;
    T *__restrict__ O = first ? O1 : O2;
    const int64_t n = first ? n1 : n2;
    const int64_t c0 = (first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - tiles1) * kBmCols;
    const int cols = n - c0 < kBmCols ? (int)(n - c0) : kBmCols;
    T v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {  // every load of the thread issued before the first LDS store
        const int i = threadIdx.x + e * kBmThreads;
        const int b = i / kBmCols, c = i % kBmCols;
        const bool ok = i < N && b < B && c < cols;
        const T x = X[ok ? (int64_t)b * n + c0 + c : 0];
        v[e] = ok ? x : T(0);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = threadIdx.x + e * kBmThreads;
        if (i < N) tile[(i % kBmCols) * (LD + 1) + i / kBmCols] = v[e];
    }
    __syncthreads();
    T *__restrict__ dst = O + c0 * LD;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = threadIdx.x + e * kBmThreads;
        if (i < cols * LD) dst[i] = tile[(i / LD) * (LD + 1) + i % LD];
    }
}

// ------------------------------------------------------------- epilogues
// What happens to a segment sum before it is stored:
//   kEpiNone      out = sum;
//   kEpiForward   y = sum + bias[seg] (bias optional); pre[b, seg] = y (optional);
//                 out = GELU(y) when gelu is set, else y;
//   kEpiActGrad   out = sum * GELU'(act_in[b, seg]): the input gradient of this
//                 layer times the derivative of the activation whose input was
//                 act_in (the previous layer's pre-activation).
// GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)); GELU'(x) = Phi(x) + x * phi(x).
enum : int { kEpiNone = 0, kEpiForward = 1, kEpiActGrad = 2 };

struct Epi {
    const void *bias = nullptr;    // [n_seg], layer dtype
    void *pre = nullptr;           // [B, n_seg], layer dtype
    const void *act_in = nullptr;  // [B, n_seg], layer dtype
    int gelu = 0;
    // Optional second copy of the output in the batch-minor layout
    // [n_seg][ldT] (slots b < B written), for the next call that gathers
    // from it: spmm_fwd_bm / spmm_bwd_bm.
    void *outT = nullptr;
    int ldT = 0;
};

__device__ inline float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ inline float gelu_grad_f(float x)
{
    return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * expf(-0.5f * x * x);
}

template <int E, class D>
__device__ inline typename D::T finish_out(float acc, int64_t b, int64_t seg, int64_t n_seg, const Epi &ep)
{
    using T = typename D::T;
    if constexpr (E == kEpiNone) {
        return D::from_f(acc);
    } else if constexpr (E == kEpiForward) {
        const float y = acc + (ep.bias ? D::load((const T *)ep.bias, seg) : 0.f);
        if (ep.pre) ((T *)ep.pre)[b * n_seg + seg] = D::from_f(y);
        return D::from_f(ep.gelu ? gelu_f(y) : y);
    } else {
        return D::from_f(acc * gelu_grad_f(D::load((const T *)ep.act_in, b * n_seg + seg)));
    }
}

// Every store of an output value: out[b, seg], and its batch-minor copy when asked.
template <int E, class D>
__device__ __forceinline__ void store_out(typename D::T *__restrict__ out, float acc, int64_t b, int64_t seg,
                                          int64_t n_seg, const Epi &ep)
{
    const typename D::T y = finish_out<E, D>(acc, b, seg, n_seg, ep);
    out[b * n_seg + seg] = y;
    if (ep.outT) reinterpret_cast<typename D::T *>(ep.outT)[seg * ep.ldT + b] = y;
}

// Lane map.  Each lane owns VW consecutive batch values of an entry (one
// 16-byte load when VW = 4), LPE = LD/VW lanes cover one entry, and the
// wave steps through S = 64/LPE entries at a time.  A pass loads 256 of the
// task's index/value words with coalesced loads (4 per lane) and then walks
// them in 64-entry blocks of IT = 64/S steps.  Gathers inside one straight
// run of blocks are all in flight together; an exit test (skip the rest once
// past the end) splits runs, so tests sit only where a run would otherwise
// grow past about 16 gathers.  Entries past the end read index word 0 (always valid) and
// their contribution is zeroed.
template <int LD>
struct Map {
    static constexpr int VW = LD >= 4 ? 4 : LD;
    static constexpr int LPE = LD / VW;
    static constexpr int S = kWave / LPE;
    static constexpr int IT = kWave / S;
    // Exit test before 64-entry block u: every block when a block holds 16 or
    // more gathers (S <= 4), only at the half pass when it holds 4 or 8, never
    // when it holds 2 or fewer.
    static constexpr bool exit_before(int u) { return S <= 4 ? u > 0 : (S < 32 ? u == 2 : false); }
    // Gathers held in registers at once within a block (B = 64 has 16 steps per block).
    static constexpr int G = IT < 8 ? IT : 8;
};

// Element offset of row c of a batch-minor operand: 32-bit unless the
// operand chunk holds 2^30 elements or more.
template <bool kWide>
__device__ inline auto row_off(int32_t c, int ld)
{
    if constexpr (kWide) return (int64_t)c * ld;
    else return (uint32_t)c * (uint32_t)ld;
}
constexpr int kPerLane = 4;
constexpr int kPass = kWave * kPerLane;

template <int VW>
__device__ inline void load_vec(const float *__restrict__ p, float (&x)[VW])
{
    if constexpr (VW == 4) {
        const float4 f = *reinterpret_cast<const float4 *>(p);
        x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    } else if constexpr (VW == 2) {
        const float2 f = *reinterpret_cast<const float2 *>(p);
        x[0] = f.x; x[1] = f.y;
    } else {
        x[0] = p[0];
    }
}
template <int VW>
__device__ inline void load_vec(const uint16_t *__restrict__ p, float (&x)[VW])
{
    if constexpr (VW == 4) {
        const uint2 f = *reinterpret_cast<const uint2 *>(p);
        x[0] = __uint_as_float(f.x << 16); x[1] = __uint_as_float(f.x & 0xFFFF0000u);
        x[2] = __uint_as_float(f.y << 16); x[3] = __uint_as_float(f.y & 0xFFFF0000u);
    } else if constexpr (VW == 2) {
        const uint32_t f = *reinterpret_cast<const uint32_t *>(p);
        x[0] = __uint_as_float(f << 16); x[1] = __uint_as_float(f & 0xFFFF0000u);
    } else {
        x[0] = __uint_as_float((uint32_t)p[0] << 16);
    }
}

// Index word of entry l of a 64-entry block (no exchange needed when S = 64).
template <int S>
__device__ inline int32_t entry_i(int32_t v, int l)
{
    if constexpr (S == kWave) return v;
    else return __builtin_amdgcn_ds_bpermute(l << 2, v);
}
template <int S>
__device__ inline float entry_f(float v, int l)
{
    return __int_as_float(entry_i<S>(__float_as_int(v), l));
}

// Keeps the gathers of the next 64-entry block from being hoisted above an
// exit test (which would put every block's gathers in registers at once).
__device__ inline void block_fence()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i mod 8), each XCD with its own L2.  Renumbering them so that XCD x
// takes one contiguous range of tasks keeps neighbouring segments -- whose
// outputs share cache lines -- on one XCD, so each output line is written
// back whole by one L2 instead of in pieces by several.
// Workgroup b of nb (both counted from a multiple of 8) to its place in the
// XCD-contiguous order.
__device__ __forceinline__ int64_t xcd_index(int64_t b, int64_t nb)
{
    const int64_t x = b & 7, per = nb >> 3, extra = nb & 7;
    return x * per + (x < extra ? x : extra) + (b >> 3);
}
__device__ __forceinline__ int64_t xcd_block() { return xcd_index(blockIdx.x, gridDim.x); }

// Waves per workgroup of the product kernels that run one task per wave
// (k_segment_spmm, k_values_rows, k_gradients).
#ifndef CSP_PRODUCT_WAVES
#define CSP_PRODUCT_WAVES 4
#endif
constexpr int kPW = CSP_PRODUCT_WAVES;

struct Task {
    int32_t seg, kb, n, slot;
};
__device__ inline Task load_task(const int4 *__restrict__ desc, int64_t t)
{
    const int4 d = desc[t];
    return Task{uniform(d.x), uniform(d.y), uniform(d.z) - uniform(d.y), uniform(d.w)};
}

// ------------------------------------------------- segment sums (fwd, dX)
// For one task of a segment: out[b, seg] = sum over its entries e of
// vals[e] * opT[idx[e]][b].  Forward: row tasks over (cols, vals, X).
// Input gradient: column tasks over (rows_by_col, column-ordered value
// copy, dY).  A split segment's task stores its partial sums instead
// (slot >= 0); the fixup launch finishes the segment.
// kStore: 0 = by the task's slot (store the output, or the partial sums of a
// split task), 1 = always the output, 2 = always the partial sums.
template <int LD, class D, bool kWide, int E, int kStore = 0>
__device__ __attribute__((always_inline)) inline void segment_task_body(const Task &T, const int32_t *__restrict__ idx,
                                    const typename D::T *__restrict__ vals, const typename D::T *__restrict__ opT,
                                    int64_t n_op, int64_t n_seg, int64_t B, float *__restrict__ partial,
                                    typename D::T *__restrict__ out, const Epi &ep)
{
    using M = Map<LD>;
    constexpr int VW = M::VW, LPE = M::LPE, S = M::S, IT = M::IT;
    const int lane = threadIdx.x & 63, s = lane / LPE, q = lane % LPE;

    const typename D::T *op = opT + q * VW;
    float acc[VW];
#pragma unroll
    for (int w = 0; w < VW; ++w) acc[w] = 0.f;
    for (int32_t p0 = 0; p0 < T.n; p0 += kPass) {
        const int32_t m = T.n - p0 < kPass ? T.n - p0 : kPass;
        int32_t ci[kPerLane];
        float vv[kPerLane];
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            const int e = u * kWave + lane;
            const bool ok = e < m;
            const int32_t ec = T.kb + p0 + (ok ? e : m - 1);
            const int32_t c = idx[ec];
            const float v = D::load(vals, ec);
            ci[u] = ok ? c : 0;
            vv[u] = ok ? v : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            if (M::exit_before(u)) {
                block_fence();
                if (u * kWave >= m) break;
            }
#pragma unroll
            for (int i0 = 0; i0 < IT; i0 += M::G) {
                if (i0 > 0) block_fence();
                float x[M::G][VW], v[M::G];
#pragma unroll
                for (int j = 0; j < M::G; ++j) {
                    const int l = (i0 + j) * S + s;
                    const int32_t c = entry_i<S>(ci[u], l);
                    v[j] = entry_f<S>(vv[u], l);
                    load_vec<VW>(op + row_off<kWide>(c, LD), x[j]);
                }
                // explicit fused multiply-adds, so that no path that shares
                // this arithmetic depends on the compiler contracting them
                if ((u + 1) * kWave <= m) {
#pragma unroll
                    for (int j = 0; j < M::G; ++j)
#pragma unroll
                        for (int w = 0; w < VW; ++w) acc[w] = __builtin_fmaf(v[j], x[j][w], acc[w]);
                } else {  // block holding the end of the task
#pragma unroll
                    for (int j = 0; j < M::G; ++j) {
                        const bool ok = u * kWave + (i0 + j) * S + s < m;
#pragma unroll
                        for (int w = 0; w < VW; ++w) acc[w] = __builtin_fmaf(v[j], ok ? x[j][w] : 0.f, acc[w]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int w = 0; w < VW; ++w) acc[w] = slot_sum<LPE>(acc[w]);
    if (s == 0) {
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            const int64_t b = q * VW + w;
            if (b >= B) continue;
            if (kStore == 1 || (kStore == 0 && T.slot < 0))
                store_out<E, D>(out, acc[w], b, T.seg, n_seg, ep);
            else
                partial[(int64_t)T.slot * LD + q * VW + w] = acc[w];
        }
    }
}

template <int LD, class D, bool kWide, int E, int kStore = 0>
__device__ __attribute__((always_inline)) inline void segment_task(const int4 *__restrict__ desc, int64_t t, const int32_t *__restrict__ idx,
                                    const typename D::T *__restrict__ vals, const typename D::T *__restrict__ opT,
                                    int64_t n_op, int64_t n_seg, int64_t B, float *__restrict__ partial,
                                    typename D::T *__restrict__ out, const Epi &ep)
{
    segment_task_body<LD, D, kWide, E, kStore>(load_task(desc, t), idx, vals, opT, n_op, n_seg, B, partial, out, ep);
}

// ---------------------------------------------- packed rows (B <= 4)
// One task of whole segments seg .. seg + nseg - 1 (nseg = -slot >= 2),
// holding the entries [kb, kb + n), n <= kPackEntries, of a narrow batch
// (LD <= 4: one entry per lane, its LD batch values in registers).  The wave
// covers the 512-entry window that starts at kb rounded down to a multiple of
// 8; lane l takes its eight consecutive entries with vector loads and gathers
// their operand rows together.  A byte per window entry in LDS marks the
// first entry of each non-empty segment (bit 7) and the last one (segment
// number + 1 in bits 0-6); lane j < nseg sets the marks of segment j.  Each
// lane then adds its entries with fused multiply-adds, restarting at every
// first entry: the sum of a segment that starts and ends in the lane is
// final; the lane's leading part and its trailing sum go through one
// segmented scan over the lanes, which gives each lane the sum of the
// segment's earlier entries (carry).  Final sums are put in LDS by segment
// (over the marks, which are read by then), and lane j finishes segment j:
// epilogue and store, zero for an empty one.  The addition order is fixed by
// the task list, so results are repeatable, but it differs from the
// one-segment task body's.
template <int LD, class D, bool kWide, int E, int NW>
__device__ __attribute__((always_inline)) inline void packed_task_body(const Task &T, const int32_t *__restrict__ seg_ptr,
                                    const int32_t *__restrict__ idx, const typename D::T *__restrict__ vals,
                                    const typename D::T *__restrict__ opT, int64_t n_seg, int64_t B,
                                    typename D::T *__restrict__ out, const Epi &ep)
{
    static_assert(LD <= 4, "one entry per lane");
    constexpr int VW = LD;
    using Tv = typename D::T;
    // Per wave: 64 x 8 mark bytes, later 64 x VW sums (at least 512 bytes).
    __shared__ float pk_w[NW][kWave * (VW < 2 ? 2 : VW)];
    const int lane = threadIdx.x & 63;
    float *res = pk_w[threadIdx.x >> 6];
    uint2 *marks2 = reinterpret_cast<uint2 *>(res);
    uint8_t *marks = reinterpret_cast<uint8_t *>(res);
    const int32_t nseg = -T.slot, kb = T.kb, ke = T.kb + T.n;
    const int32_t a0 = kb & ~7, g0 = a0 + lane * 8;
    // The window's entries, clamped to the first group when the lane's group
    // holds none of the task (every load stays inside the padded entry arrays).
    const bool any = g0 < ke && g0 + 8 > kb;
    const int32_t g = any ? g0 : a0;
    marks2[lane] = make_uint2(0u, 0u);
    const int32_t sb = seg_ptr[T.seg + (lane < nseg ? lane : nseg)];
    const int32_t se = seg_ptr[T.seg + (lane < nseg ? lane + 1 : nseg)];
    int32_t ci[8];
    float vv[8];
    {
        const int4 i0 = *reinterpret_cast<const int4 *>(idx + g), i1 = *reinterpret_cast<const int4 *>(idx + g + 4);
        ci[0] = i0.x; ci[1] = i0.y; ci[2] = i0.z; ci[3] = i0.w;
        ci[4] = i1.x; ci[5] = i1.y; ci[6] = i1.z; ci[7] = i1.w;
        if constexpr (sizeof(Tv) == 4) {
            const float4 v0 = *reinterpret_cast<const float4 *>(vals + g),
                         v1 = *reinterpret_cast<const float4 *>(vals + g + 4);
            vv[0] = v0.x; vv[1] = v0.y; vv[2] = v0.z; vv[3] = v0.w;
            vv[4] = v1.x; vv[5] = v1.y; vv[6] = v1.z; vv[7] = v1.w;
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(vals + g);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vv[2 * k] = __uint_as_float(w4[k] << 16);
                vv[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
            }
        }
    }
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ok[i] = g0 + i >= kb && g0 + i < ke;
        if (!ok[i]) ci[i] = 0;
    }
    float x[8][VW];
#pragma unroll
    for (int i = 0; i < 8; ++i) load_vec<VW>(opT + row_off<kWide>(ci[i], LD), x[i]);
    // marks (the clearing stores above come first in this wave's LDS order)
    if (lane < nseg && se > sb) {
        const int32_t rs = sb - a0, re = se - 1 - a0;
        if (rs == re) {
            marks[rs] = (uint8_t)(0x80 | (lane + 1));
        } else {
            marks[rs] = 0x80;
            marks[re] = (uint8_t)(lane + 1);
        }
    }
    __builtin_amdgcn_wave_barrier();
    const uint2 mk = marks2[lane];
    __builtin_amdgcn_wave_barrier();  // every lane's marks are read before sums overwrite them
    auto put = [&](uint32_t j, const float (&v)[VW]) {
#pragma unroll
        for (int w = 0; w < VW; ++w) res[j * VW + w] = v[w];
    };
    float r[VW], lead[VW];
#pragma unroll
    for (int w = 0; w < VW; ++w) r[w] = lead[w] = 0.f;
    bool seen = false;
    int32_t lead_end = -1;  // segment whose last entry ends the lane's leading part
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t m = ((i < 4 ? mk.x : mk.y) >> (8 * (i & 3))) & 0xFFu;
        if (m & 0x80u) {
            if (!seen) {
#pragma unroll
                for (int w = 0; w < VW; ++w) lead[w] = r[w];
            }
            seen = true;
#pragma unroll
            for (int w = 0; w < VW; ++w) r[w] = 0.f;
        }
#pragma unroll
        for (int w = 0; w < VW; ++w) r[w] = ok[i] ? __builtin_fmaf(vv[i], x[i][w], r[w]) : r[w];
        if (m & 0x7Fu) {
            if (seen) put((m & 0x7Fu) - 1, r);
            else lead_end = (int32_t)(m & 0x7Fu) - 1;
        }
    }
    if (!seen) {
#pragma unroll
        for (int w = 0; w < VW; ++w) lead[w] = r[w];
    }
    // Segmented inclusive scan of the trailing sums r over the lanes: a lane
    // adds the lanes back to the last one that holds a segment start.
    const uint64_t heads = __ballot(seen);
    const uint64_t upto = heads & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
    const int st = upto ? 63 - __builtin_clzll(upto) : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            const float y = __shfl_up(r[w], d, kWave);
            if (lane - d >= st) r[w] += y;
        }
    }
    float carry[VW];  // the segment's sum over the lanes before this one
#pragma unroll
    for (int w = 0; w < VW; ++w) carry[w] = __shfl_up(r[w], 1, kWave);
    if (lead_end >= 0) {
        float f[VW];
#pragma unroll
        for (int w = 0; w < VW; ++w) f[w] = carry[w] + lead[w];
        put((uint32_t)lead_end, f);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < nseg) {
        const bool has = se > sb;
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            const float y = has ? res[lane * VW + w] : 0.f;
            if (w < B) store_out<E, D>(out, y, w, T.seg + lane, n_seg, ep);
        }
    }
    __builtin_amdgcn_wave_barrier();  // sums read before the next task clears the marks
}

// kStore = 1 when the list has no split segments (every task stores its output).
template <int LD, class D, bool kWide, int E, int kStore>
__global__ __launch_bounds__(kPW * kWave) void k_segment_spmm(const int4 *__restrict__ desc, int64_t ntasks,
                                                      const int32_t *__restrict__ seg_ptr,
                                                      const int32_t *__restrict__ idx,
                                                      const typename D::T *__restrict__ vals,
                                                      const typename D::T *__restrict__ opT, int64_t n_op,
                                                      int64_t n_seg, int64_t B,
                                                      float *__restrict__ partial, typename D::T *__restrict__ out,
                                                      Epi ep)
{
    const int64_t t = xcd_block() * kPW + (threadIdx.x >> 6);
    if (t >= ntasks) return;
    const Task T = load_task(desc, t);
    if constexpr (LD <= 4) {
        if (T.slot < -1) {
            packed_task_body<LD, D, kWide, E, kPW>(T, seg_ptr, idx, vals, opT, n_seg, B, out, ep);
            return;
        }
    }
    segment_task_body<LD, D, kWide, E, kStore>(T, idx, vals, opT, n_op, n_seg, B, partial, out, ep);
}

// Segment pass with split segments finished in the kernel (one batch chunk,
// every segment at most kGroupMaxTasks tasks).  The first workgroups take
// the split segments by size class (split_class): a class-c workgroup holds
// 2^c segments of kGroupWaves >> c waves each, so a segment of few tasks does
// not hold a whole 16-wave workgroup.  A segment's waves run its tasks (wave
// j: tasks j, j + waves, ...) and put their sums in LDS; after a barrier one
// thread per (segment, batch index) adds them in task order -- the order the
// fixup launch uses, so results are bitwise those of the split-plus-fixup
// path.  Split segments come first so that long rows start at once.  The
// remaining workgroups take 16 consecutive tasks each and skip the split ones.
constexpr int kGroupWaves = 16;
constexpr int kGroupMaxTasks = 64;

template <int LD, class D, bool kWide, int E>
__global__ __launch_bounds__(kGroupWaves * kWave) void k_segment_grouped(
    const int4 *__restrict__ desc, int64_t ntasks, const int4 *__restrict__ split_cls, int64_t cls_stride,
    int4 ncls, const int32_t *__restrict__ seg_ptr, const int32_t *__restrict__ idx,
    const typename D::T *__restrict__ vals, const typename D::T *__restrict__ opT, int64_t n_op, int64_t n_seg,
    int64_t B, typename D::T *__restrict__ out, Epi ep)
{
    __shared__ float part[kGroupMaxTasks][LD];
    const int wave = threadIdx.x >> 6;
    int64_t g = blockIdx.x;
    const int64_t nc[kSplitClasses] = {ncls.x, ncls.y, ncls.z, ncls.w};
    int c = 0;
    for (; c < kSplitClasses; ++c) {
        const int64_t nwg = (nc[c] + (1 << c) - 1) >> c;
        if (g < nwg) break;
        g -= nwg;
    }
    if (c < kSplitClasses) {
        const int wps = kGroupWaves >> c;  // waves per segment (a class-0 segment may have 64 tasks)
        const int sl = wave / wps, wj = wave % wps;
        const int4 *recs = split_cls + c * cls_stride;
        const int64_t ri = (g << c) + sl;
        if (ri < nc[c]) {
            const int4 r = recs[ri];  // {segment, first task, task count, 0}
            const int32_t first = uniform(r.y), cnt = uniform(r.z);
            // a split task's slot is its task index, so its partial sums land in part[sl * wps + slot - first]
            float *base = &part[sl * wps][0] - (int64_t)first * LD;
            for (int32_t j = wj; j < cnt; j += wps)
                segment_task_body<LD, D, kWide, E, 2>(load_task(desc, first + j), idx, vals, opT, n_op, n_seg, B,
                                                      base, out, ep);
        }
        __syncthreads();
        if (threadIdx.x < (B << c)) {
            const int s2 = (int)(threadIdx.x / B);
            const int64_t b = threadIdx.x - (int64_t)s2 * B, r2 = (g << c) + s2;
            if (r2 < nc[c]) {
                const int4 r = recs[r2];
                float tot = 0.f;
                for (int32_t j = 0; j < r.z; ++j) tot += part[s2 * wps + j][b];
                store_out<E, D>(out, tot, b, r.x, n_seg, ep);
            }
        }
        return;
    }
    const int64_t t = g * kGroupWaves + wave;
    if (t >= ntasks) return;
    const Task T = load_task(desc, t);
    if (T.slot >= 0) return;  // part of a split segment: finished by its own workgroup
    if constexpr (LD <= 4) {
        if (T.slot < -1) {
            packed_task_body<LD, D, kWide, E, kGroupWaves>(T, seg_ptr, idx, vals, opT, n_seg, B, out, ep);
            return;
        }
    }
    segment_task_body<LD, D, kWide, E, 1>(T, idx, vals, opT, n_op, n_seg, B, nullptr, out, ep);
}

// Finish split segments: out[b, seg] = sum over the segment's tasks, in task
// order, of their partial sums.  One thread per (split segment, batch index).
template <class D, int E>
__global__ __launch_bounds__(256) void k_split_fixup(const int4 *__restrict__ split, int64_t nsplit,
                                                     const float *__restrict__ partial, int64_t B, int ld,
                                                     int64_t n_seg, typename D::T *__restrict__ out, Epi ep)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nsplit * B) return;
    const int64_t q = i / B, bg = i - q * B;
    const int4 r = split[q];
    const float *src = partial + (int64_t)r.y * ld + bg;
    const int64_t stride = ld;
    float tot = 0.f;
    int32_t p = 0;
    for (; p + 8 <= r.z; p += 8) {  // eight independent loads in flight, added in task order
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[(p + j) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) tot += v[j];
    }
    for (; p < r.z; ++p) tot += src[p * stride];
    store_out<E, D>(out, tot, bg, r.x, n_seg, ep);
}

// ----------------------------------------------- value gradient, row order
// dW[e] = sum_b dYT[row][b] * XT[col_e][b] over one row task.  Each entry's
// batch sum (VW values per lane, then LPE lanes) is staged in LDS -- every
// lane of the entry's group writes the same value to the same word, so no
// lane test is needed -- and each 64-entry block leaves as one coalesced row
// in canonical order.
// kRowMajorDy: dY is the caller's row-major [B, out] (small-table path, one
// chunk); the entry's batch values then come from B scattered words, padded
// with zeros past B.
template <int LD, class D, bool kWide, int NW = kPW, bool kRowMajorDy = false>
__device__ __attribute__((always_inline)) inline void values_task_body(const Task &T, const int32_t *__restrict__ cols,
                                   const typename D::T *__restrict__ XT, const typename D::T *__restrict__ dYT,
                                   int64_t in, int64_t out, int64_t B, float *__restrict__ dW, bool acc)
{
    using M = Map<LD>;
    constexpr int VW = M::VW, LPE = M::LPE, S = M::S, IT = M::IT;
    __shared__ float stage[NW][kWave];
    const int lane = threadIdx.x & 63, s = lane / LPE, q = lane % LPE;
    float *lds = stage[threadIdx.x >> 6];
    float dy[VW];
    if constexpr (kRowMajorDy) {
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            const int64_t b = q * VW + w;
            const float v = D::load(dYT, (b < B ? b : 0) * out + T.seg);
            dy[w] = b < B ? v : 0.f;
        }
    } else {
        load_vec<VW>(dYT + (int64_t)T.seg * LD + q * VW, dy);
    }
    const typename D::T *xt = XT + q * VW;
    for (int32_t p0 = 0; p0 < T.n; p0 += kPass) {
        const int32_t m = T.n - p0 < kPass ? T.n - p0 : kPass;
        int32_t ci[kPerLane];
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            const int e = u * kWave + lane;
            const int32_t c = cols[T.kb + p0 + (e < m ? e : m - 1)];
            ci[u] = e < m ? c : 0;
        }
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            if (M::exit_before(u)) block_fence();
            if (u * kWave >= m) break;
#pragma unroll
            for (int i0 = 0; i0 < IT; i0 += M::G) {
                if (i0 > 0) block_fence();
                float x[M::G][VW];
#pragma unroll
                for (int j = 0; j < M::G; ++j)
                    load_vec<VW>(xt + row_off<kWide>(entry_i<S>(ci[u], (i0 + j) * S + s), LD), x[j]);
#pragma unroll
                for (int j = 0; j < M::G; ++j) {
                    float p = 0.f;  // fused multiply-adds in batch order
#pragma unroll
                    for (int w = 0; w < VW; ++w) p = __builtin_fmaf(dy[w], x[j][w], p);
                    lds[(i0 + j) * S + s] = group_sum<LPE>(p);
                }
            }
            const float r = lds[lane];
            const int32_t e = p0 + u * kWave + lane;
            if (e < T.n) {
                if (!acc) dW[T.kb + e] = r;
                else dW[T.kb + e] += r;
            }
        }
    }
}

template <int LD, class D, bool kWide>
__device__ __attribute__((always_inline)) inline void values_task(const int4 *__restrict__ desc, int64_t t, const int32_t *__restrict__ cols,
                                   const typename D::T *__restrict__ XT, const typename D::T *__restrict__ dYT,
                                   int64_t in, int64_t out, float *__restrict__ dW, bool acc)
{
    values_task_body<LD, D, kWide>(load_task(desc, t), cols, XT, dYT, in, out, 0, dW, acc);
}

template <int LD, class D, bool kWide>
__global__ __launch_bounds__(kPW * kWave) void k_values_rows(const int4 *__restrict__ desc, int64_t ntasks,
                                                     const int32_t *__restrict__ cols,
                                                     const typename D::T *__restrict__ XT,
                                                     const typename D::T *__restrict__ dYT, int64_t in, int64_t out,
                                                     float *__restrict__ dW, int acc)
{
    const int64_t t = xcd_block() * kPW + (threadIdx.x >> 6);
    if (t >= ntasks) return;
    values_task<LD, D, kWide>(desc, t, cols, XT, dYT, in, out, dW, acc != 0);
}

// ------------------------------------------ value gradient, LDS tiles
// fp32, one batch chunk of width 64 (B of 33..64; the pad slots of the
// batch-minor tables are zero).  The task-list kernel above pulls one 256-byte
// operand row through its CU's vector-memory path per stored entry, and at
// this width that path bounds it.  Here one workgroup of kTileWaves waves
// takes a tile of kTileRows rows x kTileCols columns (Tiles of the row view):
// it copies the tile's operand rows XT[c][0..63] (128 KiB) into LDS once, and
// every entry of the tile reads its row from there.
// A wave runs four rows side by side, one per 16-lane DPP row: lane q holds
// batch values 4q .. 4q + 3 of dY[row] and of each gathered X row.  A row's
// entries in the tile come in windows of 16 (lane q loads entry q of the
// window; the first kTilePF windows of the next four rows are loaded while
// the current ones run), and step t of a window broadcasts entry t's LDS
// offset to the 16 lanes (row_newbcast).  Each lane keeps the 16 partial dot
// products of a window; one transposing reduction over the 16 lanes then
// leaves the sum of entry q in lane q, stored with one coalesced write.
// The partial products are the task kernel's fused multiply-add chains, and
// the reduction adds the same pairs as its 16-lane sum (lanes xor 1, then xor
// 2, then the two quads of each half, then the two halves -- the task kernel
// pairs the quads and halves by mirroring, which meets the same sums because
// they are equal across a quad or half), so the results are bitwise the same.
constexpr int kTileWaves = 16;
constexpr int kTilePF = 3;
static_assert(kTilePF == 3, "the window selections below spell out three prefetched windows");

// Tile (row block rb, column block cb) of a tile kernel's workgroup.  The
// logical tile order runs in panels of kTilePanel row blocks, column block by
// column block within a panel, and xcd_block gives each XCD a contiguous run
// of it: an XCD takes a compact block of tiles (4 row blocks x 8 column blocks
// at 8192 x 8192).  Its rows' entry runs, ~100 bytes per row and tile, then
// share their cache lines only with tiles in the same L2; ordered by column
// block alone (each XCD taking every eighth block) each run's lines were
// fetched once per XCD that needed a piece of them, 2.3 times the entry bytes.
// The price is each operand block filled once per XCD that needs it (8 MiB of
// fills rather than 2 at 8192 x 8192).
constexpr int kTilePanel = 4;
__device__ __forceinline__ void tile_of(int64_t L, int64_t ncb, int64_t nrb, int64_t &rb, int64_t &cb)
{
    const int64_t panel = L / (kTilePanel * ncb), within = L - panel * kTilePanel * ncb;
    const int64_t rows = nrb - panel * kTilePanel < kTilePanel ? nrb - panel * kTilePanel : kTilePanel;
    cb = within / rows;
    rb = panel * kTilePanel + within % rows;
}

// Work of a tile workgroup: its kTileRows segments in groups of four, one
// group per wave at a time (a 16-lane DPP row per segment).  The slots are
// sorted by entry count, most first, and the groups go to the waves on
// demand: wave w starts with group w, then takes the next group from an LDS
// counter as it starts each one, so the longest groups run first and the
// waves end together.  (With eight fixed groups per wave, the waves of a
// tile ended up to ~4 us apart, and the workgroup waits for its last.)  The
// sums do not depend on which wave adds a segment.
// tile_groups_init copies the tile's slot records to LDS (shared by all
// waves, read after the workgroup's barrier) and sets the counter; it returns
// the record of the lane's segment in the wave's first group, read from
// global memory so that its entries can load before the barrier.
__device__ __forceinline__ int2 tile_groups_init(const int2 *__restrict__ tslots, int2 *lds, int *next, int wave, int g)
{
    if (threadIdx.x < kTileRows) lds[threadIdx.x] = tslots[threadIdx.x];
    if (threadIdx.x == 0) *next = kTileWaves;
    return tslots[4 * wave + g];
}

// The wave's next group (kTileRows / 4 or more: none left).
__device__ __forceinline__ int tile_groups_next(int *next, int lane)
{
    int gn = 0;
    if (lane == 0) gn = atomicAdd(next, 1);
    return __builtin_amdgcn_readfirstlane(gn);
}

template <int T>
__device__ __forceinline__ int row_bcast(int v)
{
    return __builtin_amdgcn_mov_dpp(v, 0x150 + T, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Steps T .. T + 3 of a window: four LDS gathers in flight, then their dot products.
template <int T>
__device__ __forceinline__ void tile_dots(const char *tab, int coff, int q16, const float (&dy)[4], float (&p)[16])
{
    const int a0 = row_bcast<T>(coff) + q16, a1 = row_bcast<T + 1>(coff) + q16;
    const int a2 = row_bcast<T + 2>(coff) + q16, a3 = row_bcast<T + 3>(coff) + q16;
    const float4 x0 = *reinterpret_cast<const float4 *>(tab + a0);
    const float4 x1 = *reinterpret_cast<const float4 *>(tab + a1);
    const float4 x2 = *reinterpret_cast<const float4 *>(tab + a2);
    const float4 x3 = *reinterpret_cast<const float4 *>(tab + a3);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    const float4 xs[4] = {x0, x1, x2, x3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = 0.f;  // fused multiply-adds in batch order
        v = __builtin_fmaf(dy[0], xs[i].x, v);
        v = __builtin_fmaf(dy[1], xs[i].y, v);
        v = __builtin_fmaf(dy[2], xs[i].z, v);
        v = __builtin_fmaf(dy[3], xs[i].w, v);
        p[T + i] = v;
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
}

// On exit lane q of each 16-lane row holds the sum over the row's lanes of p[q].
// Each stage keeps the entries whose index bit matches the lane's bit and adds
// the partner lane's partial sums of the same entries.
__device__ __forceinline__ float tile_reduce16(const float (&p)[16], int q)
{
    const bool b0 = q & 1, b1 = q & 2, b2 = q & 4, b3 = q & 8;
    float a[8], b[4], c[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float keep = b0 ? p[2 * k + 1] : p[2 * k], send = b0 ? p[2 * k] : p[2 * k + 1];
        a[k] = keep + dpp_mov<0xB1>(send);  // lane xor 1
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float keep = b1 ? a[2 * k + 1] : a[2 * k], send = b1 ? a[2 * k] : a[2 * k + 1];
        b[k] = keep + dpp_mov<0x4E>(send);  // lane xor 2
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float keep = b2 ? b[2 * k + 1] : b[2 * k], send = b2 ? b[2 * k] : b[2 * k + 1];
        c[k] = keep + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x1F | (4 << 10)));  // xor 4
    }
    const float keep = b3 ? c[1] : c[0], send = b3 ? c[0] : c[1];
    return keep + dpp_mov<0x128>(send);  // row_ror 8: lane xor 8 within the 16
}

// The LDS table of a tile kernel's workgroup: the block's operand rows, then a
// row of zeros (read by the segment sums' steps past a segment's entries).
constexpr int kTileTab = (kTileCols + 1) * 16;

// One workgroup's tile (rb, cb) of the value gradient, in three phases:
// start (slot records to LDS, the operand fill's loads and the wave's first
// group's loads put in flight), fill (the operand rows to LDS; the caller then
// syncs the workgroup) and run (the groups on demand).  A caller may run
// other work between start and fill: the loads stay in flight.
struct ValuesTile {
    static constexpr int FILL = kTileCols * 16 / (kTileWaves * kWave);  // 16-byte pieces per thread
    const int32_t *cols;
    const float *dYT;
    float *dW;
    int64_t out, c0, r0, ncols;
    int acc, lane, q, g, q16;
    int2 *lslot;
    int *next;
    float4 fl[FILL];
    int cbeg, cn;
    int ci[kTilePF];
    float4 cdy;

    __device__ __forceinline__ void fetch(int2 sl, int &beg, int &n, int (&ii)[kTilePF], float4 &dy) const
    {
        beg = sl.x;
        n = sl.y & 0xFFFF;
        const int64_t r = r0 + (sl.y >> 16);
        dy = reinterpret_cast<const float4 *>(dYT)[(r < out ? r : 0) * 16 + q];
#pragma unroll
        for (int j = 0; j < kTilePF; ++j) {
            const int e = 16 * j + q;
            ii[j] = cols[e < n ? beg + e : 0];
        }
    }

    __device__ __forceinline__ void start(int64_t rb, int64_t cb, const int2 *__restrict__ slots, int64_t ncb,
                                          const int32_t *__restrict__ cols_, const float *__restrict__ XT,
                                          const float *__restrict__ dYT_, int64_t in, int64_t out_,
                                          float *__restrict__ dW_, int acc_, int2 *lslot_, int *next_)
    {
        cols = cols_, dYT = dYT_, dW = dW_, out = out_, acc = acc_, lslot = lslot_, next = next_;
        const int64_t tile = rb * ncb + cb;
        c0 = cb * kTileCols, r0 = rb * kTileRows;
        const int wave = threadIdx.x >> 6;
        lane = threadIdx.x & 63, q = lane & 15, g = lane >> 4, q16 = q * 16;
        // Groups of four rows on demand (tile_groups): this lane's row of the wave's first group.
        const int2 first = tile_groups_init(slots + tile * kTileRows, lslot, next, wave, g);
        ncols = in - c0 < kTileCols ? in - c0 : kTileCols;
        const float4 *x4 = reinterpret_cast<const float4 *>(XT);
#pragma unroll
        for (int j = 0; j < FILL; ++j) {  // every fill load in flight before the first LDS store
            const int i = threadIdx.x + kTileWaves * kWave * j, c = i >> 4;
            fl[j] = x4[(c0 + (c < ncols ? c : 0)) * 16 + (i & 15)];
        }
        fetch(first, cbeg, cn, ci, cdy);
    }

    __device__ __forceinline__ void fill(float4 *tab) const
    {
#pragma unroll
        for (int j = 0; j < FILL; ++j) {
            const int i = threadIdx.x + kTileWaves * kWave * j;
            tab[i] = (i >> 4) < ncols ? fl[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    __device__ __forceinline__ void run(const float4 *tab)
    {
        const char *base = reinterpret_cast<const char *>(tab);
        int nbeg = 0, nn = 0;
        int ni[kTilePF] = {};
        float4 ndy = make_float4(0.f, 0.f, 0.f, 0.f);
        for (;;) {
            const int gn = tile_groups_next(next, lane);
            const bool more = gn < kTileRows / 4;
            if (more) fetch(lslot[4 * gn + g], nbeg, nn, ni, ndy);
            const int nmax = max(max(__builtin_amdgcn_readlane(cn, 0), __builtin_amdgcn_readlane(cn, 16)),
                                 max(__builtin_amdgcn_readlane(cn, 32), __builtin_amdgcn_readlane(cn, 48)));
            const float dy[4] = {cdy.x, cdy.y, cdy.z, cdy.w};
            for (int k = 0; k < nmax; k += 16) {
                const int e = k + q;
                int c;
                if (k < 16 * kTilePF) {
                    const int j = k >> 4;
                    c = j == 0 ? ci[0] : (j == 1 ? ci[1] : ci[2]);
                } else {  // a row with more than 16 * kTilePF entries in the tile
                    c = cols[e < cn ? cbeg + e : 0];
                }
                const uint32_t rel = (uint32_t)((int64_t)c - c0);
                const int coff = e < cn && rel < (uint32_t)kTileCols ? (int)rel * 256 : 0;
                float p[16];
                tile_dots<0>(base, coff, q16, dy, p);
                if (k + 4 < nmax) tile_dots<4>(base, coff, q16, dy, p);
                else p[4] = p[5] = p[6] = p[7] = 0.f;
                if (k + 8 < nmax) tile_dots<8>(base, coff, q16, dy, p);
                else p[8] = p[9] = p[10] = p[11] = 0.f;
                if (k + 12 < nmax) tile_dots<12>(base, coff, q16, dy, p);
                else p[12] = p[13] = p[14] = p[15] = 0.f;
                const float r = tile_reduce16(p, q);
                if (e < cn) {
                    if (!acc) dW[cbeg + e] = r;
                    else dW[cbeg + e] += r;
                }
            }
            if (!more) break;
            cbeg = nbeg;
            cn = nn;
            cdy = ndy;
            ci[0] = ni[0];  // kTilePF == 3 (static_assert at its definition)
            ci[1] = ni[1];
            ci[2] = ni[2];
        }
    }
};

__global__ __launch_bounds__(kTileWaves * kWave) void k_values_tiles(const int2 *__restrict__ slots,
                                                                     int64_t ncb, const int32_t *__restrict__ cols,
                                                                     const float *__restrict__ XT,
                                                                     const float *__restrict__ dYT, int64_t in,
                                                                     int64_t out, float *__restrict__ dW, int acc)
{
    __shared__ float4 tab[kTileTab];
    __shared__ int2 lslot[kTileRows];
    __shared__ int next;
    int64_t rb, cb;
    tile_of(xcd_block(), ncb, gridDim.x / ncb, rb, cb);
    ValuesTile V;
    V.start(rb, cb, slots, ncb, cols, XT, dYT, in, out, dW, acc, lslot, &next);
    V.fill(tab);
    __syncthreads();
    V.run(tab);
}

// ------------------------------------------- segment sums, LDS tiles
// fp32, batch chunks of width 64: the same tiles for the forward (row view:
// segments are rows, entries their columns, operand X) and the input gradient
// (column view: segments are columns, entries their rows in the transposed
// order with the column-ordered values, operand dY).  The workgroup of a tile
// stages the operand rows of its kTileCols column block in LDS and adds, for
// each of its segments, the entries that fall in the block; the result is one
// partial sum per (column block, segment, batch slot) in P[cb][seg][64]
// (float4 stores of 256-byte runs), and k_tile_reduce adds the column blocks
// in order.  A wave runs four segments side by side as in k_values_tiles: lane
// q of a 16-lane row accumulates batch slots 4q .. 4q + 3 of its segment, one
// fused multiply-add chain per slot in entry order.
template <int T>
__device__ __forceinline__ float row_bcast_f(float v)
{
    return __int_as_float(row_bcast<T>(__float_as_int(v)));
}

template <int T>
__device__ __forceinline__ void tile_steps(const char *tab, int coff, float v, int q16, float (&acc)[4])
{
    const int a0 = row_bcast<T>(coff) + q16, a1 = row_bcast<T + 1>(coff) + q16;
    const int a2 = row_bcast<T + 2>(coff) + q16, a3 = row_bcast<T + 3>(coff) + q16;
    const float4 x0 = *reinterpret_cast<const float4 *>(tab + a0);
    const float4 x1 = *reinterpret_cast<const float4 *>(tab + a1);
    const float4 x2 = *reinterpret_cast<const float4 *>(tab + a2);
    const float4 x3 = *reinterpret_cast<const float4 *>(tab + a3);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    const float v0 = row_bcast_f<T>(v), v1 = row_bcast_f<T + 1>(v), v2 = row_bcast_f<T + 2>(v),
                v3 = row_bcast_f<T + 3>(v);
    acc[0] = __builtin_fmaf(v0, x0.x, acc[0]); acc[1] = __builtin_fmaf(v0, x0.y, acc[1]);
    acc[2] = __builtin_fmaf(v0, x0.z, acc[2]); acc[3] = __builtin_fmaf(v0, x0.w, acc[3]);
    acc[0] = __builtin_fmaf(v1, x1.x, acc[0]); acc[1] = __builtin_fmaf(v1, x1.y, acc[1]);
    acc[2] = __builtin_fmaf(v1, x1.z, acc[2]); acc[3] = __builtin_fmaf(v1, x1.w, acc[3]);
    acc[0] = __builtin_fmaf(v2, x2.x, acc[0]); acc[1] = __builtin_fmaf(v2, x2.y, acc[1]);
    acc[2] = __builtin_fmaf(v2, x2.z, acc[2]); acc[3] = __builtin_fmaf(v2, x2.w, acc[3]);
    acc[0] = __builtin_fmaf(v3, x3.x, acc[0]); acc[1] = __builtin_fmaf(v3, x3.y, acc[1]);
    acc[2] = __builtin_fmaf(v3, x3.z, acc[2]); acc[3] = __builtin_fmaf(v3, x3.w, acc[3]);
    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
}

// One workgroup's tile (rb, cb) of a segment-sum pass, in the phases of
// ValuesTile (start, fill, run); fill also writes the zero row.
struct SegmentTile {
    static constexpr int FILL = kTileCols * 16 / (kTileWaves * kWave);
    const int32_t *idx;
    const float *vals;
    float *P;
    int64_t cb, n_seg, c0, r0, ncols;
    int lane, q, g, q16;
    int2 *lslot;
    int *next;
    float4 fl[FILL];
    int cbeg, cn, crow;
    int ci[kTilePF];
    float cv[kTilePF];

    __device__ __forceinline__ void fetch(int2 sl, int &beg, int &n, int &row, int (&ii)[kTilePF],
                                          float (&vv)[kTilePF]) const
    {
        beg = sl.x;
        n = sl.y & 0xFFFF;
        row = sl.y >> 16;
#pragma unroll
        for (int j = 0; j < kTilePF; ++j) {
            const int e = 16 * j + q;
            const int p = e < n ? beg + e : 0;
            ii[j] = idx[p];
            vv[j] = vals[p];
        }
    }

    __device__ __forceinline__ void start(int64_t rb, int64_t cb_, const int2 *__restrict__ slots, int64_t ncb,
                                          const int32_t *__restrict__ idx_, const float *__restrict__ vals_,
                                          const float *__restrict__ opT, int64_t n_op, int64_t n_seg_,
                                          float *__restrict__ P_, int2 *lslot_, int *next_)
    {
        idx = idx_, vals = vals_, P = P_, cb = cb_, n_seg = n_seg_, lslot = lslot_, next = next_;
        const int64_t tile = rb * ncb + cb;
        c0 = cb * kTileCols, r0 = rb * kTileRows;
        const int wave = threadIdx.x >> 6;
        lane = threadIdx.x & 63, q = lane & 15, g = lane >> 4, q16 = q * 16;
        // Groups of four segments on demand (tile_groups): this lane's segment of the wave's first group.
        const int2 first = tile_groups_init(slots + tile * kTileRows, lslot, next, wave, g);
        ncols = n_op - c0 < kTileCols ? n_op - c0 : kTileCols;
        const float4 *o4 = reinterpret_cast<const float4 *>(opT);
#pragma unroll
        for (int j = 0; j < FILL; ++j) {
            const int i = threadIdx.x + kTileWaves * kWave * j, c = i >> 4;
            fl[j] = o4[(c0 + (c < ncols ? c : 0)) * 16 + (i & 15)];
        }
        fetch(first, cbeg, cn, crow, ci, cv);
    }

    __device__ __forceinline__ void fill(float4 *tab) const
    {
#pragma unroll
        for (int j = 0; j < FILL; ++j) {
            const int i = threadIdx.x + kTileWaves * kWave * j;
            tab[i] = (i >> 4) < ncols ? fl[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (threadIdx.x < 16) tab[kTileCols * 16 + threadIdx.x] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    __device__ __forceinline__ void run(const float4 *tab)
    {
        const char *base = reinterpret_cast<const char *>(tab);
        int nbeg = 0, nn = 0, nrow = 0;
        int ni[kTilePF] = {};
        float nv[kTilePF] = {};
        for (;;) {
            const int gn = tile_groups_next(next, lane);
            const bool more = gn < kTileRows / 4;
            if (more) fetch(lslot[4 * gn + g], nbeg, nn, nrow, ni, nv);
            const int nmax = max(max(__builtin_amdgcn_readlane(cn, 0), __builtin_amdgcn_readlane(cn, 16)),
                                 max(__builtin_amdgcn_readlane(cn, 32), __builtin_amdgcn_readlane(cn, 48)));
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k < nmax; k += 16) {
                const int e = k + q;
                int c;
                float v;
                if (k < 16 * kTilePF) {
                    const int j = k >> 4;
                    c = j == 0 ? ci[0] : (j == 1 ? ci[1] : ci[2]);
                    v = j == 0 ? cv[0] : (j == 1 ? cv[1] : cv[2]);
                } else {  // a segment with more than 16 * kTilePF entries in the tile
                    const int p = e < cn ? cbeg + e : 0;
                    c = idx[p];
                    v = vals[p];
                }
                const uint32_t rel = (uint32_t)((int64_t)c - c0);
                const bool ok = e < cn && rel < (uint32_t)kTileCols;
                // steps past the segment's entries read the zero row (an inf or NaN in
                // the block's first row must not reach the sum through a zero weight)
                const int coff = ok ? (int)rel * 256 : kTileCols * 256;
                const float vv = ok ? v : 0.f;
                tile_steps<0>(base, coff, vv, q16, acc);
                if (k + 4 >= nmax) continue;
                tile_steps<4>(base, coff, vv, q16, acc);
                if (k + 8 >= nmax) continue;
                tile_steps<8>(base, coff, vv, q16, acc);
                if (k + 12 >= nmax) continue;
                tile_steps<12>(base, coff, vv, q16, acc);
            }
            // The next group's prefetched loads are taken over before this
            // group's store is issued: stores count in the same in-order
            // memory counter as loads, so taking them over after the store
            // would wait for the store's completion at every group.
            const int64_t r = r0 + crow;
            const float4 res = make_float4(acc[0], acc[1], acc[2], acc[3]);
            if (more) {
                cbeg = nbeg;
                cn = nn;
                crow = nrow;
                ci[0] = ni[0], ci[1] = ni[1], ci[2] = ni[2];
                cv[0] = nv[0], cv[1] = nv[1], cv[2] = nv[2];
            }
            __builtin_amdgcn_sched_barrier(0);
            if (r < n_seg) reinterpret_cast<float4 *>(P)[(cb * n_seg + r) * 16 + q] = res;
            if (!more) break;
        }
    }
};

__global__ __launch_bounds__(kTileWaves * kWave) void k_segment_tiles(const int2 *__restrict__ slots,
                                                                      int64_t ncb, const int32_t *__restrict__ idx,
                                                                      const float *__restrict__ vals,
                                                                      const float *__restrict__ opT, int64_t n_op,
                                                                      int64_t n_seg, float *__restrict__ P)
{
    __shared__ float4 tab[kTileTab];
    __shared__ int2 lslot[kTileRows];
    __shared__ int next;
    int64_t rb, cb;
    tile_of(xcd_block(), ncb, gridDim.x / ncb, rb, cb);
    SegmentTile S;
    S.start(rb, cb, slots, ncb, idx, vals, opT, n_op, n_seg, P, lslot, &next);
    S.fill(tab);
    __syncthreads();
    S.run(tab);
}

// Both gradients' tile passes in one launch, one tile of each per workgroup
// (the two views have the same number of tiles): the input gradient's tile
// (column view over dY, partial sums into P), then the value gradient's (row
// view).  The value-gradient tile's start -- its slot records, operand fill
// and first groups' loads -- is issued before the input-gradient tile runs,
// so its loads arrive meanwhile instead of after it; the workgroup then
// fills the LDS table again and runs it.  The arithmetic is the two
// separate kernels'.
__global__ __launch_bounds__(kTileWaves * kWave) void k_gradient_tiles(
    const int2 *__restrict__ cslots, int64_t cncb, int64_t cnrb, const int32_t *__restrict__ rows_by_col,
    const float *__restrict__ vals_c, const int2 *__restrict__ rslots, int64_t rncb, int64_t rnrb,
    const int32_t *__restrict__ cols, const float *__restrict__ XT, const float *__restrict__ dYT, int64_t in,
    int64_t out, float *__restrict__ P, float *__restrict__ dW, int acc)
{
    __shared__ float4 tab[kTileTab];
    __shared__ int2 sslot[kTileRows], vslot[kTileRows];
    __shared__ int snext, vnext;
    const int64_t t = xcd_block();
    int64_t rb, cb;
    SegmentTile S;
    tile_of(t, cncb, cnrb, rb, cb);
    S.start(rb, cb, cslots, cncb, rows_by_col, vals_c, dYT, out, in, P, sslot, &snext);
    ValuesTile V;
    tile_of(t, rncb, rnrb, rb, cb);
    V.start(rb, cb, rslots, rncb, cols, XT, dYT, in, out, dW, acc, vslot, &vnext);
    S.fill(tab);
    __syncthreads();
    S.run(tab);
    __syncthreads();  // every wave is done with the input gradient's table
    V.fill(tab);
    __syncthreads();
    V.run(tab);
}

// out[b, seg] = epilogue(sum over column blocks cb, in order, of P[cb][seg][b]).
// A block takes kReduceSegs segments: thread t adds the float4 t (and t + 256)
// of their 64-slot runs over the column blocks (eight loads in flight), the
// sums are turned around in LDS, and each batch row leaves as one run of
// kReduceSegs values.
constexpr int kReduceSegs = 32;
template <int E>
__global__ __launch_bounds__(256) void k_tile_reduce(const float *__restrict__ P, int64_t ncb, int64_t n_seg, int64_t B,
                                                     float *__restrict__ out, Epi ep)
{
    constexpr int PER = kReduceSegs * 16 / 256;  // float4 per thread
    __shared__ float t[kReduceSegs][65];
    const int64_t s0 = (int64_t)blockIdx.x * kReduceSegs;
    const int nsg = (int)(n_seg - s0 < kReduceSegs ? n_seg - s0 : kReduceSegs);
    const float4 *src = reinterpret_cast<const float4 *>(P) + s0 * 16;
    const int64_t stride = n_seg * 16;
    float4 a[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) a[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    int64_t cb = 0;
    for (; cb + 8 <= ncb; cb += 8) {
        float4 x[8][PER];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int f = threadIdx.x + 256 * i;
                x[j][i] = (f >> 4) < nsg ? src[(cb + j) * stride + f] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                a[i].x += x[j][i].x; a[i].y += x[j][i].y; a[i].z += x[j][i].z; a[i].w += x[j][i].w;
            }
    }
    for (; cb < ncb; ++cb)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = threadIdx.x + 256 * i;
            const float4 x = (f >> 4) < nsg ? src[cb * stride + f] : make_float4(0.f, 0.f, 0.f, 0.f);
            a[i].x += x.x; a[i].y += x.y; a[i].z += x.z; a[i].w += x.w;
        }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int f = threadIdx.x + 256 * i, sl = f >> 4, b0 = (f & 15) * 4;
        t[sl][b0] = a[i].x; t[sl][b0 + 1] = a[i].y; t[sl][b0 + 2] = a[i].z; t[sl][b0 + 3] = a[i].w;
    }
    __syncthreads();
    const int sl = threadIdx.x % kReduceSegs;
#pragma unroll
    for (int i = 0; i < 64 * kReduceSegs / 256; ++i) {
        const int64_t b = threadIdx.x / kReduceSegs + (256 / kReduceSegs) * i;
        if (b < B && sl < nsg) store_out<E, F32>(out, t[sl][b], b, s0 + sl, n_seg, ep);
    }
}

// --------------------------------------------------- both gradients
// The two gradients are independent; one launch runs both so that their
// latency chains overlap: even/odd blocks alternate between input-gradient
// column tasks and value-gradient row tasks, the longer list's surplus
// blocks come last.
template <int LD, class D, bool kWide, int E, int kStore>
__global__ __launch_bounds__(kPW * kWave) void k_gradients(const int4 *__restrict__ col_desc, int64_t ncol_tasks,
                                                   const int4 *__restrict__ row_desc, int64_t nrow_tasks,
                                                   const int32_t *__restrict__ rows_by_col,
                                                   const typename D::T *__restrict__ vals_c,
                                                   const int32_t *__restrict__ cols,
                                                   const typename D::T *__restrict__ XT,
                                                   const typename D::T *__restrict__ dYT, int64_t in, int64_t out,
                                                   int64_t B, float *__restrict__ partial,
                                                   typename D::T *__restrict__ dX, float *__restrict__ dW, Epi ep,
                                                   int acc)
{
    const int64_t ncb = (ncol_tasks + kPW - 1) / kPW, nrb = (nrow_tasks + kPW - 1) / kPW;
    const int64_t m = ncb < nrb ? ncb : nrb;
    // Plain dispatch order here: with the two task kinds interleaved, renumbering by XCD
    // measured 6% more HBM traffic for this kernel (and 6% less for the single-kind ones).
    const int64_t bid = blockIdx.x;
    bool col;
    int64_t blk;
    if (bid < 2 * m) {
        col = (bid & 1) == 0;
        blk = bid >> 1;
    } else {
        col = ncb > nrb;
        blk = m + (bid - 2 * m);
    }
    const int64_t t = blk * kPW + (threadIdx.x >> 6);
    if (col) {
        if (t < ncol_tasks)
            segment_task<LD, D, kWide, E, kStore>(col_desc, t, rows_by_col, vals_c, dYT, out, in, B, partial, dX, ep);
    } else if (t < nrow_tasks) {
        values_task<LD, D, kWide>(row_desc, t, cols, XT, dYT, in, out, dW, acc != 0);
    }
}

// --------------------------------------------- small operand tables in LDS
// When the operand a pass gathers from is small (2 <= B <= 64, so one chunk,
// and n * ld * esz <= kLdsTableBytes), each workgroup of kLdsWaves waves
// first copies it from the caller's row-major [B, n] into LDS in the
// batch-minor layout [n][ld] (pad slots zero), then runs its tasks against
// that copy.  No copy launch precedes the product, and the gathers become LDS
// reads instead of one L2 line request each.  The tasks are the same code as
// with the global table, so results are bitwise the same.  The gain is the
// copy launch: with B = 1 there is none to save, and with tables above 64 KiB
// the per-workgroup fill and the lower occupancy cost more than the L2
// gathers they replace (measured on 16384-column layers at B = 1 and 4).
constexpr int kLdsWaves = 16;
constexpr int kLdsThreads = kLdsWaves * kWave;
constexpr size_t kLdsTableBytes = size_t(64) << 10;

// tab[c * LD + b] = src[b * n + c] for b < B, 0 for B <= b < LD.  Loads are
// unconditional (row 0 stands in for pad rows) so they all issue together.
template <int LD, class D>
__device__ inline void fill_table(const typename D::T *__restrict__ src, int64_t n, int64_t B, typename D::T *tab)
{
    using T = typename D::T;
    if constexpr (LD == 1) {
        // A plain copy: 16-byte pieces when the source is 16-byte aligned.
        int64_t head = 0;
        if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
            constexpr int P = 16 / (int)sizeof(T);
            const int64_t np = n / P;
            const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
            uint4 *t4 = reinterpret_cast<uint4 *>(tab);
            for (int64_t i = threadIdx.x; i < np; i += kLdsThreads) t4[i] = s4[i];
            head = np * P;
        }
        for (int64_t i = head + threadIdx.x; i < n; i += kLdsThreads) tab[i] = src[i];
    } else {
        constexpr int W = LD * (int)sizeof(T) / 4;  // 32-bit words per column
        for (int64_t c = threadIdx.x; c < n; c += kLdsThreads) {
            uint32_t w[W];
            if constexpr (sizeof(T) == 4) {
#pragma unroll
                for (int b = 0; b < LD; ++b) {
                    const uint32_t x = __float_as_uint(src[(b < B ? b : 0) * n + c]);
                    w[b] = b < B ? x : 0u;
                }
            } else {
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const int b0 = 2 * k, b1 = 2 * k + 1;
                    const uint32_t x0 = src[(b0 < B ? b0 : 0) * n + c], x1 = src[(b1 < B ? b1 : 0) * n + c];
                    w[k] = (b0 < B ? x0 : 0u) | ((b1 < B ? x1 : 0u) << 16);
                }
            }
            uint32_t *dst = reinterpret_cast<uint32_t *>(tab + c * LD);
            if constexpr (W % 4 == 0) {
#pragma unroll
                for (int k = 0; k < W / 4; ++k)
                    reinterpret_cast<uint4 *>(dst)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
            } else if constexpr (W == 2) {
                *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
            } else {
                dst[0] = w[0];
            }
        }
    }
}

// Forward (row tasks over X) or input gradient (column tasks over dY) with
// the operand table in LDS.  The grid is persistent (about two workgroups per
// CU), so each workgroup fills the table once.  It then takes every grid-th
// split segment (its 16 waves run the segment's tasks and add their sums in
// LDS in task order, as in k_segment_grouped), and after those each wave
// takes every (16 * grid)-th task, skipping split ones.  Fixed strides need
// no shared counter: one counter on one address, taken by every workgroup,
// costs more in serialised atomics than the balance it buys.  Which wave runs
// a task does not change its arithmetic, so the outputs are bitwise those of
// the global-table kernels.
template <int LD, class D, int E>
__global__ __launch_bounds__(kLdsThreads) void k_segment_lds(const int4 *__restrict__ desc, int64_t ntasks,
                                                             const int4 *__restrict__ split, int64_t nsplit,
                                                             const int32_t *__restrict__ seg_ptr,
                                                             const int32_t *__restrict__ idx,
                                                             const typename D::T *__restrict__ vals,
                                                             const typename D::T *__restrict__ op, int64_t n_op,
                                                             int64_t n_seg, int64_t B, typename D::T *__restrict__ out,
                                                             Epi ep)
{
    extern __shared__ __align__(16) unsigned char lds_table[];
    __shared__ float part[kGroupMaxTasks][LD];
    auto *tab = reinterpret_cast<typename D::T *>(lds_table);
    const int wave = threadIdx.x >> 6;
    fill_table<LD, D>(op, n_op, B, tab);
    __syncthreads();
    // Split segments first, a whole workgroup each.
    for (int64_t g = blockIdx.x; g < nsplit; g += gridDim.x) {
        const int4 r = split[g];  // {segment, first task, task count, 0}
        const int32_t seg = uniform(r.x), first = uniform(r.y), cnt = uniform(r.z);
        float *base = &part[0][0] - (int64_t)first * LD;  // slot = task index
        for (int32_t j = wave; j < cnt; j += kLdsWaves)
            segment_task_body<LD, D, false, E, 2>(load_task(desc, first + j), idx, vals, tab, n_op, n_seg, B, base,
                                                  out, ep);
        __syncthreads();
        if (threadIdx.x < B) {
            const int64_t b = threadIdx.x;
            float tot = 0.f;
            for (int32_t j = 0; j < cnt; ++j) tot += part[j][b];
            store_out<E, D>(out, tot, b, seg, n_seg, ep);
        }
        __syncthreads();  // partial sums consumed before the next group writes them
    }
    // Then the unsplit tasks, each wave on its own stride (no barrier: a
    // wave that drew short tasks moves on at once).  The next descriptor is
    // loaded before the current task runs, so its latency hides behind it.
    const int64_t nw = (int64_t)gridDim.x * kLdsWaves;
    int64_t t = (int64_t)blockIdx.x * kLdsWaves + wave;
    if (t >= ntasks) return;
    int4 d = desc[t];
    for (; t < ntasks; t += nw) {
        const int4 dn = desc[t + nw < ntasks ? t + nw : t];
        const Task T{uniform(d.x), uniform(d.y), uniform(d.z) - uniform(d.y), uniform(d.w)};
        if constexpr (LD <= 4) {
            if (T.slot < -1) packed_task_body<LD, D, false, E, kLdsWaves>(T, seg_ptr, idx, vals, tab, n_seg, B, out, ep);
        }
        if (T.slot == -1) segment_task_body<LD, D, false, E, 1>(T, idx, vals, tab, n_op, n_seg, B, nullptr, out, ep);
        d = dn;
    }
}

// Both gradients: workgroups alternate between input-gradient column tasks
// (table: dY) and value-gradient row tasks (table: X), as in k_gradients.
template <int LD, class D, int E, int kStore>
__global__ __launch_bounds__(kLdsThreads) void k_gradients_lds(const int4 *__restrict__ col_desc, int64_t ncol_tasks,
                                                               const int4 *__restrict__ row_desc, int64_t nrow_tasks,
                                                               const int32_t *__restrict__ rows_by_col,
                                                               const typename D::T *__restrict__ vals_c,
                                                               const int32_t *__restrict__ cols,
                                                               const typename D::T *__restrict__ X,
                                                               const typename D::T *__restrict__ dY, int64_t in,
                                                               int64_t out, int64_t B, float *__restrict__ partial,
                                                               typename D::T *__restrict__ dX, float *__restrict__ dW,
                                                               Epi ep, int acc)
{
    extern __shared__ __align__(16) unsigned char lds_table[];
    auto *tab = reinterpret_cast<typename D::T *>(lds_table);
    const int64_t ncb = (ncol_tasks + kLdsWaves - 1) / kLdsWaves, nrb = (nrow_tasks + kLdsWaves - 1) / kLdsWaves;
    const int64_t m = ncb < nrb ? ncb : nrb;
    const int64_t bid = blockIdx.x;
    bool col;
    int64_t blk;
    if (bid < 2 * m) {
        col = (bid & 1) == 0;
        blk = bid >> 1;
    } else {
        col = ncb > nrb;
        blk = m + (bid - 2 * m);
    }
    const int64_t t = blk * kLdsWaves + (threadIdx.x >> 6);
    const bool has = t < (col ? ncol_tasks : nrow_tasks);
    const Task T = load_task(col ? col_desc : row_desc, has ? t : 0);
    if (col) fill_table<LD, D>(dY, out, B, tab);
    else fill_table<LD, D>(X, in, B, tab);
    __syncthreads();
    if (!has) return;
    if (col) segment_task_body<LD, D, false, E, kStore>(T, rows_by_col, vals_c, tab, out, in, B, partial, dX, ep);
    else values_task_body<LD, D, false, kLdsWaves, true>(T, cols, tab, dY, in, out, B, dW, acc != 0);
}

// ------------------------------------------------------------ host side
// Batch-minor copies of up to two operands (B == 1 needs none: [1, n] already is).
csp_status batch_minor(csp_layer *L, int64_t B, const void *X1, int64_t n1, void *O1, const void *X2, int64_t n2,
                       void *O2, hipStream_t s)
{
    if (B == 1) return CSP_OK;
    if (!X1) {  // only the second operand
        X1 = X2, n1 = n2, O1 = O2;
        X2 = nullptr;
    }
    if (!X1) return CSP_OK;
    const int ld = pow2_ld(B);
    if (!X2) n2 = 0;
    const int64_t blocks = ceil_div(n1, kBmCols) + ceil_div(n2, kBmCols);
#define CSP_BMT(T, LDV)                                                                                        \
    k_batch_minor<T, LDV><<<(unsigned)blocks, kBmThreads, 0, s>>>((const T *)X1, n1, (T *)O1, (const T *)X2, n2, \
                                                                  (T *)O2, B)
#define CSP_BM(LDV)                               \
    if (L->esz == 4) CSP_BMT(float, LDV);         \
    else CSP_BMT(uint16_t, LDV)
    switch (ld) {
    case 2: CSP_BM(2); break;
    case 4: CSP_BM(4); break;
    case 8: CSP_BM(8); break;
    case 16: CSP_BM(16); break;
    case 32: CSP_BM(32); break;
    default: CSP_BM(64); break;
    }
#undef CSP_BM
#undef CSP_BMT
    CSP_LAUNCHED("k_batch_minor");
    return CSP_OK;
}

// Launch of a product call's main kernel.  When the caller has asked for the
// next main kernel to be timed (sparse_layer_time_next), the launch goes
// through hipExtLaunchKernel with the request's events attached to the
// dispatch itself, so they carry the kernel's own start and end times; mark
// says which of the two this launch carries (a pass of two kernels puts the
// start on the first and the end on the second).
enum : int { kTimeStart = 1, kTimeStop = 2, kTimeBoth = 3 };

template <typename... KArgs, typename... Args>
inline void launch_main(csp_layer *L, int mark, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                        hipStream_t s, Args... args)
{
    hipEvent_t a = (mark & kTimeStart) ? L->time_before : nullptr;
    hipEvent_t b = (mark & kTimeStop) ? L->time_after : nullptr;
    if (a || b)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, a, b, 0u, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
    if (mark & kTimeStop) L->time_before = L->time_after = nullptr;
}

#define CSP_LD_SWITCH_W(ld, MACRO, W) \
    switch (ld) {                     \
    case 1: MACRO(1, W); break;       \
    case 2: MACRO(2, W); break;       \
    case 4: MACRO(4, W); break;       \
    case 8: MACRO(8, W); break;       \
    case 16: MACRO(16, W); break;     \
    case 32: MACRO(32, W); break;     \
    default: MACRO(64, W); break;     \
    }
#define CSP_LD_SWITCH(ld, wide, MACRO)             \
    do {                                           \
        if (wide) CSP_LD_SWITCH_W(ld, MACRO, true) \
        else CSP_LD_SWITCH_W(ld, MACRO, false)     \
    } while (0)

// Operands whose chunk holds 2^30 or more elements need 64-bit offsets.
inline bool wide_operand(int64_t n, int ld) { return n * (int64_t)ld >= (int64_t(1) << 30); }

template <class D, int E>
csp_status split_fixup(csp_layer *L, const TaskList &TL, int64_t B, int64_t n_seg, void *out, const Epi &ep,
                       hipStream_t s, float *partial = nullptr)
{
    if (TL.nsplit == 0) return CSP_OK;
    const int ld = pow2_ld(B);
    k_split_fixup<D, E><<<(unsigned)ceil_div(TL.nsplit * B, 256), 256, 0, s>>>(
        TL.split, TL.nsplit, partial ? partial : L->act.partial, B, ld, n_seg, (typename D::T *)out, ep);
    CSP_LAUNCHED("k_split_fixup");
    return CSP_OK;
}

// Small-table paths (see fill_table) for a pass that gathers from an operand
// of n columns, 2 <= B <= 64.  At B = 1 the operand is a single row that
// stays cached near the CUs anyway and no copy launch is saved, so filling
// tables costs more than it returns (measured: 1 us slower on a 16384-column
// bf16 layer).  The segment pass (k_segment_lds) also needs every segment to
// be at most kGroupMaxTasks tasks; its segments are at most n long.
// COOSPMM_LDS_TABLES=0 forces the global-table paths (A/B runs and tests).
inline bool lds_tables_enabled()
{
    const char *e = std::getenv("COOSPMM_LDS_TABLES");
    return !(e && e[0] == '0');
}
inline bool lds_table_fits(const csp_layer *L, int64_t B, int64_t n)
{
    if (B < 2 || B > 64 || (size_t)n * (size_t)pow2_ld(B) * (size_t)L->esz > kLdsTableBytes) return false;
    return lds_tables_enabled();
}
inline bool lds_segment_fits(const csp_layer *L, int64_t B, int64_t n)
{
    return ceil_div(n, kTaskChunk) <= kGroupMaxTasks && lds_table_fits(L, B, n);
}

// The kernel's dynamic LDS limit is raised to the table size once per kernel
// (the value-gradient stage array is static LDS on top of it).
template <auto Kern>
csp_status allow_lds(size_t)
{
    static bool done = false;
    if (!done) {
        CSP_HIP(hipFuncSetAttribute(reinterpret_cast<const void *>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)kLdsTableBytes));
        done = true;
    }
    return CSP_OK;
}

#define CSP_LD_SWITCH_LDS(ld, MACRO) \
    switch (ld) {                    \
    case 1: MACRO(1); break;         \
    case 2: MACRO(2); break;         \
    case 4: MACRO(4); break;         \
    case 8: MACRO(8); break;         \
    case 16: MACRO(16); break;       \
    case 32: MACRO(32); break;       \
    default: MACRO(64); break;       \
    }

// One segment pass (forward: rows over X; input gradient: columns over dY)
// from a row-major operand through an LDS table: a persistent grid of at
// most two workgroups per CU (one when the batch is wider than 8 and the
// kernel's registers allow no more), each taking every grid-th group of
// tasks.  Split segments finish inside the pass, so no fixup launch follows.
template <class D, int E>
csp_status segment_lds_dispatch(csp_layer *L, const TaskList &TL, const int32_t *seg_ptr, const int32_t *idx,
                                const void *vals, const void *op, int64_t n_op, int64_t n_seg, int64_t B, void *out,
                                const Epi &ep, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    const int64_t ngroups = TL.nsplit + ceil_div(TL.count, kLdsWaves);
    const int64_t cap = (int64_t)L->act.cus * (ld <= 8 ? 2 : 1);
    const unsigned grid = (unsigned)(ngroups < cap ? ngroups : cap);
    if (grid == 0) return CSP_OK;
    const size_t lds = (size_t)n_op * ld * L->esz;
    csp_status st = CSP_OK;
#define CSP_SEGL(LDV)                                                                                              \
    if ((st = allow_lds<k_segment_lds<LDV, D, E>>(lds)) == CSP_OK)                                                \
        launch_main(L, kTimeBoth, k_segment_lds<LDV, D, E>, grid, kLdsThreads, lds, s, TL.desc, TL.count, TL.split, \
                    TL.nsplit, seg_ptr, idx, (const T *)vals, (const T *)op, n_op, n_seg, B, (T *)out, ep)
    CSP_LD_SWITCH_LDS(ld, CSP_SEGL);
#undef CSP_SEGL
    if (st != CSP_OK) return st;
    CSP_LAUNCHED("k_segment_lds");
    return CSP_OK;
}

// Both gradients (or only the value gradient when with_dx is false) from
// row-major X and dY through LDS tables.
template <class D, int E>
csp_status gradients_lds_dispatch(csp_layer *L, const void *X, const void *dY, int64_t B, void *dX, float *dW,
                                  bool with_dx, bool acc, const Epi &ep, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    const TaskList &CT = L->col_tasks, &RT = L->row_tasks;
    const int64_t ncol = with_dx ? CT.count : 0;
    const int64_t nrow = L->nnz > 0 ? RT.count : 0;  // no value-gradient work for an empty layer
    const unsigned grid = (unsigned)(ceil_div(ncol, kLdsWaves) + ceil_div(nrow, kLdsWaves));
    if (grid == 0) return CSP_OK;
    // the value gradient alone needs only the X table
    const int64_t n_tab = with_dx && L->out > L->in ? L->out : L->in;
    const size_t lds = (size_t)n_tab * ld * L->esz;
    csp_status st = CSP_OK;
    const bool ks = CT.nsplit == 0 || !with_dx;
#define CSP_GRADL_ARGS                                                                                   \
    CT.desc, ncol, RT.desc, nrow, L->rows_by_col, (const T *)L->vals_c, L->cols, (const T *)X, (const T *)dY, \
        L->in, L->out, B, L->act.partial, (T *)dX, dW, ep, (int)acc
#define CSP_GRADL(LDV)                                                                                       \
    if (ks) {                                                                                                \
        if ((st = allow_lds<k_gradients_lds<LDV, D, E, 1>>(lds)) == CSP_OK)                                 \
            launch_main(L, kTimeBoth, k_gradients_lds<LDV, D, E, 1>, grid, kLdsThreads, lds, s, CSP_GRADL_ARGS);                   \
    } else if ((st = allow_lds<k_gradients_lds<LDV, D, E, 0>>(lds)) == CSP_OK) {                             \
        launch_main(L, kTimeBoth, k_gradients_lds<LDV, D, E, 0>, grid, kLdsThreads, lds, s, CSP_GRADL_ARGS);                       \
    }
    CSP_LD_SWITCH_LDS(ld, CSP_GRADL);
#undef CSP_GRADL
#undef CSP_GRADL_ARGS
    if (st != CSP_OK) return st;
    CSP_LAUNCHED("k_gradients_lds");
    return with_dx ? split_fixup<D, E>(L, CT, B, L->in, dX, ep, s) : CSP_OK;
}

// The forward's task list: the packed one when a lane holds one entry
// (B <= 4), where a task of one short row would leave most lanes idle, and
// the packed list is current (see csp_layer::narrow_seen).  COOSPMM_PACKED=0
// keeps the plain list.
inline const TaskList &fwd_tasks(csp_layer *L, int64_t B)
{
    if (pow2_ld(B) > 4) return L->row_tasks;
    L->narrow_seen = true;  // later restructures rebuild the packed list
    const char *e = std::getenv("COOSPMM_PACKED");
    return (e && e[0] == '0') || !L->packed_valid ? L->row_tasks : L->row_packed;
}

// Split segments finished inside the segment pass (k_segment_grouped) when
// there are any, B <= 8, and no segment can have more than kGroupMaxTasks
// tasks (its length is at most max_len, the other dimension).  Up to B = 8
// the kernel keeps 8 waves per SIMD, two 16-wave workgroups per CU; at larger
// widths its registers leave one workgroup per CU and the split-plus-fixup
// path was faster (B = 64: 56 against 43 us for the pass).
// COOSPMM_GROUPED_SPLITS=0 keeps the split-plus-fixup path.
inline bool grouped_splits(const TaskList &TL, int64_t B, int64_t max_len, int64_t n_op)
{
    if (TL.nsplit == 0 || B > 8 || ceil_div(max_len, kTaskChunk) > kGroupMaxTasks) return false;
    if (wide_operand(n_op, pow2_ld(B))) return false;
    const char *e = std::getenv("COOSPMM_GROUPED_SPLITS");
    return !(e && e[0] == '0');
}

template <class D, int E>
csp_status grouped_dispatch(csp_layer *L, const TaskList &TL, const int32_t *seg_ptr, const int32_t *idx,
                            const void *vals, const void *opT, int64_t n_op, int64_t n_seg, int64_t B, void *out,
                            const Epi &ep, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    int64_t nsw = 0;  // workgroups of the split segments, by class
    for (int c = 0; c < kSplitClasses; ++c) nsw += (TL.ncls[c] + (1 << c) - 1) >> c;
    const unsigned grid = (unsigned)(nsw + ceil_div(TL.count, kGroupWaves));
    const int4 ncls = make_int4((int)TL.ncls[0], (int)TL.ncls[1], (int)TL.ncls[2], (int)TL.ncls[3]);
    const int64_t stride = TL.nsplit > 0 ? n_seg : 0;
#define CSP_GRP(LDV)                                                                                            \
    launch_main(L, kTimeBoth, k_segment_grouped<LDV, D, false, E>, grid, kGroupWaves * kWave, 0, s,                                    \
        TL.desc, TL.count, TL.split_cls, stride, ncls, seg_ptr, idx, (const T *)vals, (const T *)opT, n_op, n_seg, B, (T *)out, ep)
    CSP_LD_SWITCH_LDS(ld, CSP_GRP);
#undef CSP_GRP
    CSP_LAUNCHED("k_segment_grouped");
    return CSP_OK;
}

template <class D, int E>
csp_status fwd_dispatch(csp_layer *L, const void *XT, int64_t B, void *Y, const Epi &ep, hipStream_t s,
                        float *partial)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    const TaskList &TL = fwd_tasks(L, B);
    if (grouped_splits(TL, B, L->in, L->in))
        return grouped_dispatch<D, E>(L, TL, L->row_ptr, L->cols, L->vals, XT, L->in, L->out, B, Y, ep, s);
    const unsigned grid = (unsigned)ceil_div(TL.count, kPW);
    const bool ks = TL.nsplit == 0;
#define CSP_FWD_ARGS \
    TL.desc, TL.count, L->row_ptr, L->cols, (const T *)L->vals, (const T *)XT, L->in, L->out, B, partial, (T *)Y, ep
#define CSP_FWD(LDV, W)                                                             \
    if (ks) launch_main(L, kTimeBoth, k_segment_spmm<LDV, D, W, E, 1>, grid, kPW * kWave, 0, s, CSP_FWD_ARGS);    \
    else launch_main(L, kTimeBoth, k_segment_spmm<LDV, D, W, E, 0>, grid, kPW * kWave, 0, s, CSP_FWD_ARGS)
    CSP_LD_SWITCH(ld, wide_operand(L->in, ld), CSP_FWD);
#undef CSP_FWD
#undef CSP_FWD_ARGS
    CSP_LAUNCHED("k_segment_spmm (forward)");
    return split_fixup<D, E>(L, TL, B, L->out, Y, ep, s, partial);
}

template <class D, int E>
csp_status bwd_input_dispatch(csp_layer *L, const void *dYT, int64_t B, void *dX, const Epi &ep, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    const TaskList &TL = L->col_tasks;
    if (grouped_splits(TL, B, L->out, L->out))
        return grouped_dispatch<D, E>(L, TL, L->col_ptr, L->rows_by_col, L->vals_c, dYT, L->out, L->in, B, dX, ep, s);
    const unsigned grid = (unsigned)ceil_div(TL.count, kPW);
    const bool ks = TL.nsplit == 0;
#define CSP_DX_ARGS                                                                                                 \
    TL.desc, TL.count, L->col_ptr, L->rows_by_col, (const T *)L->vals_c, (const T *)dYT, L->out, L->in, B, L->act.partial, \
        (T *)dX, ep
#define CSP_DX(LDV, W)                                                            \
    if (ks) launch_main(L, kTimeBoth, k_segment_spmm<LDV, D, W, E, 1>, grid, kPW * kWave, 0, s, CSP_DX_ARGS);   \
    else launch_main(L, kTimeBoth, k_segment_spmm<LDV, D, W, E, 0>, grid, kPW * kWave, 0, s, CSP_DX_ARGS)
    CSP_LD_SWITCH(ld, wide_operand(L->out, ld), CSP_DX);
#undef CSP_DX
#undef CSP_DX_ARGS
    CSP_LAUNCHED("k_segment_spmm (input gradient)");
    return split_fixup<D, E>(L, TL, B, L->in, dX, ep, s);
}

// The tile kernel for the value gradient: fp32 layers that have tiles, a
// batch chunk of width 64, and at least one tile per compute unit (fewer
// would leave CUs idle; the task list then spreads better).  The variable
// COOSPMM_VALUE_TILES=0 turns it off (a test hook: the results are the same).
inline bool value_tiles_usable(const csp_layer *L, int ld)
{
    if (!L->tile_partial || ld != 64) return false;
    const char *e = std::getenv("COOSPMM_VALUE_TILES");
    return !(e && e[0] == '0');
}

csp_status launch_value_tiles(csp_layer *L, int mark, const float *XT, const float *dYT, float *dW, bool acc,
                              hipStream_t s)
{
    const Tiles &T = L->tiles_r;
    launch_main(L, mark, k_values_tiles, dim3((unsigned)(T.nrb * T.ncb)), dim3(kTileWaves * kWave), 0u, s, T.slots,
                T.ncb, L->cols, XT, dYT, L->in, L->out, dW, (int)acc);
    CSP_LAUNCHED("k_values_tiles");
    return CSP_OK;
}

// The tile kernels for the segment sums (forward: row view; input gradient:
// column view) at batch chunks of width 64.  The sums are added in another
// order than the task kernel's (per tile, then the tiles in column-block
// order), so they agree with it to rounding, not bitwise.  The variable
// COOSPMM_SEGMENT_TILES=0 turns them off (a test hook).
inline bool segment_tiles_usable(const csp_layer *L, int ld)
{
    if (!L->tile_partial || ld != 64) return false;
    const char *e = std::getenv("COOSPMM_SEGMENT_TILES");
    return !(e && e[0] == '0');
}

template <int E>
csp_status launch_segment_tiles(csp_layer *L, int mark, const Tiles &T, const int32_t *idx, const float *vals,
                                const float *opT, int64_t B, float *out, const Epi &ep, hipStream_t s)
{
    launch_main(L, mark & kTimeStart, k_segment_tiles, dim3((unsigned)(T.nrb * T.ncb)), dim3(kTileWaves * kWave), 0u,
                s, T.slots, T.ncb, idx, vals, opT, T.nop, T.nseg, L->tile_partial);
    CSP_LAUNCHED("k_segment_tiles");
    launch_main(L, mark & kTimeStop, k_tile_reduce<E>, dim3((unsigned)ceil_div(T.nseg, kReduceSegs)), dim3(256), 0u, s,
                (const float *)L->tile_partial, T.ncb, T.nseg, B, out, ep);
    CSP_LAUNCHED("k_tile_reduce");
    return CSP_OK;
}

// Both gradients' tiles in one launch (k_gradient_tiles), then the input
// gradient's reduce.  The variable COOSPMM_FUSED_TILES=0 launches the two
// tile kernels separately instead (a test hook; the results are the same bits).
inline bool gradient_tiles_fused()
{
    const char *e = std::getenv("COOSPMM_FUSED_TILES");
    return !(e && e[0] == '0');
}

template <int E>
csp_status launch_gradient_tiles(csp_layer *L, const float *XT, const float *dYT, int64_t B, float *dX, float *dW,
                                 bool acc, const Epi &ep, hipStream_t s)
{
    const Tiles &C = L->tiles_c, &R = L->tiles_r;
    launch_main(L, kTimeStart, k_gradient_tiles, dim3((unsigned)(C.nrb * C.ncb)), dim3(kTileWaves * kWave), 0u, s,
                C.slots, C.ncb, C.nrb, L->rows_by_col, (const float *)L->vals_c, R.slots, R.ncb, R.nrb, L->cols, XT,
                dYT, L->in, L->out, L->tile_partial, dW, (int)acc);
    CSP_LAUNCHED("k_gradient_tiles");
    launch_main(L, kTimeStop, k_tile_reduce<E>, dim3((unsigned)ceil_div(C.nseg, kReduceSegs)), dim3(256), 0u, s,
                (const float *)L->tile_partial, C.ncb, C.nseg, B, dX, ep);
    CSP_LAUNCHED("k_tile_reduce");
    return CSP_OK;
}

template <class D>
csp_status bwd_values_dispatch(csp_layer *L, const void *XT, const void *dYT, int64_t B, float *dW, bool acc,
                               hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    if constexpr (sizeof(T) == 4)
        if (value_tiles_usable(L, ld))
            return launch_value_tiles(L, kTimeBoth, (const float *)XT, (const float *)dYT, dW, acc, s);
    const csp_status st = tasks_ready(L, s);
    if (st != CSP_OK) return st;
    const TaskList &TL = L->row_tasks;
    const unsigned grid = (unsigned)ceil_div(TL.count, kPW);
#define CSP_DW(LDV, W)                                                                                            \
    launch_main(L, kTimeBoth, k_values_rows<LDV, D, W>, grid, kPW * kWave, 0, s, TL.desc, TL.count, L->cols, (const T *)XT, (const T *)dYT, L->in, \
                                                  L->out, dW, (int)acc)
    CSP_LD_SWITCH(ld, wide_operand(L->in > L->out ? L->in : L->out, ld), CSP_DW);
#undef CSP_DW
    CSP_LAUNCHED("k_values_rows");
    return CSP_OK;
}

template <class D, int E>
csp_status bwd_dispatch(csp_layer *L, const void *XT, const void *dYT, int64_t B, void *dX, float *dW, bool acc,
                        const Epi &ep, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    const int64_t table_bytes = (int64_t)L->esz * ld * (L->in + L->out);
    bool both_tiled = false;  // then the task counts are not read (beyond being nonzero with entries)
    if constexpr (sizeof(T) == 4)
        both_tiled = table_bytes > (int64_t(2) << 20) && L->nnz > 0 && segment_tiles_usable(L, ld) &&
                     value_tiles_usable(L, ld);
    if (!both_tiled) {
        const csp_status st = tasks_ready(L, s);
        if (st != CSP_OK) return st;
    }
    const TaskList &CT = L->col_tasks, &RT = L->row_tasks;
    const int64_t nrow = L->nnz > 0 ? RT.count : 0;  // no value-gradient work for an empty layer
    const bool wide = wide_operand(L->in > L->out ? L->in : L->out, ld);
    // One launch for both gradients overlaps their latency chains, but the two
    // interleaved passes gather from both batch-minor tables at once; when the
    // tables together exceed about half an XCD's 4 MiB L2 they evict each
    // other, so the passes run as two launches instead.
    if (table_bytes > (int64_t(2) << 20)) {
        const unsigned gx = (unsigned)ceil_div(CT.count, kPW), gw = (unsigned)ceil_div(nrow, kPW);
        const int m1 = gw > 0 ? kTimeStart : kTimeBoth;  // the value-gradient kernel carries the end
        const bool ks = CT.nsplit == 0;
        bool dx_tiled = false, dw_tiled = false;
        if constexpr (sizeof(T) == 4) {
            dx_tiled = segment_tiles_usable(L, ld);
            dw_tiled = gw > 0 && value_tiles_usable(L, ld);
            if (dx_tiled && dw_tiled && gradient_tiles_fused() &&
                L->tiles_c.nrb * L->tiles_c.ncb == L->tiles_r.nrb * L->tiles_r.ncb)
                return launch_gradient_tiles<E>(L, (const float *)XT, (const float *)dYT, B, (float *)dX, dW, acc, ep,
                                                 s);
        }
        if (dx_tiled) {
            const csp_status st = launch_segment_tiles<E>(L, m1, L->tiles_c, L->rows_by_col, (const float *)L->vals_c,
                                                          (const float *)dYT, B, (float *)dX, ep, s);
            if (st != CSP_OK) return st;
        } else {
#define CSP_DX2_ARGS                                                                                                \
    CT.desc, CT.count, L->col_ptr, L->rows_by_col, (const T *)L->vals_c, (const T *)dYT, L->out, L->in, B, L->act.partial, \
        (T *)dX, ep
#define CSP_DX2(LDV, W)                                                         \
    if (ks) launch_main(L, m1, k_segment_spmm<LDV, D, W, E, 1>, gx, kPW * kWave, 0, s, CSP_DX2_ARGS);  \
    else launch_main(L, m1, k_segment_spmm<LDV, D, W, E, 0>, gx, kPW * kWave, 0, s, CSP_DX2_ARGS)
        CSP_LD_SWITCH(ld, wide, CSP_DX2);
#undef CSP_DX2
#undef CSP_DX2_ARGS
        CSP_LAUNCHED("k_segment_spmm (input gradient)");
        }
        if (dw_tiled) {
            const csp_status st = launch_value_tiles(L, kTimeStop, (const float *)XT, (const float *)dYT, dW, acc, s);
            if (st != CSP_OK) return st;
        } else if (gw > 0) {
#define CSP_DW2(LDV, W)                                                                                           \
    launch_main(L, kTimeStop, k_values_rows<LDV, D, W>, gw, kPW * kWave, 0, s, RT.desc, nrow, L->cols, (const T *)XT, (const T *)dYT, L->in, L->out, \
                                                dW, (int)acc)
            CSP_LD_SWITCH(ld, wide, CSP_DW2);
#undef CSP_DW2
            CSP_LAUNCHED("k_values_rows");
        }
        return dx_tiled ? CSP_OK : split_fixup<D, E>(L, CT, B, L->in, dX, ep, s);
    }
    const unsigned grid = (unsigned)(ceil_div(CT.count, kPW) + ceil_div(nrow, kPW));
    const bool ks = CT.nsplit == 0;
#define CSP_BOTH_ARGS                                                                                            \
    CT.desc, CT.count, RT.desc, nrow, L->rows_by_col, (const T *)L->vals_c, L->cols, (const T *)XT, (const T *)dYT, \
        L->in, L->out, B, L->act.partial, (T *)dX, dW, ep, (int)acc
#define CSP_BOTH(LDV, W)                                                        \
    if (ks) launch_main(L, kTimeBoth, k_gradients<LDV, D, W, E, 1>, grid, kPW * kWave, 0, s, CSP_BOTH_ARGS);  \
    else launch_main(L, kTimeBoth, k_gradients<LDV, D, W, E, 0>, grid, kPW * kWave, 0, s, CSP_BOTH_ARGS)
    CSP_LD_SWITCH(ld, wide, CSP_BOTH);
#undef CSP_BOTH
#undef CSP_BOTH_ARGS
    CSP_LAUNCHED("k_gradients");
    return split_fixup<D, E>(L, CT, B, L->in, dX, ep, s);
}

Epi make_epi(const FwdEpilogue *fe)
{
    Epi ep;
    if (fe) {
        ep.bias = fe->bias;
        ep.pre = fe->pre;
        ep.gelu = fe->gelu;
    }
    return ep;
}

csp_status fwd_slice(csp_layer *L, const void *X, int64_t B, void *Y, const FwdEpilogue *fe, hipStream_t s,
                     const FwdWork &wk, const BmIO &io)
{
    csp_status st = CSP_OK;
    Epi ep = make_epi(fe);
    ep.outT = io.outt;
    ep.ldT = pow2_ld(B);
    if (lds_segment_fits(L, B, L->in)) {
        if ((st = tasks_ready(L, s)) != CSP_OK) return st;
        const TaskList &RT = fwd_tasks(L, B);
        const int32_t *rp = L->row_ptr, *ci = L->cols;
        const void *v = L->vals;
        if (L->dtype == CSP_BF16)
            return fe ? segment_lds_dispatch<BF16, kEpiForward>(L, RT, rp, ci, v, X, L->in, L->out, B, Y, ep, s)
                      : segment_lds_dispatch<BF16, kEpiNone>(L, RT, rp, ci, v, X, L->in, L->out, B, Y, ep, s);
        return fe ? segment_lds_dispatch<F32, kEpiForward>(L, RT, rp, ci, v, X, L->in, L->out, B, Y, ep, s)
                  : segment_lds_dispatch<F32, kEpiNone>(L, RT, rp, ci, v, X, L->in, L->out, B, Y, ep, s);
    }
    const bool tiled = L->dtype == CSP_F32 && wk.operand == L->act.a && segment_tiles_usable(L, pow2_ld(B));
    if (!tiled && (st = tasks_ready(L, s)) != CSP_OK) return st;
    st = batch_minor(L, B, io.xt ? nullptr : X, L->in, wk.operand, nullptr, 0, nullptr, s);
    if (st != CSP_OK) return st;
    const void *xt = io.xt ? io.xt : (B == 1 ? X : wk.operand);
    float *pt = wk.partial;
    // LDS tiles need the layer's own partial-sum buffer (not a caller's workspace)
    if (tiled) {
        const Tiles &T = L->tiles_r;
        const float *v = (const float *)L->vals, *x = (const float *)xt;
        return fe ? launch_segment_tiles<kEpiForward>(L, kTimeBoth, T, L->cols, v, x, B, (float *)Y, ep, s)
                  : launch_segment_tiles<kEpiNone>(L, kTimeBoth, T, L->cols, v, x, B, (float *)Y, ep, s);
    }
    if (L->dtype == CSP_BF16)
        return fe ? fwd_dispatch<BF16, kEpiForward>(L, xt, B, Y, ep, s, pt) : fwd_dispatch<BF16, kEpiNone>(L, xt, B, Y, ep, s, pt);
    return fe ? fwd_dispatch<F32, kEpiForward>(L, xt, B, Y, ep, s, pt) : fwd_dispatch<F32, kEpiNone>(L, xt, B, Y, ep, s, pt);
}

// Workspace one forward slice of B rows needs: the batch-minor operand copy
// (none for B = 1 or the LDS-table path) and the split tasks' partial sums
// (none without split rows or when they finish inside the pass).
void fwd_slice_work(csp_layer *L, int64_t B, size_t *operand_bytes, size_t *partial_bytes)
{
    *operand_bytes = *partial_bytes = 0;
    if (lds_segment_fits(L, B, L->in)) return;
    const int ld = pow2_ld(B);
    if (B > 1) *operand_bytes = (size_t)L->esz * ld * (size_t)L->in;
    const TaskList &TL = fwd_tasks(L, B);
    if (TL.nsplit > 0 && !grouped_splits(TL, B, L->in, L->in)) *partial_bytes = sizeof(float) * ld * (size_t)TL.count;
}

csp_status bwd_input_slice(csp_layer *L, const void *dY, int64_t B, void *dX, const void *act_in, hipStream_t s,
                           const BmIO &io)
{
    csp_status st = CSP_OK;
    Epi ep;
    ep.act_in = act_in;
    ep.outT = io.outt;
    ep.ldT = pow2_ld(B);
    if (lds_segment_fits(L, B, L->out)) {
        if ((st = tasks_ready(L, s)) != CSP_OK) return st;
        const TaskList &CT = L->col_tasks;
        const int32_t *cp = L->col_ptr, *rc = L->rows_by_col;
        const void *vc = L->vals_c;
        if (L->dtype == CSP_BF16)
            return act_in ? segment_lds_dispatch<BF16, kEpiActGrad>(L, CT, cp, rc, vc, dY, L->out, L->in, B, dX, ep, s)
                          : segment_lds_dispatch<BF16, kEpiNone>(L, CT, cp, rc, vc, dY, L->out, L->in, B, dX, ep, s);
        return act_in ? segment_lds_dispatch<F32, kEpiActGrad>(L, CT, cp, rc, vc, dY, L->out, L->in, B, dX, ep, s)
                      : segment_lds_dispatch<F32, kEpiNone>(L, CT, cp, rc, vc, dY, L->out, L->in, B, dX, ep, s);
    }
    const bool tiled = L->dtype == CSP_F32 && segment_tiles_usable(L, pow2_ld(B));
    if (!tiled && (st = tasks_ready(L, s)) != CSP_OK) return st;
    st = batch_minor(L, B, io.dyt ? nullptr : dY, L->out, L->act.a, nullptr, 0, nullptr, s);
    if (st != CSP_OK) return st;
    const void *dyt = io.dyt ? io.dyt : (B == 1 ? dY : L->act.a);
    if (tiled) {
        const Tiles &T = L->tiles_c;
        const float *v = (const float *)L->vals_c, *g = (const float *)dyt;
        return act_in ? launch_segment_tiles<kEpiActGrad>(L, kTimeBoth, T, L->rows_by_col, v, g, B, (float *)dX, ep, s)
                      : launch_segment_tiles<kEpiNone>(L, kTimeBoth, T, L->rows_by_col, v, g, B, (float *)dX, ep, s);
    }
    if (L->dtype == CSP_BF16)
        return act_in ? bwd_input_dispatch<BF16, kEpiActGrad>(L, dyt, B, dX, ep, s)
                      : bwd_input_dispatch<BF16, kEpiNone>(L, dyt, B, dX, ep, s);
    return act_in ? bwd_input_dispatch<F32, kEpiActGrad>(L, dyt, B, dX, ep, s)
                  : bwd_input_dispatch<F32, kEpiNone>(L, dyt, B, dX, ep, s);
}

csp_status bwd_values_slice(csp_layer *L, const void *dY, const void *X, int64_t B, float *dW, bool acc, hipStream_t s,
                            const BmIO &io)
{
    csp_status st = CSP_OK;
    if (lds_table_fits(L, B, L->in)) {
        if ((st = tasks_ready(L, s)) != CSP_OK) return st;
        const Epi ep;
        return L->dtype == CSP_BF16 ? gradients_lds_dispatch<BF16, kEpiNone>(L, X, dY, B, nullptr, dW, false, acc, ep, s)
                                    : gradients_lds_dispatch<F32, kEpiNone>(L, X, dY, B, nullptr, dW, false, acc, ep, s);
    }
    st = batch_minor(L, B, io.xt ? nullptr : X, L->in, L->act.a, io.dyt ? nullptr : dY, L->out, L->act.b, s);
    if (st != CSP_OK) return st;
    const void *xt = io.xt ? io.xt : (B == 1 ? X : L->act.a);
    const void *dyt = io.dyt ? io.dyt : (B == 1 ? dY : L->act.b);
    return L->dtype == CSP_BF16 ? bwd_values_dispatch<BF16>(L, xt, dyt, B, dW, acc, s)
                                : bwd_values_dispatch<F32>(L, xt, dyt, B, dW, acc, s);
}

csp_status bwd_slice(csp_layer *L, const void *dY, const void *X, int64_t B, void *dX, float *dW, const void *act_in,
                     bool acc, hipStream_t s, const BmIO &io)
{
    csp_status st = CSP_OK;
    Epi ep;
    ep.act_in = act_in;
    ep.outT = io.outt;
    ep.ldT = pow2_ld(B);
    if (lds_table_fits(L, B, L->in > L->out ? L->in : L->out)) {
        if ((st = tasks_ready(L, s)) != CSP_OK) return st;
        if (L->dtype == CSP_BF16)
            return act_in ? gradients_lds_dispatch<BF16, kEpiActGrad>(L, X, dY, B, dX, dW, true, acc, ep, s)
                          : gradients_lds_dispatch<BF16, kEpiNone>(L, X, dY, B, dX, dW, true, acc, ep, s);
        return act_in ? gradients_lds_dispatch<F32, kEpiActGrad>(L, X, dY, B, dX, dW, true, acc, ep, s)
                      : gradients_lds_dispatch<F32, kEpiNone>(L, X, dY, B, dX, dW, true, acc, ep, s);
    }
    st = batch_minor(L, B, io.xt ? nullptr : X, L->in, L->act.a, io.dyt ? nullptr : dY, L->out, L->act.b, s);
    if (st != CSP_OK) return st;
    const void *xt = io.xt ? io.xt : (B == 1 ? X : L->act.a);
    const void *dyt = io.dyt ? io.dyt : (B == 1 ? dY : L->act.b);
    if (L->dtype == CSP_BF16)
        return act_in ? bwd_dispatch<BF16, kEpiActGrad>(L, xt, dyt, B, dX, dW, acc, ep, s)
                      : bwd_dispatch<BF16, kEpiNone>(L, xt, dyt, B, dX, dW, acc, ep, s);
    return act_in ? bwd_dispatch<F32, kEpiActGrad>(L, xt, dyt, B, dX, dW, acc, ep, s)
                  : bwd_dispatch<F32, kEpiNone>(L, xt, dyt, B, dX, dW, acc, ep, s);
}

}  // namespace

// Batches above kSliceB run as consecutive slices of kSliceB rows of the
// row-major operands (one batch-minor chunk each), so the operand workspace
// sized at create serves every batch and no call allocates.  The value
// gradient of a later slice is added to the earlier ones in slice order.
constexpr int64_t kSliceB = kSliceRows;

namespace {
inline const void *rows_at(const void *p, int64_t r, int64_t n, int esz)
{
    return p ? (const char *)p + r * n * esz : nullptr;
}
inline void *rows_at(void *p, int64_t r, int64_t n, int esz) { return p ? (char *)p + r * n * esz : nullptr; }
}  // namespace

csp_status fwd_work_bytes(csp_layer *L, int64_t B, size_t *operand_bytes, size_t *partial_bytes)
{
    *operand_bytes = *partial_bytes = 0;
    // the slices are kSliceB rows, then the remainder
    const int64_t sizes[2] = {B < kSliceB ? B : kSliceB, B > kSliceB ? (B - 1) % kSliceB + 1 : 0};
    for (int64_t bs : sizes) {
        if (bs <= 0) continue;
        size_t o = 0, p = 0;
        fwd_slice_work(L, bs, &o, &p);
        if (o > *operand_bytes) *operand_bytes = o;
        if (p > *partial_bytes) *partial_bytes = p;
    }
    return CSP_OK;
}

csp_status launch_fwd(csp_layer *L, const void *X, int64_t B, void *Y, const FwdEpilogue *fe, hipStream_t s,
                      const FwdWork *work, const BmIO &io)
{
    FwdWork wk;
    if (work) wk = *work;
    else {
        wk.operand = L->act.a;
        wk.partial = L->act.partial;
    }
    for (int64_t b0 = 0; b0 < B; b0 += kSliceB) {
        const int64_t bs = B - b0 < kSliceB ? B - b0 : kSliceB;
        FwdEpilogue f{};
        if (fe) {
            f = *fe;
            f.pre = rows_at(f.pre, b0, L->out, L->esz);
        }
        const csp_status st = fwd_slice(L, rows_at(X, b0, L->in, L->esz), bs, rows_at(Y, b0, L->out, L->esz),
                                        fe ? &f : nullptr, s, wk, io);
        if (st != CSP_OK) return st;
    }
    return CSP_OK;
}

csp_status launch_bwd_input(csp_layer *L, const void *dY, int64_t B, void *dX, const void *act_in, hipStream_t s,
                            const BmIO &io)
{
    for (int64_t b0 = 0; b0 < B; b0 += kSliceB) {
        const int64_t bs = B - b0 < kSliceB ? B - b0 : kSliceB;
        const csp_status st = bwd_input_slice(L, rows_at(dY, b0, L->out, L->esz), bs, rows_at(dX, b0, L->in, L->esz),
                                              rows_at(act_in, b0, L->in, L->esz), s, io);
        if (st != CSP_OK) return st;
    }
    return CSP_OK;
}

csp_status launch_bwd_values(csp_layer *L, const void *dY, const void *X, int64_t B, float *dW, hipStream_t s,
                             const BmIO &io)
{
    if (L->nnz == 0) return CSP_OK;
    for (int64_t b0 = 0; b0 < B; b0 += kSliceB) {
        const int64_t bs = B - b0 < kSliceB ? B - b0 : kSliceB;
        const csp_status st = bwd_values_slice(L, rows_at(dY, b0, L->out, L->esz), rows_at(X, b0, L->in, L->esz), bs, dW,
                                               b0 > 0, s, io);
        if (st != CSP_OK) return st;
    }
    return CSP_OK;
}

csp_status launch_bwd(csp_layer *L, const void *dY, const void *X, int64_t B, void *dX, float *dW, const void *act_in,
                      hipStream_t s, const BmIO &io)
{
    for (int64_t b0 = 0; b0 < B; b0 += kSliceB) {
        const int64_t bs = B - b0 < kSliceB ? B - b0 : kSliceB;
        const csp_status st = bwd_slice(L, rows_at(dY, b0, L->out, L->esz), rows_at(X, b0, L->in, L->esz), bs,
                                        rows_at(dX, b0, L->in, L->esz), dW, rows_at(act_in, b0, L->in, L->esz),
                                        b0 > 0, s, io);
        if (st != CSP_OK) return st;
    }
    return CSP_OK;
}

// spmm_batch_minor: the copy itself, for a caller's operand.
csp_status batch_minor_copy(int esz, int64_t B, const void *src, int64_t n, void *dst, hipStream_t s)
{
    csp_layer tmp;  // only its element size is read
    tmp.esz = esz;
    return batch_minor(&tmp, B, src, n, dst, nullptr, 0, nullptr, s);
}

}  // namespace csp
