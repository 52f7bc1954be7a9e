// spmm.hip -- forward product, input gradient and value gradient of the
// truly sparse COO layer ("Beyond Masked Sparsity: SNACK ...", Abstract:
// the layer computes only its stored connections, forward and backward).
//
//   forward      Y[b,r]  = sum_{k in row r} v_k X[b,col_k]
//   input grad   dX[b,c] = sum_{k in col c} v_k dY[b,row_k]
//   value grad   dW_k    = sum_b dY[b,row_k] X[b,col_k]
//
// Memory layout.  Dense operands arrive row-major ([B, n]).  For B > 1 each
// kernel first copies its gathered operand to a batch-minor layout [n][ld]
// (ld = batch padded to a power of two, at most 64; larger batches are cut
// into chunks of 64), so that the B values one stored entry needs are one
// contiguous 4*ld-byte run: a single coalesced load instead of B scattered
// ones.  Inside a wavefront, lane = (slot s, batch b) with S = 64/ld slots:
// each slot walks every S-th entry of a segment, and slots are summed with
// cross-lane shuffles at the end of the segment.  No MFMA: an unstructured
// gather is not a dense contraction; the kernels are bound by HBM for the
// COO stream and by L2/L1 for the operand gathers.
#include "common.h"

namespace csp {
namespace {

// ----------------------------------------------------------------- dtype glue
struct F32 {
    using T = float;
    __device__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ static float to_f(float v) { return v; }
    __device__ static float from_f(float v) { return v; }
};
struct BF16 {
    using T = uint16_t;
    __device__ static float load(const uint16_t *p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
    __device__ static float to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
    __device__ static uint16_t from_f(float f)  // round to nearest even
    {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};

inline int pow2_ld(int64_t B)
{
    int ld = 1;
    while (ld < B && ld < 64) ld <<= 1;
    return ld;
}

// ------------------------------------------------------- batch-minor copy
// X [B, n] row-major -> XT[ch][n][ld], zero-padded in the batch dimension.
template <typename T>
__global__ __launch_bounds__(256) void k_batch_minor(const T *__restrict__ X, int64_t B, int64_t n, int ld,
                                                     T *__restrict__ XT)
{
    __shared__ T tile[64][65];
    const int t = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int64_t ch = blockIdx.y;
    const int tot = ld * 64;
    for (int e = t; e < tot; e += 256) {
        int bl = e >> 6, c = e & 63;
        int64_t b = ch * ld + bl;
        tile[bl][c] = (b < B && c0 + c < n) ? X[b * n + c0 + c] : T(0);
    }
    __syncthreads();
    for (int e = t; e < tot; e += 256) {
        int c = e / ld, bl = e % ld;
        if (c0 + c < n) XT[((ch * n) + c0 + c) * ld + bl] = tile[bl][c];
    }
}

// ------------------------------------------------------------- forward
// One wavefront per output row; 4 rows per 256-thread block.
template <int LD, typename D>
__global__ __launch_bounds__(256) void k_fwd_rows(int64_t out, int64_t in, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ cols,
                                                  const typename D::T *__restrict__ vals,
                                                  const typename D::T *__restrict__ XT, int64_t B,
                                                  typename D::T *__restrict__ Y)
{
    constexpr int S = kWave / LD;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= out) return;
    const int lane = threadIdx.x & 63, s = lane / LD, b = lane % LD;
    const int64_t ch = blockIdx.y;
    const typename D::T *xt = XT + ch * in * LD;
    const int k0 = row_ptr[r], k1 = row_ptr[r + 1];
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int k = k0 + s;
    for (; k + 3 * S < k1; k += 4 * S) {
        int c0 = cols[k], c1 = cols[k + S], c2 = cols[k + 2 * S], c3 = cols[k + 3 * S];
        float v0 = D::load(vals, k), v1 = D::load(vals, k + S), v2 = D::load(vals, k + 2 * S),
              v3 = D::load(vals, k + 3 * S);
        a0 += v0 * D::load(xt, (int64_t)c0 * LD + b);
        a1 += v1 * D::load(xt, (int64_t)c1 * LD + b);
        a2 += v2 * D::load(xt, (int64_t)c2 * LD + b);
        a3 += v3 * D::load(xt, (int64_t)c3 * LD + b);
    }
    for (; k < k1; k += S) a0 += D::load(vals, k) * D::load(xt, (int64_t)cols[k] * LD + b);
    float acc = (a0 + a1) + (a2 + a3);
#pragma unroll
    for (int off = LD; off < kWave; off <<= 1) acc += __shfl_xor(acc, off, 64);
    const int64_t bg = ch * LD + b;
    if (s == 0 && bg < B) Y[bg * out + r] = D::from_f(acc);
}

// ---------------------------------------------------------- input gradient
// One wavefront per input column, over the transposed view.
template <int LD>
__global__ __launch_bounds__(256) void k_bwd_input_cols(int64_t out, int64_t in, const int32_t *__restrict__ col_ptr,
                                                        const int32_t *__restrict__ rows_by_col,
                                                        const int32_t *__restrict__ perm_c,
                                                        const float *__restrict__ vals,
                                                        const float *__restrict__ dYT, int64_t B,
                                                        float *__restrict__ dX)
{
    constexpr int S = kWave / LD;
    const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= in) return;
    const int lane = threadIdx.x & 63, s = lane / LD, b = lane % LD;
    const int64_t ch = blockIdx.y;
    const float *dyt = dYT + ch * out * LD;
    const int j0 = col_ptr[c], j1 = col_ptr[c + 1];
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int j = j0 + s;
    for (; j + 3 * S < j1; j += 4 * S) {
        int r0 = rows_by_col[j], r1 = rows_by_col[j + S], r2 = rows_by_col[j + 2 * S], r3 = rows_by_col[j + 3 * S];
        float v0 = vals[perm_c[j]], v1 = vals[perm_c[j + S]], v2 = vals[perm_c[j + 2 * S]],
              v3 = vals[perm_c[j + 3 * S]];
        a0 += v0 * dyt[(int64_t)r0 * LD + b];
        a1 += v1 * dyt[(int64_t)r1 * LD + b];
        a2 += v2 * dyt[(int64_t)r2 * LD + b];
        a3 += v3 * dyt[(int64_t)r3 * LD + b];
    }
    for (; j < j1; j += S) a0 += vals[perm_c[j]] * dyt[(int64_t)rows_by_col[j] * LD + b];
    float acc = (a0 + a1) + (a2 + a3);
#pragma unroll
    for (int off = LD; off < kWave; off <<= 1) acc += __shfl_xor(acc, off, 64);
    const int64_t bg = ch * LD + b;
    if (s == 0 && bg < B) dX[bg * in + c] = acc;
}

// ---------------------------------------------------------- value gradient
// One thread per stored entry: dot product over the batch of two
// batch-minor rows (dY row of row_k, X row of col_k).
template <int LD>
__global__ __launch_bounds__(256) void k_bwd_values(int64_t nnz, int64_t out, int64_t in, int nch,
                                                    const int32_t *__restrict__ rows,
                                                    const int32_t *__restrict__ cols, const float *__restrict__ dYT,
                                                    const float *__restrict__ XT, float *__restrict__ dW)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    const int64_t r = rows[k], c = cols[k];
    float acc0 = 0.f, acc1 = 0.f;
    for (int ch = 0; ch < nch; ++ch) {
        const float *dy = dYT + ((int64_t)ch * out + r) * LD;
        const float *x = XT + ((int64_t)ch * in + c) * LD;
        if constexpr (LD >= 4) {
#pragma unroll
            for (int b = 0; b < LD; b += 4) {
                float4 p = *(const float4 *)(dy + b);
                float4 q = *(const float4 *)(x + b);
                acc0 += p.x * q.x + p.z * q.z;
                acc1 += p.y * q.y + p.w * q.w;
            }
        } else {
#pragma unroll
            for (int b = 0; b < LD; ++b) acc0 += dy[b] * x[b];
        }
    }
    dW[k] = acc0 + acc1;
}

// ------------------------------------------------------------ host side
csp_status ensure_act(csp_layer *L, size_t bytes)
{
    if (L->act.bytes >= bytes) return CSP_OK;
    if (L->act.a) CSP_HIP(hipFree(L->act.a));
    if (L->act.b) CSP_HIP(hipFree(L->act.b));
    L->act.a = L->act.b = nullptr;
    L->act.bytes = 0;
    if (hipMalloc(&L->act.a, bytes) != hipSuccess || hipMalloc(&L->act.b, bytes) != hipSuccess) {
        (void)hipGetLastError();
        if (L->act.a) (void)hipFree(L->act.a);
        L->act.a = nullptr;
        return set_error(CSP_ERR_NO_MEMORY, "cannot allocate %zu bytes of operand workspace", bytes);
    }
    L->act.bytes = bytes;
    return CSP_OK;
}

// Copy a [B, n] operand to batch-minor layout; returns the pointer to use.
csp_status batch_minor(csp_layer *L, const void *X, int64_t B, int64_t n, void *dst, const void **xt,
                       hipStream_t s)
{
    if (B == 1) {  // [1, n] is already batch-minor
        *xt = X;
        return CSP_OK;
    }
    const int ld = pow2_ld(B);
    const int64_t nch = ceil_div(B, ld);
    dim3 grid((unsigned)ceil_div(n, 64), (unsigned)nch);
    if (L->esz == 4)
        k_batch_minor<float><<<grid, 256, 0, s>>>((const float *)X, B, n, ld, (float *)dst);
    else
        k_batch_minor<uint16_t><<<grid, 256, 0, s>>>((const uint16_t *)X, B, n, ld, (uint16_t *)dst);
    CSP_LAUNCHED("k_batch_minor");
    *xt = dst;
    return CSP_OK;
}

size_t batch_minor_bytes(const csp_layer *L, int64_t B, int64_t n)
{
    const int ld = pow2_ld(B);
    return (size_t)ceil_div(B, ld) * (size_t)n * (size_t)ld * (size_t)L->esz;
}

template <typename D>
csp_status fwd_dispatch(csp_layer *L, const void *XT, int64_t B, void *Y, hipStream_t s)
{
    using T = typename D::T;
    const int ld = pow2_ld(B);
    dim3 grid((unsigned)ceil_div(L->out, 4), (unsigned)ceil_div(B, ld));
    const T *v = (const T *)L->vals;
    const T *x = (const T *)XT;
    T *y = (T *)Y;
    switch (ld) {
    case 1: k_fwd_rows<1, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    case 2: k_fwd_rows<2, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    case 4: k_fwd_rows<4, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    case 8: k_fwd_rows<8, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    case 16: k_fwd_rows<16, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    case 32: k_fwd_rows<32, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    default: k_fwd_rows<64, D><<<grid, 256, 0, s>>>(L->out, L->in, L->row_ptr, L->cols, v, x, B, y); break;
    }
    CSP_LAUNCHED("k_fwd_rows");
    return CSP_OK;
}

}  // namespace

csp_status launch_fwd(csp_layer *L, const void *X, int64_t B, void *Y, hipStream_t s)
{
    csp_status st = ensure_act(L, batch_minor_bytes(L, B, L->in));
    if (st != CSP_OK) return st;
    const void *xt = nullptr;
    st = batch_minor(L, X, B, L->in, L->act.a, &xt, s);
    if (st != CSP_OK) return st;
    return L->dtype == CSP_BF16 ? fwd_dispatch<BF16>(L, xt, B, Y, s) : fwd_dispatch<F32>(L, xt, B, Y, s);
}

csp_status launch_bwd_input(csp_layer *L, const void *dY, int64_t B, void *dX, hipStream_t s)
{
    csp_status st = ensure_act(L, batch_minor_bytes(L, B, L->out));
    if (st != CSP_OK) return st;
    const void *dyt = nullptr;
    st = batch_minor(L, dY, B, L->out, L->act.a, &dyt, s);
    if (st != CSP_OK) return st;
    const int ld = pow2_ld(B);
    dim3 grid((unsigned)ceil_div(L->in, 4), (unsigned)ceil_div(B, ld));
    const float *v = (const float *)L->vals, *g = (const float *)dyt;
    float *o = (float *)dX;
#define CSP_BWD_IN(LDV)                                                                                      \
    k_bwd_input_cols<LDV><<<grid, 256, 0, s>>>(L->out, L->in, L->col_ptr, L->rows_by_col, L->perm_c, v, g, B, o)
    switch (ld) {
    case 1: CSP_BWD_IN(1); break;
    case 2: CSP_BWD_IN(2); break;
    case 4: CSP_BWD_IN(4); break;
    case 8: CSP_BWD_IN(8); break;
    case 16: CSP_BWD_IN(16); break;
    case 32: CSP_BWD_IN(32); break;
    default: CSP_BWD_IN(64); break;
    }
#undef CSP_BWD_IN
    CSP_LAUNCHED("k_bwd_input_cols");
    return CSP_OK;
}

csp_status launch_bwd_values(csp_layer *L, const void *dY, const void *X, int64_t B, float *dW, hipStream_t s)
{
    if (L->nnz == 0) return CSP_OK;
    size_t need = batch_minor_bytes(L, B, L->in > L->out ? L->in : L->out);
    csp_status st = ensure_act(L, need);
    if (st != CSP_OK) return st;
    const void *xt = nullptr, *dyt = nullptr;
    st = batch_minor(L, X, B, L->in, L->act.a, &xt, s);
    if (st != CSP_OK) return st;
    st = batch_minor(L, dY, B, L->out, L->act.b, &dyt, s);
    if (st != CSP_OK) return st;
    const int ld = pow2_ld(B);
    const int nch = (int)ceil_div(B, ld);
    const unsigned grid = (unsigned)ceil_div(L->nnz, 256);
    const float *g = (const float *)dyt, *x = (const float *)xt;
#define CSP_BWD_V(LDV) \
    k_bwd_values<LDV><<<grid, 256, 0, s>>>(L->nnz, L->out, L->in, nch, L->rows, L->cols, g, x, dW)
    switch (ld) {
    case 1: CSP_BWD_V(1); break;
    case 2: CSP_BWD_V(2); break;
    case 4: CSP_BWD_V(4); break;
    case 8: CSP_BWD_V(8); break;
    case 16: CSP_BWD_V(16); break;
    case 32: CSP_BWD_V(32); break;
    default: CSP_BWD_V(64); break;
    }
#undef CSP_BWD_V
    CSP_LAUNCHED("k_bwd_values");
    return CSP_OK;
}

}  // namespace csp
