// layer.hip -- the C ABI of the truly sparse COO layer (include/coospmm.h):
// argument checks on the host, layer memory, and the calls into the kernels.
// Method: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks
// on GPU", Abstract (COO storage of non-zero connections only; forward and
// backward on the sparse storage; restructuring for dynamic sparse training).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "common.h"

namespace csp {

static thread_local char g_last_error[512] = "";

csp_status set_error(csp_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

csp_status hip_error(hipError_t e, const char *what)
{
    if (e == hipErrorOutOfMemory) return set_error(CSP_ERR_NO_MEMORY, "%s: %s", what, hipGetErrorString(e));
    return set_error(CSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

constexpr int64_t kIndexLimit = 0x7FFFFFFF;  // int32 indices and offsets

// Runs the body with the layer's device current, restoring the caller's.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard()
    {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

csp_status dalloc(void **p, size_t bytes, const char *what)
{
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return set_error(CSP_ERR_NO_MEMORY, "cannot allocate %zu bytes for %s", bytes, what);
    }
    return CSP_OK;
}

void free_layer(csp_layer *L)
{
    if (!L) return;
    void *ptrs[] = {L->rows, L->cols, L->vals, L->row_ptr, L->perm_c, L->rows_by_col, L->col_ptr, L->vals_c,
                    L->ws.key_a, L->ws.key_b, L->ws.idx_a, L->ws.idx_b, L->ws.u_a, L->ws.u_b, L->ws.hist,
                    L->ws.rows_k, L->ws.cols_k, L->ws.vals_k, L->ws.rp_k, L->ws.rp_new, L->ws.acc_a, L->ws.acc_b, L->ws.sel,
                    L->ws.occ, L->ws.occ_next, L->ws.occ_pref, L->ws.occ_pref_next, L->ws.tcnt, L->ws.hash, L->ws.score,
                    L->act.a, L->act.b, L->act.partial,
                    L->row_tasks.desc, L->row_tasks.split, L->row_tasks.seg_first,
                    L->col_tasks.desc, L->col_tasks.split, L->col_tasks.seg_first,
                    L->row_packed.desc, L->row_packed.split,
                    L->row_tasks.split_cls, L->col_tasks.split_cls, L->row_packed.split_cls,
                    L->tiles_r.ptr, L->tiles_r.slots, L->tiles_c.ptr, L->tiles_c.slots, L->tile_partial};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    delete L;
}

csp_status alloc_layer(csp_layer *L)
{
    const int64_t nnz = L->nnz, out = L->out, in = L->in;
    // Entry arrays carry 8 spare elements: the packed forward loads whole
    // 8-entry groups, and the last group of a layer may reach 7 past its end.
    const size_t n = (size_t)nnz + 8;
    Workspace &W = L->ws;
    W.nkey_cap = nnz > 65536 ? nnz : 65536;
    W.hist_words = sort_hist_words(W.nkey_cap);
    const int64_t nseg_max = out > in ? out : in;
    // scan partials of the three task lists
    const size_t task_words = (size_t)(2 * ceil_div(nseg_max, 1024) + ceil_div(out, (int64_t)kPackSegs) + 64);
    if (W.hist_words < task_words) W.hist_words = task_words;
    const bool bitmap = plan_bitmap(L);
    if (bitmap && W.hist_words < bitmap_hist_words(L)) W.hist_words = bitmap_hist_words(L);
    const size_t cap = (size_t)W.nkey_cap;
    L->row_tasks.cap = task_cap(out, nnz);
    L->col_tasks.cap = task_cap(in, nnz);
    L->row_packed.cap = L->row_tasks.cap;  // packing only merges whole-row tasks
    const size_t act_bytes = (size_t)L->esz * kSliceRows * (size_t)nseg_max;
    const size_t tcap = (size_t)(L->row_tasks.cap > L->col_tasks.cap ? L->row_tasks.cap : L->col_tasks.cap);
    const size_t partial_bytes = sizeof(float) * kSliceRows * tcap;
    L->act.bytes = act_bytes;
    L->act.partial_bytes = partial_bytes;
    struct Req { void **p; size_t bytes; const char *what; } reqs[] = {
        {(void **)&L->rows, 4 * n, "rows"},
        {(void **)&L->cols, 4 * n, "cols"},
        {(void **)&L->vals, (size_t)L->esz * n, "values"},
        {(void **)&L->row_ptr, 4 * (size_t)(out + 1), "row offsets"},
        {(void **)&L->perm_c, 4 * n, "column permutation"},
        {(void **)&L->rows_by_col, 4 * n, "rows by column"},
        {(void **)&L->col_ptr, 4 * (size_t)(in + 1), "column offsets"},
        {&L->vals_c, (size_t)L->esz * n, "column-ordered values"},
        {&W.key_a, 8 * cap, "sort keys"},
        {&W.key_b, 8 * cap, "sort keys"},
        {(void **)&W.idx_a, 4 * cap, "sort values"},
        {(void **)&W.idx_b, 4 * cap, "sort values"},
        {(void **)&W.u_a, 4 * cap, "scan scratch"},
        {(void **)&W.u_b, 4 * cap, "scan scratch"},
        {(void **)&W.hist, 4 * W.hist_words, "histograms"},
        {(void **)&W.rows_k, 4 * n, "kept rows"},
        {(void **)&W.cols_k, 4 * n, "kept cols"},
        {&W.vals_k, (size_t)L->esz * n, "kept values"},
        {(void **)&W.rp_k, 4 * (size_t)(out + 1), "kept offsets"},
        {(void **)&W.rp_new, 4 * (size_t)(out + 1), "regrown offsets"},
        {(void **)&W.acc_a, 8 * n, "regrow positions"},
        {(void **)&W.acc_b, 8 * n, "regrow positions"},
        {(void **)&W.sel, 4 * (size_t)kSelAllocWords, "select state"},
        {(void **)&L->row_tasks.desc, 16 * (size_t)L->row_tasks.cap, "row tasks"},
        {(void **)&L->row_tasks.split, 16 * (size_t)out, "split rows"},
        {(void **)&L->row_tasks.seg_first, 4 * (size_t)(out + 1), "row task offsets"},
        {(void **)&L->col_tasks.desc, 16 * (size_t)L->col_tasks.cap, "column tasks"},
        {(void **)&L->col_tasks.split, 16 * (size_t)in, "split columns"},
        {(void **)&L->col_tasks.seg_first, 4 * (size_t)(in + 1), "column task offsets"},
        {(void **)&L->row_packed.desc, 16 * (size_t)L->row_packed.cap, "packed row tasks"},
        {(void **)&L->row_packed.split, 16 * (size_t)out, "split rows (packed list)"},
        {(void **)&L->row_tasks.split_cls, 16 * (size_t)kSplitClasses * out, "split rows by class"},
        {(void **)&L->col_tasks.split_cls, 16 * (size_t)kSplitClasses * in, "split columns by class"},
        {(void **)&L->row_packed.split_cls, 16 * (size_t)kSplitClasses * out, "split rows by class (packed list)"},
        // batch-minor operand copies for one slice of up to 64 batch rows, and the split partial sums
        {&L->act.a, act_bytes, "operand copy"},
        {&L->act.b, act_bytes, "operand copy"},
        {(void **)&L->act.partial, partial_bytes, "split partial sums"},
    };
    for (auto &r : reqs) {
        csp_status st = dalloc(r.p, r.bytes, r.what);
        if (st != CSP_OK) return st;
    }
    // LDS tiles: fp32, and at least one tile per compute unit (fewer would leave units idle)
    if (L->esz == 4 && ceil_div(out, kTileRows) * ceil_div(in, kTileCols) >= L->act.cus) {
        Tiles *T[2] = {&L->tiles_r, &L->tiles_c};
        const int64_t nseg[2] = {out, in}, nop[2] = {in, out};
        size_t partial = 0;
        for (int v = 0; v < 2; ++v) {
            T[v]->nseg = nseg[v];
            T[v]->nop = nop[v];
            T[v]->ncb = ceil_div(nop[v], kTileCols);
            T[v]->nrb = ceil_div(nseg[v], kTileRows);
            csp_status st = dalloc((void **)&T[v]->ptr, 4 * (size_t)nseg[v] * (size_t)(T[v]->ncb + 1), "tile offsets");
            if (st == CSP_OK)
                st = dalloc((void **)&T[v]->slots, sizeof(int2) * (size_t)(T[v]->nrb * T[v]->ncb) * kTileRows,
                            "tile segment slots");
            if (st != CSP_OK) return st;
            const size_t p = sizeof(float) * kSliceRows * (size_t)T[v]->ncb * (size_t)nseg[v];
            partial = p > partial ? p : partial;
        }
        csp_status st = dalloc((void **)&L->tile_partial, partial, "tile partial sums");
        if (st != CSP_OK) return st;
    }
    if (!bitmap) return CSP_OK;
    Req breqs[] = {
        {(void **)&W.occ, 4 * (size_t)W.occ_words, "position bitmap"},
        {(void **)&W.occ_next, 4 * (size_t)W.occ_words, "position bitmap"},
        {(void **)&W.occ_pref, 4 * (size_t)(W.occ_words + 1), "bitmap ranks"},
        {(void **)&W.occ_pref_next, 4 * (size_t)(W.occ_words + 1), "bitmap ranks"},
        {(void **)&W.tcnt, 4 * (size_t)W.tcnt_words, "transposition counts"},
        {(void **)&W.hash, 8 * (size_t)W.hash_slots, "regrow hash table"},
    };
    for (auto &r : breqs) {
        csp_status st = dalloc(r.p, r.bytes, r.what);
        if (st != CSP_OK) return st;
    }
    return CSP_OK;
}

// ---------------------------------------------------------------------------
// Static workspace of spmm_fwd_static: one array per GPU, held until the
// process ends.  In host code the array's name stands for a host-side symbol;
// its device address on each GPU comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address reaches kernels.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

csp_status scratch_on(int dev, void **ptr)
{
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(CSP_ERR_HIP, "device %d is beyond the static workspace table (%d devices)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress(scratch)");
        if (!p) return set_error(CSP_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return CSP_OK;
}

// Every call that reads or changes the layer's contents refuses a layer left
// incomplete by a failed restructure.
csp_status check_usable(const csp_layer *L)
{
    if (L->broken)
        return set_error(CSP_ERR_INVALID_ARG,
                         "the layer was left incomplete by a failed restructure; destroy it and create it again");
    return CSP_OK;
}

#define CSP_USABLE(L)                                     \
    do {                                                  \
        const csp_status u_ = ::csp::check_usable(L);     \
        if (u_ != CSP_OK) return u_;                      \
    } while (0)

uint32_t regrow_word(const csp_layer *L, float v)
{
    uint32_t u;
    std::memcpy(&u, &v, 4);
    if (L->dtype == CSP_F32) return u;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;                  // nearest even
}

}  // namespace
}  // namespace csp

using namespace csp;

extern "C" {

csp_status sparse_layer_create(int64_t out_features, int64_t in_features, int64_t nnz, const int32_t *rows,
                               const int32_t *cols, const void *vals, csp_dtype dtype, void *stream,
                               sparse_layer_t *out_layer)
{
    if (!out_layer) return set_error(CSP_ERR_INVALID_ARG, "out_layer is NULL");
    *out_layer = nullptr;
    if (out_features <= 0 || in_features <= 0 || out_features > kIndexLimit || in_features > kIndexLimit)
        return set_error(CSP_ERR_INVALID_ARG, "shape %lld x %lld outside [1, 2^31)", (long long)out_features,
                         (long long)in_features);
    if (nnz < 0 || nnz > kIndexLimit || nnz > out_features * in_features)
        return set_error(CSP_ERR_INVALID_ARG, "nnz %lld outside [0, min(out*in, 2^31))", (long long)nnz);
    if (nnz > 0 && (!rows || !cols || !vals)) return set_error(CSP_ERR_INVALID_ARG, "NULL triple array");
    if (dtype != CSP_F32 && dtype != CSP_BF16) return set_error(CSP_ERR_DTYPE, "unknown dtype %d", (int)dtype);

    csp_layer *L = new (std::nothrow) csp_layer;
    if (!L) return set_error(CSP_ERR_NO_MEMORY, "host allocation failed");
    L->out = out_features;
    L->in = in_features;
    L->nnz = nnz;
    L->dtype = dtype;
    L->esz = dtype == CSP_BF16 ? 2 : 4;
    if (hipGetDevice(&L->device) != hipSuccess) {
        delete L;
        return set_error(CSP_ERR_HIP, "hipGetDevice failed");
    }
    hipStream_t s = (hipStream_t)stream;
    if (hipDeviceGetAttribute(&L->act.cus, hipDeviceAttributeMultiprocessorCount, L->device) != hipSuccess ||
        L->act.cus <= 0) {
        delete L;
        return set_error(CSP_ERR_HIP, "cannot query the compute-unit count");
    }
    csp_status st = alloc_layer(L);
    if (st == CSP_OK) st = fill_u32(L->ws.sel, 0u, kSelAllocWords, s);
    if (st == CSP_OK) st = build_canonical(L, rows, cols, vals, L->ws.sel, s);
    if (st == CSP_OK) st = build_index(L, s);
    if (st == CSP_OK) st = build_tiles(L, s);
    if (st == CSP_OK) st = occupancy_init(L, s);
    uint32_t flags = 0;
    if (st == CSP_OK) {
        hipError_t e = hipMemcpyAsync(&flags, L->ws.sel, sizeof flags, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) st = hip_error(e, "reading the validation flags");
    }
    if (st == CSP_OK && (flags & 2u)) st = set_error(CSP_ERR_INDEX_RANGE, "a row or column index is out of range");
    if (st == CSP_OK && (flags & 4u)) st = set_error(CSP_ERR_DUPLICATE, "a (row, col) pair appears more than once");
    if (st != CSP_OK) {
        (void)hipStreamSynchronize(s);
        free_layer(L);
        return st;
    }
    L->created = true;
    *out_layer = L;
    return CSP_OK;
}

void sparse_layer_destroy(sparse_layer_t layer)
{
    if (!layer) return;
    DeviceGuard g(layer->device);
    (void)hipDeviceSynchronize();
    free_layer(layer);
}

csp_status spmm_fwd(sparse_layer_t L, const void *X, int64_t B, void *Y, void *stream)
{
    if (!L || !X || !Y) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_fwd");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_fwd(L, X, B, Y, nullptr, (hipStream_t)stream);
}

csp_status spmm_fwd_act(sparse_layer_t L, const void *X, int64_t B, const void *bias, csp_act act, void *Y, void *H,
                        void *stream)
{
    if (!L || !X || !Y) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_fwd_act");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    if (act != CSP_ACT_NONE && act != CSP_ACT_GELU) return set_error(CSP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if (H && H == Y) return set_error(CSP_ERR_INVALID_ARG, "H must not overlap Y");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    FwdEpilogue fe;
    fe.bias = bias;
    fe.pre = H;
    fe.gelu = act == CSP_ACT_GELU;
    return launch_fwd(L, X, B, Y, &fe, (hipStream_t)stream);
}

csp_status spmm_fwd_static(sparse_layer_t L, const void *X, int64_t B, void *Y, void *stream)
{
    if (!L || !X || !Y) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_fwd_static");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    size_t ob = 0, pb = 0;
    csp_status st = tasks_ready(L, (hipStream_t)stream);  // the workspace size depends on the task lists
    if (st != CSP_OK) return st;
    st = fwd_work_bytes(L, B, &ob, &pb);
    if (st != CSP_OK) return st;
    const size_t ob_al = (ob + 255) & ~size_t(255);
    if (ob_al + pb > kScratchBytes)
        return set_error(CSP_ERR_INVALID_ARG,
                         "spmm_fwd_static needs %zu bytes of workspace for this layer and batch; its static "
                         "array holds %zu (use spmm_fwd)", ob_al + pb, kScratchBytes);
    void *base = nullptr;
    st = scratch_on(L->device, &base);
    if (st != CSP_OK) return st;
    FwdWork wk;
    wk.operand = base;
    wk.partial = reinterpret_cast<float *>(static_cast<unsigned char *>(base) + ob_al);
    return launch_fwd(L, X, B, Y, nullptr, (hipStream_t)stream, &wk);
}

csp_status spmm_bwd_input(sparse_layer_t L, const void *dY, int64_t B, void *dX, void *stream)
{
    if (!L || !dY || !dX) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd_input");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_bwd_input(L, dY, B, dX, nullptr, (hipStream_t)stream);
}

csp_status spmm_bwd_input_act(sparse_layer_t L, const void *dY, int64_t B, csp_act act, const void *H_in, void *dX,
                              void *stream)
{
    if (!L || !dY || !dX) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd_input_act");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    if (act != CSP_ACT_NONE && act != CSP_ACT_GELU) return set_error(CSP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if (act == CSP_ACT_GELU && !H_in) return set_error(CSP_ERR_INVALID_ARG, "CSP_ACT_GELU needs H_in");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_bwd_input(L, dY, B, dX, act == CSP_ACT_GELU ? H_in : nullptr, (hipStream_t)stream);
}

csp_status spmm_bwd_values(sparse_layer_t L, const void *dY, const void *X, int64_t B, float *dW, void *stream)
{
    if (!L || !dY || !X || (!dW && L->nnz > 0)) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd_values");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_bwd_values(L, dY, X, B, dW, (hipStream_t)stream);
}

csp_status spmm_bwd(sparse_layer_t L, const void *dY, const void *X, int64_t B, void *dX, float *dW, void *stream)
{
    if (!L || !dY || !X || !dX || (!dW && L->nnz > 0)) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_bwd(L, dY, X, B, dX, dW, nullptr, (hipStream_t)stream);
}

csp_status spmm_bwd_act(sparse_layer_t L, const void *dY, const void *X, int64_t B, csp_act act, const void *H_in,
                        void *dX, float *dW, void *stream)
{
    if (!L || !dY || !X || !dX || (!dW && L->nnz > 0)) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd_act");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    if (act != CSP_ACT_NONE && act != CSP_ACT_GELU) return set_error(CSP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if (act == CSP_ACT_GELU && !H_in) return set_error(CSP_ERR_INVALID_ARG, "CSP_ACT_GELU needs H_in");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    return launch_bwd(L, dY, X, B, dX, dW, act == CSP_ACT_GELU ? H_in : nullptr, (hipStream_t)stream);
}

csp_status spmm_fwd_bm(sparse_layer_t L, const void *X, const void *XT, int64_t B, const void *bias, csp_act act,
                       void *Y, void *H, void *YT, void *stream)
{
    if (!L || !X || !Y) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_fwd_bm");
    if (B < 2 || B > kSliceRows)
        return set_error(CSP_ERR_INVALID_ARG, "spmm_fwd_bm takes batch-minor operands for 2 <= B <= %d, got %lld",
                         (int)kSliceRows, (long long)B);
    if (act != CSP_ACT_NONE && act != CSP_ACT_GELU) return set_error(CSP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if ((H && H == Y) || (YT && (YT == Y || YT == H))) return set_error(CSP_ERR_INVALID_ARG, "outputs must not overlap");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    FwdEpilogue fe;
    fe.bias = bias;
    fe.pre = H;
    fe.gelu = act == CSP_ACT_GELU;
    const bool plain = !bias && !H && act == CSP_ACT_NONE;  // then exactly spmm_fwd's arithmetic
    BmIO io;
    io.xt = XT;
    io.outt = YT;
    return launch_fwd(L, X, B, Y, plain ? nullptr : &fe, (hipStream_t)stream, nullptr, io);
}

csp_status spmm_bwd_bm(sparse_layer_t L, const void *dY, const void *dYT, const void *X, const void *XT, int64_t B,
                       csp_act act, const void *H_in, void *dX, void *dXT, float *dW, void *stream)
{
    if (!L || !dY || !X || !dX || (!dW && L->nnz > 0)) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_bwd_bm");
    if (B < 2 || B > kSliceRows)
        return set_error(CSP_ERR_INVALID_ARG, "spmm_bwd_bm takes batch-minor operands for 2 <= B <= %d, got %lld",
                         (int)kSliceRows, (long long)B);
    if (act != CSP_ACT_NONE && act != CSP_ACT_GELU) return set_error(CSP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if (act == CSP_ACT_GELU && !H_in) return set_error(CSP_ERR_INVALID_ARG, "CSP_ACT_GELU needs H_in");
    if (dXT && dXT == dX) return set_error(CSP_ERR_INVALID_ARG, "outputs must not overlap");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    BmIO io;
    io.xt = XT;
    io.dyt = dYT;
    io.outt = dXT;
    return launch_bwd(L, dY, X, B, dX, dW, act == CSP_ACT_GELU ? H_in : nullptr, (hipStream_t)stream, io);
}

csp_status spmm_batch_minor(const void *src, int64_t n, int64_t B, int32_t dtype, void *dst, void *stream)
{
    if (!src || !dst) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to spmm_batch_minor");
    if (B < 2 || B > kSliceRows || n < 0 || n > kIndexLimit)
        return set_error(CSP_ERR_INVALID_ARG, "spmm_batch_minor: B %lld outside [2, %d] or n %lld outside [0, 2^31)",
                         (long long)B, (int)kSliceRows, (long long)n);
    if (dtype != CSP_F32 && dtype != CSP_BF16) return set_error(CSP_ERR_DTYPE, "unknown dtype %d", (int)dtype);
    if (n == 0) return CSP_OK;
    return batch_minor_copy(dtype == CSP_F32 ? 4 : 2, B, src, n, dst, (hipStream_t)stream);
}

csp_status restructure(sparse_layer_t L, int64_t n_prune, uint64_t seed, uint64_t step, float regrow_value,
                       void *stream)
{
    if (!L) return set_error(CSP_ERR_INVALID_ARG, "NULL layer");
    if (n_prune < 0 || n_prune > L->nnz)
        return set_error(CSP_ERR_INVALID_ARG, "n_prune %lld outside [0, nnz = %lld]", (long long)n_prune,
                         (long long)L->nnz);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    hipStream_t s = (hipStream_t)stream;
    csp_status st = async_checked(L, s);  // a pending restructure_async must have completed in full
    if (st != CSP_OK) return st;
    st = run_restructure(L, n_prune, seed, step, regrow_word(L, regrow_value), s);
    if (st == CSP_OK && n_prune > 0) st = build_tiles(L, s);
    if (st == CSP_OK && n_prune > 0) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) st = hip_error(e, "restructure");
    }
    if (st != CSP_OK) L->broken = true;
    return st;
}

csp_status restructure_grad(sparse_layer_t L, int64_t n_prune, const void *dY, const void *X, int64_t B,
                            float regrow_value, void *stream)
{
    if (!L || !dY || !X) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to restructure_grad");
    if (B <= 0 || B > kIndexLimit) return set_error(CSP_ERR_INVALID_ARG, "batch %lld outside [1, 2^31)", (long long)B);
    if (n_prune < 0 || n_prune > L->nnz)
        return set_error(CSP_ERR_INVALID_ARG, "n_prune %lld outside [0, nnz = %lld]", (long long)n_prune,
                         (long long)L->nnz);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    hipStream_t s = (hipStream_t)stream;
    csp_status st = async_checked(L, s);
    if (st != CSP_OK) return st;
    st = restructure_gradient(L, n_prune, dY, X, B, regrow_word(L, regrow_value), s);
    if (st == CSP_OK && n_prune > 0) st = build_tiles(L, s);
    if (st == CSP_OK && n_prune > 0) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) st = hip_error(e, "restructure_grad");
    }
    if (st != CSP_OK) L->broken = true;
    return st;
}

csp_status restructure_async(sparse_layer_t L, int64_t n_prune, uint64_t seed, uint64_t *step_dev, float regrow_value,
                             void *stream)
{
    if (!L || !step_dev) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to restructure_async");
    if (n_prune < 0 || n_prune > L->nnz)
        return set_error(CSP_ERR_INVALID_ARG, "n_prune %lld outside [0, nnz = %lld]", (long long)n_prune,
                         (long long)L->nnz);
    if (!L->ws.bitmap)
        return set_error(CSP_ERR_INVALID_ARG, "restructure_async needs the position bitmaps (out * in < 2^32 and "
                                              "bitmaps within 1 GiB); use restructure");
    if (n_prune > 0 && async_batch(L, n_prune) == 0)
        return set_error(CSP_ERR_INVALID_ARG, "restructure_async: %lld regrow candidates do not fit one batch; use "
                                              "restructure", (long long)n_prune);
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    if (n_prune == 0) return CSP_OK;
    hipStream_t s = (hipStream_t)stream;
    if (stream_capturing(s)) {
        if (L->tasks_in_graph)
            return set_error(CSP_ERR_INVALID_ARG, "restructure_async cannot be captured on a layer with captured "
                                                  "calls that read its task lists (their launch sizes would go "
                                                  "stale at its replays)");
        L->async_in_graph = true;
    }
    csp_status st = restructure_bitmap_async(L, n_prune, seed, step_dev, regrow_word(L, regrow_value), s);
    if (st == CSP_OK) st = build_tiles(L, s);
    if (st == CSP_OK) L->counts_stale = true;
    else L->broken = true;
    return st;
}

csp_status sparse_layer_sync(sparse_layer_t L, void *stream)
{
    if (!L) return set_error(CSP_ERR_INVALID_ARG, "NULL layer");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    if (!g.ok) return set_error(CSP_ERR_HIP, "cannot select the layer's device");
    hipStream_t s = (hipStream_t)stream;
    if (stream_capturing(s)) {  // nothing is launched: only a layer with nothing pending passes
        if (L->counts_stale || L->tasks_pending || L->async_in_graph)
            return set_error(CSP_ERR_INVALID_ARG, "sparse_layer_sync cannot run under stream capture");
        return CSP_OK;
    }
    return tasks_ready(L, s);
}

int64_t sparse_layer_nnz(sparse_layer_t L) { return L ? L->nnz : -1; }

csp_status sparse_layer_shape(sparse_layer_t L, int64_t *out_features, int64_t *in_features, int32_t *dtype)
{
    if (!L || !out_features || !in_features || !dtype) return set_error(CSP_ERR_INVALID_ARG, "NULL argument");
    *out_features = L->out;
    *in_features = L->in;
    *dtype = L->dtype;
    return CSP_OK;
}

csp_status sparse_layer_export(sparse_layer_t L, int32_t *rows, int32_t *cols, void *vals, void *stream)
{
    if (!L) return set_error(CSP_ERR_INVALID_ARG, "NULL layer");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    hipStream_t s = (hipStream_t)stream;
    const size_t n = (size_t)L->nnz;
    if (n == 0) return CSP_OK;
    if (rows) CSP_HIP(hipMemcpyAsync(rows, L->rows, 4 * n, hipMemcpyDeviceToDevice, s));
    if (cols) CSP_HIP(hipMemcpyAsync(cols, L->cols, 4 * n, hipMemcpyDeviceToDevice, s));
    if (vals) CSP_HIP(hipMemcpyAsync(vals, L->vals, (size_t)L->esz * n, hipMemcpyDeviceToDevice, s));
    return CSP_OK;
}

csp_status sparse_layer_export_index(sparse_layer_t L, int32_t *row_ptr, int32_t *perm_c, int32_t *rows_by_col,
                                     int32_t *col_ptr, void *stream)
{
    if (!L) return set_error(CSP_ERR_INVALID_ARG, "NULL layer");
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    hipStream_t s = (hipStream_t)stream;
    const size_t n = (size_t)L->nnz;
    if (row_ptr) CSP_HIP(hipMemcpyAsync(row_ptr, L->row_ptr, 4 * (size_t)(L->out + 1), hipMemcpyDeviceToDevice, s));
    if (col_ptr) CSP_HIP(hipMemcpyAsync(col_ptr, L->col_ptr, 4 * (size_t)(L->in + 1), hipMemcpyDeviceToDevice, s));
    if (n == 0) return CSP_OK;
    if (perm_c) CSP_HIP(hipMemcpyAsync(perm_c, L->perm_c, 4 * n, hipMemcpyDeviceToDevice, s));
    if (rows_by_col) CSP_HIP(hipMemcpyAsync(rows_by_col, L->rows_by_col, 4 * n, hipMemcpyDeviceToDevice, s));
    return CSP_OK;
}

csp_status sparse_layer_set_values(sparse_layer_t L, const void *vals, void *stream)
{
    if (!L) return set_error(CSP_ERR_INVALID_ARG, "NULL layer");
    if (L->nnz == 0) return CSP_OK;
    DeviceGuard g(L->device);
    CSP_USABLE(L);
    hipStream_t s = (hipStream_t)stream;
    if (vals)
        CSP_HIP(hipMemcpyAsync(L->vals, vals, (size_t)L->esz * (size_t)L->nnz, hipMemcpyDeviceToDevice, s));
    return refresh_column_values(L, s);
}

void *sparse_layer_values(sparse_layer_t L) { return L ? L->vals : nullptr; }

csp_status sparse_layer_time_next(sparse_layer_t L, void *ev_before, void *ev_after)
{
    if (!L || !ev_before || !ev_after) return set_error(CSP_ERR_INVALID_ARG, "NULL argument to sparse_layer_time_next");
    L->time_before = (hipEvent_t)ev_before;
    L->time_after = (hipEvent_t)ev_after;
    return CSP_OK;
}

const char *sparse_layer_last_error(void) { return g_last_error; }

}  // extern "C"
