/*
 * coospmm.h -- C ABI of the truly sparse COO layer for AMD MI355X (gfx950).
 *
 * Method: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks
 * on GPU" (arXiv:2610.04093), Abstract.  The page describes a layer that keeps
 * only the non-zero connections of a weight matrix, in COO form, computes the
 * forward product and the backward gradients on that sparse storage alone (no
 * dense weight tensor and no mask), and offers an API to restructure the
 * connections during dynamic sparse training.  It prints no formulas; this
 * header states the definitions the library implements.
 *
 * Notation.  W has out_features rows and in_features columns and is stored as
 * nnz triples (row_k, col_k, v_k).  Dense operands are row-major, contiguous:
 *   X, dX : [B, in_features]      Y, dY : [B, out_features]
 *
 * Conventions shared by every call:
 *   - Device pointers unless stated otherwise; all arrays must be 4-byte
 *     aligned (values of a bf16 layer: 2-byte aligned).
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue their kernels on it and return without waiting, except
 *     where a call says it synchronizes.
 *   - Outputs are overwritten, never accumulated into.
 *   - Errors are returned as a negative csp_status; nothing aborts.  The text
 *     of the last error of the calling thread is sparse_layer_last_error().
 *   - A layer must not be used by two streams at the same time.
 *   - Index limits: out_features, in_features, nnz < 2^31; B >= 1.
 */
#ifndef COOSPMM_H
#define COOSPMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct csp_layer *sparse_layer_t;

typedef enum {
    CSP_OK = 0,
    CSP_ERR_INVALID_ARG = -1, /* bad pointer, size or count (checked on the host, before any launch) */
    CSP_ERR_INDEX_RANGE = -2, /* a row or column index outside the layer (found on the device) */
    CSP_ERR_DUPLICATE = -3,   /* a (row, col) pair given twice (found on the device) */
    CSP_ERR_NO_MEMORY = -4,   /* a device allocation failed */
    CSP_ERR_HIP = -5,         /* a HIP runtime call failed */
    CSP_ERR_DTYPE = -6        /* the call does not support the layer's value type */
} csp_status;

typedef enum {
    CSP_F32 = 0, /* fp32 values and activations, fp32 accumulation */
    CSP_BF16 = 1 /* bf16 values and activations, fp32 accumulation, bf16 output */
} csp_dtype;

/* Activation of the fused epilogues: GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)). */
typedef enum {
    CSP_ACT_NONE = 0,
    CSP_ACT_GELU = 1
} csp_act;

/*
 * sparse_layer_create -- build a layer from COO triples (the page's COO
 * weight storage, Abstract).
 *   rows[nnz], cols[nnz] : int32 device arrays, any order, 0 <= row < out,
 *                          0 <= col < in, no repeated (row, col) pair.
 *   vals[nnz]            : device array of dtype.
 * The layer copies the triples into memory it owns and puts them in canonical
 * order: sorted by (row, col).  It also builds row offsets, and the transposed
 * view (canonical indices sorted by (col, row)) used by the input gradient.
 * nnz = 0 is valid.  Synchronizes on "stream" once, to read the validation
 * result; returns CSP_ERR_INDEX_RANGE or CSP_ERR_DUPLICATE without creating a
 * layer when the triples are invalid.  On success *out_layer owns device
 * memory until sparse_layer_destroy: the COO arrays and their index, the
 * restructure state, and the product workspace -- two batch-minor operand
 * copies of max(out, in) * 64 elements and 64 fp32 partial sums per task --
 * so that no product call allocates (batches above 64 rows run as
 * consecutive slices of 64 rows).
 */
csp_status sparse_layer_create(int64_t out_features, int64_t in_features, int64_t nnz, const int32_t *rows,
                               const int32_t *cols, const void *vals, csp_dtype dtype, void *stream,
                               sparse_layer_t *out_layer);

/* Frees the layer's device memory (waits for the device first).  NULL is a no-op. */
void sparse_layer_destroy(sparse_layer_t layer);

/*
 * spmm_fwd -- forward product of the sparse layer (Abstract: the layer
 * computes only its stored connections):
 *     Y[b, r] = sum over stored k with row_k = r of v_k * X[b, col_k]
 * i.e. Y = X W^T.  X [B, in] and Y [B, out] have the layer's dtype.  A row
 * with no stored entry gives exactly 0.  fp32 accumulation in any order.
 * This and the other product calls (spmm_bwd_input, spmm_bwd_values,
 * spmm_bwd and their _act forms) are asynchronous on "stream", allocate
 * nothing, set no memory with memset, and may be captured in a HIP graph.
 */
csp_status spmm_fwd(sparse_layer_t layer, const void *X, int64_t B, void *Y, void *stream);

/*
 * spmm_fwd_static -- spmm_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments as spmm_fwd, and its task-list kernels, but the
 * call's workspace -- the batch-minor copy of X and the partial sums of rows
 * split over several tasks -- lives in one static device array of 16 MiB per
 * GPU (held until the process ends) instead of the layer's own workspace.
 * Results are bit for bit those of spmm_fwd except where spmm_fwd takes its
 * LDS-tile path (fp32 layers with at least one 512 x 512 tile per compute
 * unit, batch slices of 33..64 rows), whose per-tile partial sums do not fit
 * the array: there both are within the fp32 bound of the exact sum and agree
 * to rounding.  The call allocates and frees nothing.  Its largest
 * batch slice (at most 64 rows) needs esz * ld * in bytes for the copy of X
 * (ld = the slice's rows rounded up to a power of two; esz = 4 for fp32, 2 for
 * bf16; none for one row, or when the forward reads X through the on-chip
 * table path) and, when some row is split over several tasks and finished in
 * a separate pass, 4 * ld bytes per task of the layer's row task list; a layer
 * and batch that need more than 16 MiB get CSP_ERR_INVALID_ARG before any
 * launch (use spmm_fwd).  Nothing in the array
 * needs to start at zero.  All calls on one GPU share its array: calls that
 * overlap on one GPU (two streams, or two host threads) race and give wrong
 * results; serialize them.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) once.
 */
csp_status spmm_fwd_static(sparse_layer_t layer, const void *X, int64_t B, void *Y, void *stream);

/*
 * spmm_bwd_input -- gradient with respect to the layer input (Abstract:
 * gradients are backpropagated on the sparse storage):
 *     dX[b, c] = sum over stored k with col_k = c of v_k * dY[b, row_k]
 * i.e. dX = dY W.  dY [B, out], dX [B, in], both in the layer's dtype
 * (bf16 layers: bf16 in and out, fp32 accumulation).
 */
csp_status spmm_bwd_input(sparse_layer_t layer, const void *dY, int64_t B, void *dX, void *stream);

/*
 * spmm_bwd_values -- gradient with respect to the stored values only
 * (Abstract: the layer backpropagates its gradients entirely on the sparse
 * storage, so the weight gradient exists only at the stored connections), a
 * sampled dense-dense product:
 *     dW[k] = sum_b dY[b, row_k] * X[b, col_k]   for every stored k
 * dW [nnz] is fp32 and in canonical (row, col) order (the order of
 * sparse_layer_export and sparse_layer_values).  dY and X have the layer's
 * dtype (bf16 products are exact in fp32); dW is fp32 for either dtype.
 */
csp_status spmm_bwd_values(sparse_layer_t layer, const void *dY, const void *X, int64_t B, float *dW,
                           void *stream);

/*
 * spmm_bwd -- both gradients of one backward step in a single pass over the
 * transposed view: dX as in spmm_bwd_input and dW as in spmm_bwd_values, with
 * each gathered dY row used for both.  Same layouts, dtypes and results
 * (within the tolerance of each) as the two separate calls.
 */
csp_status spmm_bwd(sparse_layer_t layer, const void *dY, const void *X, int64_t B, void *dX, float *dW,
                    void *stream);

/*
 * Fused epilogues for a stack of layers with an activation between them (the
 * page reports end-to-end GPT-2 training with truly sparse layers, Abstract;
 * its MLP block is linear -> GELU -> linear).  The activation is applied where
 * the segment sum is stored, so it costs no extra pass over the activations.
 *
 * spmm_fwd_act -- Y = act(X W^T + bias), computed in fp32 from the fp32 sum:
 *   bias [out] in the layer dtype, or NULL for none;
 *   act  CSP_ACT_NONE or CSP_ACT_GELU (else CSP_ERR_INVALID_ARG);
 *   H    [B, out] in the layer dtype, or NULL: receives the pre-activation
 *        X W^T + bias (what the backward needs); must not overlap Y.
 */
csp_status spmm_fwd_act(sparse_layer_t layer, const void *X, int64_t B, const void *bias, csp_act act, void *Y,
                        void *H, void *stream);

/*
 * spmm_bwd_input_act -- the input gradient times the derivative of the
 * activation that produced this layer's input:
 *     dX = (dY W) * act'(H_in)   (elementwise; GELU'(x) = Phi(x) + x phi(x))
 * H_in [B, in] is that activation's input (the previous layer's H), layer
 * dtype; required for CSP_ACT_GELU, ignored for CSP_ACT_NONE (then this is
 * spmm_bwd_input).
 */
csp_status spmm_bwd_input_act(sparse_layer_t layer, const void *dY, int64_t B, csp_act act, const void *H_in,
                              void *dX, void *stream);

/* spmm_bwd_act -- spmm_bwd with the input gradient of spmm_bwd_input_act; dW is unchanged. */
csp_status spmm_bwd_act(sparse_layer_t layer, const void *dY, const void *X, int64_t B, csp_act act,
                        const void *H_in, void *dX, float *dW, void *stream);

/*
 * Batch-minor operands.  For 2 <= B <= 64 the products gather their dense
 * operand through a batch-minor copy: T[c * ld + b] = A[b, c] for b < B,
 * where ld is the smallest power of two >= B and the pad slots B <= b < ld
 * hold zeros.  The calls below let a caller keep such copies and hand them
 * from one call to the next instead of each call making its own (one launch
 * per operand): a producing call writes its output's copy beside the
 * row-major output, and a consuming call takes it.  This is how a layer
 * chain (the page's GPT-2 training with truly sparse layers, Abstract) avoids
 * re-laying out every activation.  Copies are device arrays [n][ld] of the
 * layer dtype, caller-owned.  A call writes slots b < B of an output copy; the
 * caller keeps its pad slots zero (e.g. a buffer zeroed once, reused at the
 * same B).  Results are bitwise those of the plain calls.
 */

/* spmm_batch_minor -- T = the batch-minor copy of the row-major [B, n]
 * array src (dtype CSP_F32 or CSP_BF16), pad slots written as zeros.
 * 2 <= B <= 64, else CSP_ERR_INVALID_ARG.  Asynchronous on stream. */
csp_status spmm_batch_minor(const void *src, int64_t n, int64_t B, int32_t dtype, void *dst, void *stream);

/* spmm_fwd_bm -- spmm_fwd_act (bias and act optional: with neither, and no
 * H, exactly spmm_fwd) for 2 <= B <= 64, with
 *   XT  the batch-minor copy of X, or NULL (the call makes its own; X itself
 *       is always passed: some paths read it row-major);
 *   YT  NULL, or [out][ld]: also receives Y's batch-minor copy. */
csp_status spmm_fwd_bm(sparse_layer_t layer, const void *X, const void *XT, int64_t B, const void *bias, csp_act act,
                       void *Y, void *H, void *YT, void *stream);

/* spmm_bwd_bm -- spmm_bwd_act (act CSP_ACT_NONE: exactly spmm_bwd) for
 * 2 <= B <= 64, with dYT and XT the batch-minor copies of dY and X, or NULL,
 * and dXT NULL or [in][ld]: also receives dX's batch-minor copy (the next
 * layer down takes it as its dYT). */
csp_status spmm_bwd_bm(sparse_layer_t layer, const void *dY, const void *dYT, const void *X, const void *XT, int64_t B,
                       csp_act act, const void *H_in, void *dX, void *dXT, float *dW, void *stream);

/*
 * restructure -- one prune-and-regrow step of dynamic sparse training
 * (Abstract: an API for restructuring connections).  The rule:
 *  1. prune the n_prune stored entries with the smallest |v|, ordered by the
 *     bit pattern of |v| (so +0 = -0 and NaN sorts above +inf), ties broken
 *     by canonical index;
 *  2. regrow n_prune entries, value regrow_value, at positions that are empty
 *     after the prune (a just-pruned position may come back).  Candidates come
 *     from a counter-based stream: candidate i is word (i mod 4) of the
 *     Philox4x64-10 block with counter (i div 4, step, 0, 0) and key
 *     (seed, 0), mapped to position floor(u * out * in / 2^64) = row * in +
 *     col; walking i = 0, 1, 2, ..., a candidate is taken when its position
 *     is empty and not taken before, until n_prune are taken;
 *  3. restore canonical order and rebuild offsets and the transposed view.
 * nnz is unchanged, and the result is a pure function of (layer contents,
 * n_prune, seed, step, regrow_value).  0 <= n_prune <= nnz, else
 * CSP_ERR_INVALID_ARG.  Synchronizes on "stream" (it reads back how many
 * candidates were accepted and the new task counts; usually once).
 * regrow_value is rounded to the layer's dtype.  The layer may move its
 * canonical arrays to other buffers of its own: pointers obtained from
 * sparse_layer_values before the call are stale afterwards, and work captured
 * in a graph before it must be captured again.
 */
csp_status restructure(sparse_layer_t layer, int64_t n_prune, uint64_t seed, uint64_t step, float regrow_value,
                       void *stream);

/*
 * restructure_grad -- prune-and-regrow with gradient-informed regrowth (the
 * page's Abstract restructures connections during dynamic sparse training and
 * fixes no regrow rule; this variant ranks the empty positions by the
 * magnitude of the dense weight gradient, the quantity the value gradient
 * computes at the stored positions only).
 *  1. prune exactly as restructure (the n_prune smallest |v|);
 *  2. every position (r, c) empty after the prune gets the score |s| with
 *         s = 0; for b = 0 .. B-1: s = fmaf(dY[b, r], X[b, c], s)
 *     in fp32 (bf16 operands widen exactly), a fused-multiply-add chain in
 *     batch order so that the result is reproducible bit for bit;
 *  3. the n_prune empty positions with the largest scores are regrown with
 *     value regrow_value, ties (equal fp32 scores) to the smaller r * in + c;
 *  4. canonical order, offsets and the transposed view are rebuilt.
 * dY [B, out] and X [B, in] have the layer's dtype.  Layers whose position
 * bitmaps do not fit (out * in >= 2^32, or more than 1 GiB) return
 * CSP_ERR_INVALID_ARG.  The first call allocates the score workspace
 * (4 bytes per position).  Synchronizes on "stream"; pointers from
 * sparse_layer_values are stale afterwards, as after restructure.
 */
csp_status restructure_grad(sparse_layer_t layer, int64_t n_prune, const void *dY, const void *X, int64_t B,
                            float regrow_value, void *stream);

/*
 * restructure_async -- the step of restructure (same rule, same result bit
 * for bit for the same seed and step) enqueued on "stream" with no host
 * synchronization and no allocation, so that a dynamic-sparse-training step
 * (products, optimizer update, restructure) can be captured in one HIP graph
 * (Abstract: restructuring connections during dynamic sparse training).
 *   step_dev  device pointer to a uint64 step counter: the call draws its
 *             candidates with step *step_dev and then adds 1 to it on the
 *             device, so every replay of a captured call draws a new stream.
 * Differences from restructure:
 *  - layers with position bitmaps only (out * in < 2^32, bitmaps within
 *    1 GiB), and n_prune whose candidates fit one batch; else
 *    CSP_ERR_INVALID_ARG before anything is enqueued;
 *  - one batch of candidates, about 1.2 times the expected need plus 4096:
 *    should it hold fewer than n_prune empty, first-seen positions (a
 *    deviation of hundreds of standard deviations for layers of 10^5
 *    entries and more), a device flag is set, and the next call that
 *    synchronizes on the layer (sparse_layer_sync, or a call that needs the
 *    task lists) returns CSP_ERR_INVALID_ARG and refuses the layer;
 *  - the canonical arrays stay in the layer's own buffers (values are written
 *    back, not moved): sparse_layer_values pointers and captured graphs
 *    remain valid;
 *  - the host-side task-list counts are read back later, by the first call
 *    that needs them (a product outside the LDS-tile path, spmm_fwd_static,
 *    restructure, restructure_grad) or by sparse_layer_sync.  Such a call on
 *    a stream under capture returns CSP_ERR_INVALID_ARG instead: call
 *    sparse_layer_sync before capturing it.  The LDS-tile products
 *    (fp32 layers with tiles, batch chunks of 33..64 rows) need no counts;
 *  - on a layer with LDS tiles the task lists themselves are not rebuilt
 *    either: the first product outside the LDS-tile path, spmm_fwd_static or
 *    sparse_layer_sync builds them on "stream" before reading the counts (a
 *    restructure or restructure_grad rebuilds them itself);
 *  - once captured, it may change the layer at any replay, which the host
 *    cannot follow: from then on every call that needs the task lists
 *    rebuilds them (layers with tiles) and reads them back first, and such a
 *    call cannot itself be captured (CSP_ERR_INVALID_ARG).  Capturing it on
 *    a layer with such a call already captured is refused the same way,
 *    since that call's launch sizes would go stale.
 * Calls on one layer must be ordered on one stream, as for every call.
 */
csp_status restructure_async(sparse_layer_t layer, int64_t n_prune, uint64_t seed, uint64_t *step_dev,
                             float regrow_value, void *stream);

/*
 * sparse_layer_sync -- completes the bookkeeping of earlier restructure_async
 * calls: builds the task lists they left pending, synchronizes on "stream",
 * reads back the task-list counts and the short-regrow flag
 * (CSP_ERR_INVALID_ARG, and the layer refused, if set).
 * Returns at once when nothing is pending.  Not for use under capture.
 */
csp_status sparse_layer_sync(sparse_layer_t layer, void *stream);

/* Number of stored entries; -1 for NULL. */
int64_t sparse_layer_nnz(sparse_layer_t layer);
/* Shape and dtype; returns CSP_ERR_INVALID_ARG for NULL arguments. */
csp_status sparse_layer_shape(sparse_layer_t layer, int64_t *out_features, int64_t *in_features, int32_t *dtype);

/*
 * sparse_layer_export -- copy the canonical triples into caller device arrays
 * rows[nnz], cols[nnz] (int32) and vals[nnz] (layer dtype).  Any pointer may
 * be NULL to skip that array.
 */
csp_status sparse_layer_export(sparse_layer_t layer, int32_t *rows, int32_t *cols, void *vals, void *stream);

/*
 * sparse_layer_export_index -- copy the derived index arrays into caller
 * device arrays: row_ptr[out+1] (first canonical index of each row),
 * perm_c[nnz] (canonical indices in (col, row) order), rows_by_col[nnz]
 * (row of each perm_c entry) and col_ptr[in+1] (first perm_c position of each
 * column).  Any pointer may be NULL.
 */
csp_status sparse_layer_export_index(sparse_layer_t layer, int32_t *row_ptr, int32_t *perm_c,
                                     int32_t *rows_by_col, int32_t *col_ptr, void *stream);

/*
 * sparse_layer_values -- device pointer to the layer's canonical values
 * (nnz elements of the layer dtype), for in-place optimizer updates between
 * calls.  Valid until the next restructure or the layer's destruction
 * (restructure may move the values: ask again afterwards).  NULL for a NULL
 * layer.  The input-gradient pass reads a
 * column-ordered copy of the values: after writing through this pointer,
 * call sparse_layer_set_values(layer, NULL, stream) before the next
 * spmm_bwd_input or spmm_bwd.
 */
void *sparse_layer_values(sparse_layer_t layer);

/*
 * sparse_layer_set_values -- overwrite the canonical values with vals[nnz]
 * (device array of the layer dtype, canonical order), e.g. after an
 * optimizer step kept outside the library, and refresh the column-ordered
 * copy.  vals = NULL only refreshes the copy (values already changed in
 * place).  Structure is unchanged.  Asynchronous on stream.
 */
csp_status sparse_layer_set_values(sparse_layer_t layer, const void *vals, void *stream);

/*
 * sparse_layer_time_next -- profiling aid: the next product call on this
 * layer (spmm_fwd, spmm_bwd_input, spmm_bwd_values, spmm_bwd or their _act
 * forms) attaches ev_before and ev_after to the dispatch of its main kernel
 * (hipExtLaunchKernel), so hipEventElapsedTime(ev_before, ev_after) is that
 * kernel's own duration; then the request is forgotten.  When the pass has
 * two main kernels (input gradient and value gradient as separate launches
 * for large operand tables) the pair spans both.  The events are
 * caller-owned hipEvent_t handles passed as void*.  Operand copies and other
 * helper kernels of the call fall outside.  Not for use under graph capture.
 */
csp_status sparse_layer_time_next(sparse_layer_t layer, void *ev_before, void *ev_after);

/* Text of the calling thread's last error ("" if none). */
const char *sparse_layer_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* COOSPMM_H */
