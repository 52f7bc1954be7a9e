/*
 * parallel.c -- all-core CPU baseline of the truly sparse COO layer.
 *
 * BENCHMARK INFRASTRUCTURE ONLY: only the cpu_baseline leg of bench.py and
 * its CPU test load it.  It is not the oracle (oracle.c accumulates in fp64
 * on one core and is what parity is checked against) and shares no code with
 * it or with the HIP library.  It times the plain loops of the layer's three
 * products with fp32 accumulation, spread over all host cores with OpenMP, as
 * a reported baseline beside the GPU figures.
 *
 * Source of the method: "Beyond Masked Sparsity: SNACK Enables Truly Sparse
 * Neural Networks on GPU" (arXiv:2610.04093), Abstract: the layer stores only
 * its non-zero connections (COO) and runs the forward product and both
 * gradients on that storage.
 *
 *   forward      Y[b,r]  = sum_{k in row r} v_k X[b,col_k]     parallel over rows
 *   input grad   dX[b,c] = sum_{k in col c} v_k dY[b,row_k]    parallel over columns (col_ptr view)
 *   value grad   dW_k    = sum_b dY[b,row_k] X[b,col_k]        parallel over rows
 *
 * Inputs are the canonical arrays: row_ptr[out+1], cols[nnz], vals[nnz] in
 * (row, col) order; col_ptr[in+1], perm_c[nnz], rows_by_col[nnz] for the
 * transposed view.  Dense operands are row-major fp32; each call first copies
 * the operand it gathers to the batch-minor layout (in parallel, inside the
 * timed call), so the loops read contiguous runs.
 */
#include <omp.h>
#include <stdint.h>

int par_threads(void) { return omp_get_max_threads(); }

/* t[c * B + b] = a[b * n + c]: a dense operand to the batch-minor layout, so that the B values one
 * stored entry needs are contiguous (the loops below then read whole cache lines). */
static void to_batch_minor(int64_t B, int64_t n, const float *a, float *t)
{
#pragma omp parallel for schedule(static)
    for (int64_t c0 = 0; c0 < n; c0 += 64) {
        const int64_t c1 = c0 + 64 < n ? c0 + 64 : n;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t c = c0; c < c1; ++c) t[c * B + b] = a[b * n + c];
    }
}

/* Each call takes row-major operands and a scratch buffer of max(out, in) * B floats per
 * transposed operand; acc_all holds nthreads * B floats of per-thread accumulators.  Results are
 * row-major. */
void par_spmm_fwd(int64_t out, int64_t in, int64_t B, const int32_t *row_ptr, const int32_t *cols,
                  const float *vals, const float *X, float *Y, float *acc_all, float *Xt)
{
    to_batch_minor(B, in, X, Xt);
#pragma omp parallel
    {
        float *acc = acc_all + (int64_t)omp_get_thread_num() * B;
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < out; ++r) {
            for (int64_t b = 0; b < B; ++b) acc[b] = 0.f;
            for (int32_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
                const float v = vals[k];
                const float *x = Xt + (int64_t)cols[k] * B;
                for (int64_t b = 0; b < B; ++b) acc[b] += v * x[b];
            }
            for (int64_t b = 0; b < B; ++b) Y[b * out + r] = acc[b];
        }
    }
}

void par_spmm_bwd_input(int64_t out, int64_t in, int64_t B, const int32_t *col_ptr, const int32_t *perm_c,
                        const int32_t *rows_by_col, const float *vals, const float *dY, float *dX, float *acc_all,
                        float *dYt)
{
    to_batch_minor(B, out, dY, dYt);
#pragma omp parallel
    {
        float *acc = acc_all + (int64_t)omp_get_thread_num() * B;
#pragma omp for schedule(dynamic, 64)
        for (int64_t c = 0; c < in; ++c) {
            for (int64_t b = 0; b < B; ++b) acc[b] = 0.f;
            for (int32_t j = col_ptr[c]; j < col_ptr[c + 1]; ++j) {
                const float v = vals[perm_c[j]];
                const float *g = dYt + (int64_t)rows_by_col[j] * B;
                for (int64_t b = 0; b < B; ++b) acc[b] += v * g[b];
            }
            for (int64_t b = 0; b < B; ++b) dX[b * in + c] = acc[b];
        }
    }
}

void par_spmm_bwd_values(int64_t out, int64_t in, int64_t B, const int32_t *row_ptr, const int32_t *cols,
                         const float *dY, const float *X, float *dW, float *dYt, float *Xt)
{
    to_batch_minor(B, out, dY, dYt);
    to_batch_minor(B, in, X, Xt);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < out; ++r) {
        const float *g = dYt + r * B;
        for (int32_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
            const float *x = Xt + (int64_t)cols[k] * B;
            float s = 0.f;
            for (int64_t b = 0; b < B; ++b) s += g[b] * x[b];
            dW[k] = s;
        }
    }
}
