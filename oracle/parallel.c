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
 * transposed view.  Dense operands are row-major fp32.  acc is a caller
 * buffer of nthreads * B floats (per-thread accumulators).
 */
#include <omp.h>
#include <stdint.h>

int par_threads(void) { return omp_get_max_threads(); }

void par_spmm_fwd(int64_t out, int64_t in, int64_t B, const int32_t *row_ptr, const int32_t *cols,
                  const float *vals, const float *X, float *Y, float *acc_all)
{
#pragma omp parallel
    {
        float *acc = acc_all + (int64_t)omp_get_thread_num() * B;
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < out; ++r) {
            for (int64_t b = 0; b < B; ++b) acc[b] = 0.f;
            for (int32_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
                const float v = vals[k];
                const int64_t c = cols[k];
                for (int64_t b = 0; b < B; ++b) acc[b] += v * X[b * in + c];
            }
            for (int64_t b = 0; b < B; ++b) Y[b * out + r] = acc[b];
        }
    }
}

void par_spmm_bwd_input(int64_t out, int64_t in, int64_t B, const int32_t *col_ptr, const int32_t *perm_c,
                        const int32_t *rows_by_col, const float *vals, const float *dY, float *dX, float *acc_all)
{
#pragma omp parallel
    {
        float *acc = acc_all + (int64_t)omp_get_thread_num() * B;
#pragma omp for schedule(dynamic, 64)
        for (int64_t c = 0; c < in; ++c) {
            for (int64_t b = 0; b < B; ++b) acc[b] = 0.f;
            for (int32_t j = col_ptr[c]; j < col_ptr[c + 1]; ++j) {
                const float v = vals[perm_c[j]];
                const int64_t r = rows_by_col[j];
                for (int64_t b = 0; b < B; ++b) acc[b] += v * dY[b * out + r];
            }
            for (int64_t b = 0; b < B; ++b) dX[b * in + c] = acc[b];
        }
    }
}

void par_spmm_bwd_values(int64_t out, int64_t in, int64_t B, const int32_t *row_ptr, const int32_t *cols,
                         const float *dY, const float *X, float *dW)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < out; ++r) {
        for (int32_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
            const int64_t c = cols[k];
            float s = 0.f;
            for (int64_t b = 0; b < B; ++b) s += dY[b * out + r] * X[b * in + c];
            dW[k] = s;
        }
    }
}
