/*
 * oracle.c -- plain, slow CPU oracle for the truly sparse COO layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library; the two are written separately from the same
 * definitions.
 *
 * Source of the method: "Beyond Masked Sparsity: SNACK Enables Truly Sparse
 * Neural Networks on GPU" (arXiv:2610.04093), Abstract.  The page describes a
 * layer that keeps only the non-zero connections of W in COO form, runs the
 * forward product and both backward gradients on that sparse storage alone,
 * and lets dynamic sparse training restructure (prune and regrow) the
 * connections.  The page prints no formulas; the definitions below are the
 * plain reading of that description:
 *
 *   W is out x in, stored as triples (row_k, col_k, v_k), k = 0..nnz-1.
 *   forward      Y[b,r]  = sum_{k: row_k = r} v_k * X[b,col_k]     (Y = X W^T)
 *   input grad   dX[b,c] = sum_{k: col_k = c} v_k * dY[b,row_k]    (dX = dY W)
 *   value grad   dW_k    = sum_b dY[b,row_k] * X[b,col_k]          (stored k only)
 *
 * Arithmetic: every product of two fp32 (or bf16) numbers is exact in fp64,
 * and sums are accumulated in fp64.  Each output also gets S = sum |term|,
 * the magnitude sum that the comparison tolerance is scaled by.
 *
 * Parity pins (checked by the CPU tests, never by this file): dense matmul of
 * the densified W on tiny inputs, bit-identity with a naive dense loop at 0%
 * sparsity, exactness on integer-valued inputs, the adjoint identity
 * <dY, X W^T> = <dY W, X> = <dW, v>, finite differences, special cases
 * (permutation W, single nnz, empty layer), brute-force sorting for the
 * canonical order, restructure invariants plus an independent set-based
 * re-implementation driven by numpy's own Philox generator, the
 * gradient-informed regrow against integer-valued brute force (exact scores,
 * many ties) plus its ranking invariants, Philox blocks
 * against numpy.random.Philox, bf16 decoding against torch, and GELU against
 * scipy's erf.  Every exported function is pinned; none is "parity unpinned".
 *
 * Mutation hooks: building with -DORACLE_MUTANT=<n> plants one plausible
 * mistake (see MUTANT() uses below).  The CPU tests build each mutant and
 * require that at least one pin rejects it.  The default build has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUTANT(n) (ORACLE_MUTANT == (n))

enum { OR_OK = 0, OR_ERR_ARG = -1, OR_ERR_RANGE = -2, OR_ERR_DUP = -3, OR_ERR_NOMEM = -4 };
enum { OR_F32 = 0, OR_BF16 = 1 };

/* ------------------------------------------------------------------ */
/* Value decoding.  fp32 words are reinterpreted; a bf16 word is the top */
/* half of an fp32 word (sign, 8 exponent bits, 7 fraction bits), so it  */
/* widens exactly by a 16-bit left shift.                                */
/* ------------------------------------------------------------------ */
static double word_to_double(const void *base, int dtype, int64_t i)
{
    float f;
    uint32_t w;
    if (dtype == OR_BF16)
        w = (uint32_t)((const uint16_t *)base)[i] << 16;
    else
        w = ((const uint32_t *)base)[i];
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

double oracle_decode(const void *base, int dtype, int64_t i) { return word_to_double(base, dtype, i); }

static int elem_bytes(int dtype) { return dtype == OR_BF16 ? 2 : 4; }

/* ------------------------------------------------------------------ */
/* Canonical order.  Entries are ordered by (row, col); the transposed   */
/* view orders the canonical indices by (col, row).  Both are total      */
/* orders once duplicates are rejected, so the result is unique.         */
/* ------------------------------------------------------------------ */
typedef struct {
    int64_t a, b; /* primary, secondary key */
    int64_t idx;  /* position in the input  */
} triple_t;

static int cmp_triple(const void *pa, const void *pb)
{
    const triple_t *x = (const triple_t *)pa, *y = (const triple_t *)pb;
    if (x->a != y->a) return x->a < y->a ? -1 : 1;
    if (x->b != y->b) return x->b < y->b ? -1 : 1;
    if (x->idx != y->idx) return x->idx < y->idx ? -1 : 1;
    return 0;
}

/*
 * oracle_canonicalize: validate and order a COO triple list.
 *   rows, cols, vals : input triples in any order (vals as raw fp32/bf16 words)
 *   src[nnz]         : canonical position -> input position
 *   rows_c, cols_c, vals_c[nnz] : triples in (row, col) order; values moved bit-exactly
 *   row_ptr[out+1]   : first canonical index of each row (row_ptr[out] = nnz)
 *   perm_c[nnz]      : canonical indices ordered by (col, row)
 *   rows_by_col[nnz] : rows_c[perm_c[j]]
 *   col_ptr[in+1]    : first position in perm_c of each column
 * Returns OR_ERR_RANGE for an index outside [0,out) x [0,in), OR_ERR_DUP when a
 * (row, col) pair repeats.  Any output pointer may be NULL.
 */
int oracle_canonicalize(int64_t out, int64_t in, int64_t nnz, const int32_t *rows, const int32_t *cols,
                        const void *vals, int dtype, int64_t *src, int32_t *rows_c, int32_t *cols_c,
                        void *vals_c, int32_t *row_ptr, int32_t *perm_c, int32_t *rows_by_col,
                        int32_t *col_ptr)
{
    if (out < 0 || in < 0 || nnz < 0) return OR_ERR_ARG;
    for (int64_t k = 0; k < nnz; ++k)
        if (rows[k] < 0 || rows[k] >= out || cols[k] < 0 || cols[k] >= in) return OR_ERR_RANGE;

    triple_t *t = (triple_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *t);
    if (!t) return OR_ERR_NOMEM;
    for (int64_t k = 0; k < nnz; ++k) {
        t[k].a = rows[k];
        t[k].b = cols[k];
        t[k].idx = k;
    }
    qsort(t, (size_t)nnz, sizeof *t, cmp_triple);
    for (int64_t k = 1; k < nnz; ++k)
        if (t[k].a == t[k - 1].a && t[k].b == t[k - 1].b) {
            free(t);
            return OR_ERR_DUP;
        }

    int eb = elem_bytes(dtype);
    for (int64_t k = 0; k < nnz; ++k) {
        if (src) src[k] = t[k].idx;
        if (rows_c) rows_c[k] = (int32_t)t[k].a;
        if (cols_c) cols_c[k] = (int32_t)t[k].b;
        if (vals_c) memcpy((char *)vals_c + k * eb, (const char *)vals + t[k].idx * eb, (size_t)eb);
    }
    if (row_ptr) {
        /* counts, then running sum */
        for (int64_t r = 0; r <= out; ++r) row_ptr[r] = 0;
        for (int64_t k = 0; k < nnz; ++k) row_ptr[t[k].a + 1] += 1;
        for (int64_t r = 0; r < out; ++r) row_ptr[r + 1] += row_ptr[r];
    }

    /* transposed order: canonical index k keyed by (col_k, row_k) */
    triple_t *u = (triple_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *u);
    if (!u) {
        free(t);
        return OR_ERR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        u[k].a = t[k].b;
        u[k].b = t[k].a;
        u[k].idx = k;
    }
    qsort(u, (size_t)nnz, sizeof *u, cmp_triple);
    for (int64_t j = 0; j < nnz; ++j) {
        if (perm_c) perm_c[j] = (int32_t)u[j].idx;
        if (rows_by_col) rows_by_col[j] = (int32_t)u[j].b;
    }
    if (col_ptr) {
        for (int64_t c = 0; c <= in; ++c) col_ptr[c] = 0;
        for (int64_t j = 0; j < nnz; ++j) col_ptr[u[j].a + 1] += 1;
        for (int64_t c = 0; c < in; ++c) col_ptr[c + 1] += col_ptr[c];
    }
    free(u);
    free(t);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* The three products.  They take triples in any order: the definitions */
/* do not depend on the storage order.                                   */
/* ------------------------------------------------------------------ */

/* Y[b,r] = sum_{k: row_k=r} v_k X[b,col_k];  X is [B,in], Y and S are [B,out]. */
void oracle_spmm_fwd(int64_t out, int64_t in, int64_t nnz, const int32_t *rows, const int32_t *cols,
                     const void *vals, int dtype, const void *X, int64_t B, double *Y, double *S)
{
    for (int64_t i = 0; i < B * out; ++i) {
        Y[i] = 0.0;
        if (S) S[i] = 0.0;
    }
    int64_t kend = MUTANT(2) && nnz > 0 ? nnz - 1 : nnz; /* mutant 2: drops the last term */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t k = 0; k < kend; ++k) {
            int64_t r = rows[k], c = cols[k];
            if (MUTANT(1)) { /* mutant 1: reads X through the row index */
                r = cols[k] % out;
                c = rows[k] % in;
            }
            double term = word_to_double(vals, dtype, k) * word_to_double(X, dtype, b * in + c);
            Y[b * out + r] += term;
            if (S) S[b * out + r] += fabs(term);
        }
}

/* dX[b,c] = sum_{k: col_k=c} v_k dY[b,row_k];  dY is [B,out], dX and S are [B,in]. */
void oracle_spmm_bwd_input(int64_t out, int64_t in, int64_t nnz, const int32_t *rows, const int32_t *cols,
                           const void *vals, int dtype, const void *dY, int64_t B, double *dX, double *S)
{
    for (int64_t i = 0; i < B * in; ++i) {
        dX[i] = 0.0;
        if (S) S[i] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t k = 0; k < nnz; ++k) {
            int64_t r = rows[k], c = cols[k];
            double term = word_to_double(vals, dtype, k) * word_to_double(dY, dtype, b * out + r);
            if (MUTANT(3)) term = -term; /* mutant 3: sign flip */
            dX[b * in + c] += term;
            if (S) S[b * in + c] += fabs(term);
        }
}

/* dW_k = sum_b dY[b,row_k] X[b,col_k] for every stored k; dW and S are [nnz]. */
void oracle_spmm_bwd_values(int64_t out, int64_t in, int64_t nnz, const int32_t *rows, const int32_t *cols,
                            int dtype, const void *dY, const void *X, int64_t B, double *dW, double *S)
{
    for (int64_t k = 0; k < nnz; ++k) {
        double acc = 0.0, mag = 0.0;
        int64_t r = rows[k], c = cols[k];
        if (MUTANT(4)) { /* mutant 4: transposed operand (row and col swapped) */
            r = cols[k] % out;
            c = rows[k] % in;
        }
        for (int64_t b = 0; b < B; ++b) {
            double term = word_to_double(dY, dtype, b * out + r) * word_to_double(X, dtype, b * in + c);
            acc += term;
            mag += fabs(term);
        }
        dW[k] = acc;
        if (S) S[k] = mag;
    }
}

/* ------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: */
/* as easy as 1, 2, 3", SC 2011).  One block maps a 4-word counter and a  */
/* 2-word key to 4 pseudo-random 64-bit words: ten rounds, each rounds     */
/* two 64x64->128 multiplies, with the key advanced by two Weyl constants */
/* between rounds.  Constants are the published Philox4x64 ones.          */
/* ------------------------------------------------------------------ */
static const uint64_t PHILOX_M0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t PHILOX_M1 = 0xCA5A826395121157ULL;
static const uint64_t PHILOX_W0 = 0x9E3779B97F4A7C15ULL;
static const uint64_t PHILOX_W1 = 0xBB67AE8584CAA73BULL;

void oracle_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        unsigned __int128 p0 = (unsigned __int128)PHILOX_M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)PHILOX_M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/*
 * Regrow candidate stream.  Candidate i draws word (i mod 4) of the Philox
 * block with counter (i div 4, step, 0, 0) and key (seed, 0), and maps the
 * 64-bit word u to a flat position floor(u * (out*in) / 2^64) in [0, out*in).
 */
uint64_t oracle_regrow_draw(uint64_t seed, uint64_t step, uint64_t i)
{
    uint64_t ctr[4] = {i / 4, step, 0, 0}, key[2] = {seed, 0}, w[4];
    oracle_philox4x64_10(ctr, key, w);
    return w[i % 4];
}

int64_t oracle_regrow_position(uint64_t u, int64_t out, int64_t in)
{
    unsigned __int128 prod = (unsigned __int128)u * (unsigned __int128)(uint64_t)(out * in);
    int64_t p = (int64_t)(prod >> 64);
    if (MUTANT(5)) p = (p + 1) % (out * in); /* mutant 5: off-by-one position map */
    return p;
}

/* ------------------------------------------------------------------ */
/* Restructure (dynamic sparse training step on the stored connections). */
/*                                                                       */
/* Reading adopted for the page's "restructuring connections":           */
/*  1. prune: order the canonical entries by (|v| as an unsigned bit      */
/*     pattern, canonical index) ascending and remove the first n_prune;  */
/*     +0 and -0 tie, NaN orders above +inf;                             */
/*  2. occupied = positions of the entries that were kept;               */
/*  3. walk the candidate stream i = 0, 1, 2, ...: a candidate position  */
/*     is accepted when it is not occupied, and is then marked occupied; */
/*     stop after n_prune acceptances (a just-pruned position may return);*/
/*  4. each accepted position becomes (p div in, p mod in, regrow_value);*/
/*  5. kept and new entries together are put back in canonical order.    */
/* nnz is unchanged.  Input must be canonical (sorted, no duplicates).    */
/* ------------------------------------------------------------------ */
typedef struct {
    uint32_t key;
    int64_t idx;
} absent_t;

static int cmp_absent(const void *pa, const void *pb)
{
    const absent_t *x = (const absent_t *)pa, *y = (const absent_t *)pb;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->idx != y->idx) return x->idx < y->idx ? -1 : 1;
    return 0;
}

static uint32_t magnitude_key(const void *vals, int dtype, int64_t k)
{
    if (dtype == OR_BF16) return (uint32_t)(((const uint16_t *)vals)[k] & 0x7FFFu);
    return ((const uint32_t *)vals)[k] & 0x7FFFFFFFu;
}

/*
 * Outputs rows_new, cols_new, vals_new (canonical order, nnz entries) and,
 * when non-NULL, n_draws = number of candidates consumed.  regrow_bits is
 * the raw word (fp32 or bf16 pattern) of the regrown value.
 */
int oracle_restructure(int64_t out, int64_t in, int64_t nnz, const int32_t *rows_c, const int32_t *cols_c,
                       const void *vals_c, int dtype, int64_t n_prune, uint64_t seed, uint64_t step,
                       uint32_t regrow_bits, int32_t *rows_new, int32_t *cols_new, void *vals_new,
                       int64_t *n_draws)
{
    if (n_prune < 0 || n_prune > nnz || out <= 0 || in <= 0) return OR_ERR_ARG;
    int64_t npos = out * in;
    int eb = elem_bytes(dtype);

    /* 1. prune order */
    absent_t *ord = (absent_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *ord);
    unsigned char *pruned = (unsigned char *)calloc((size_t)(nnz ? nnz : 1), 1);
    unsigned char *occ = (unsigned char *)calloc((size_t)((npos + 7) / 8), 1);
    triple_t *all = (triple_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *all);
    if (!ord || !pruned || !occ || !all) {
        free(ord);
        free(pruned);
        free(occ);
        free(all);
        return OR_ERR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        ord[k].key = magnitude_key(vals_c, dtype, k);
        if (MUTANT(6)) ord[k].key = 0x7FFFFFFFu - ord[k].key; /* mutant 6: prunes the largest */
        ord[k].idx = k;
    }
    qsort(ord, (size_t)nnz, sizeof *ord, cmp_absent);
    for (int64_t j = 0; j < n_prune; ++j) pruned[ord[j].idx] = 1;

    /* 2. occupancy bitmap of kept positions */
    int64_t m = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (pruned[k]) continue;
        int64_t p = (int64_t)rows_c[k] * in + cols_c[k];
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        all[m].a = rows_c[k];
        all[m].b = cols_c[k];
        all[m].idx = k; /* >= 0: kept entry, value from vals_c[k] */
        ++m;
    }

    /* 3-4. regrow from the candidate stream */
    uint64_t i = 0;
    int64_t grown = 0;
    while (grown < n_prune) {
        int64_t p = oracle_regrow_position(oracle_regrow_draw(seed, step, i), out, in);
        ++i;
        int taken = (occ[p >> 3] >> (p & 7)) & 1;
        if (MUTANT(7)) taken = 0; /* mutant 7: ignores occupancy */
        if (taken) continue;
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        all[m].a = p / in;
        all[m].b = p % in;
        all[m].idx = -1; /* regrown entry */
        ++m;
        ++grown;
    }
    if (n_draws) *n_draws = (int64_t)i;

    /* 5. back to canonical order */
    qsort(all, (size_t)m, sizeof *all, cmp_triple);
    for (int64_t k = 0; k < m; ++k) {
        rows_new[k] = (int32_t)all[k].a;
        cols_new[k] = (int32_t)all[k].b;
        char *dst = (char *)vals_new + k * eb;
        if (all[k].idx >= 0)
            memcpy(dst, (const char *)vals_c + all[k].idx * eb, (size_t)eb);
        else if (dtype == OR_BF16) {
            uint16_t h = (uint16_t)regrow_bits;
            memcpy(dst, &h, 2);
        } else
            memcpy(dst, &regrow_bits, 4);
    }
    free(ord);
    free(pruned);
    free(occ);
    free(all);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Gradient-informed restructure (the regrow variant ranked next after   */
/* random regrow; the page's Abstract speaks of restructuring the        */
/* connections during dynamic sparse training and fixes no regrow rule). */
/* Prune exactly as oracle_restructure.  Then every position that is     */
/* empty after the prune gets the score                                  */
/*     g(r, c) = | sum_b dY[b, r] * X[b, c] |                            */
/* -- the magnitude of the dense weight gradient at that position -- in  */
/* fp32, as a fused-multiply-add chain in batch order:                   */
/*     s = 0; for b = 0..B-1: s = fmaf(dY[b, r], X[b, c], s)             */
/* (bf16 inputs widen exactly to fp32 first).  The n_prune empty         */
/* positions with the largest scores are regrown, ordered by (bit        */
/* pattern of |s| descending, position r * in + c ascending); regrown    */
/* entries take regrow_bits.  Kept and new entries return to canonical   */
/* order.  Input must be canonical.                                      */
/* ------------------------------------------------------------------ */
typedef struct {
    uint32_t key;
    int64_t pos;
} scored_t;

static int cmp_scored(const void *pa, const void *pb)
{
    const scored_t *x = (const scored_t *)pa, *y = (const scored_t *)pb;
    if (x->key != y->key) return x->key > y->key ? -1 : 1; /* larger score first */
    if (x->pos != y->pos) {
        int before = x->pos < y->pos;
        if (MUTANT(8)) before = !before; /* mutant 8: ties go to the larger position */
        return before ? -1 : 1;
    }
    return 0;
}

static float word_to_float(const void *base, int dtype, int64_t i)
{
    return (float)word_to_double(base, dtype, i); /* exact: every word is an fp32 or bf16 value */
}

int oracle_restructure_grad(int64_t out, int64_t in, int64_t nnz, const int32_t *rows_c, const int32_t *cols_c,
                            const void *vals_c, int dtype, int64_t n_prune, const void *dY, const void *X, int64_t B,
                            uint32_t regrow_bits, int32_t *rows_new, int32_t *cols_new, void *vals_new)
{
    if (n_prune < 0 || n_prune > nnz || out <= 0 || in <= 0 || B <= 0) return OR_ERR_ARG;
    int64_t npos = out * in;
    int eb = elem_bytes(dtype);

    /* 1. prune, as in oracle_restructure */
    absent_t *ord = (absent_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *ord);
    unsigned char *pruned = (unsigned char *)calloc((size_t)(nnz ? nnz : 1), 1);
    unsigned char *occ = (unsigned char *)calloc((size_t)((npos + 7) / 8), 1);
    triple_t *all = (triple_t *)malloc((size_t)(nnz ? nnz : 1) * sizeof *all);
    scored_t *cand = (scored_t *)malloc((size_t)npos * sizeof *cand);
    float *dyf = (float *)malloc((size_t)(B * out) * sizeof *dyf);
    float *xf = (float *)malloc((size_t)(B * in) * sizeof *xf);
    if (!ord || !pruned || !occ || !all || !cand || !dyf || !xf) {
        free(ord);
        free(pruned);
        free(occ);
        free(all);
        free(cand);
        free(dyf);
        free(xf);
        return OR_ERR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        ord[k].key = magnitude_key(vals_c, dtype, k);
        ord[k].idx = k;
    }
    qsort(ord, (size_t)nnz, sizeof *ord, cmp_absent);
    for (int64_t j = 0; j < n_prune; ++j) pruned[ord[j].idx] = 1;

    /* 2. kept entries and their positions */
    int64_t m = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (pruned[k]) continue;
        int64_t p = (int64_t)rows_c[k] * in + cols_c[k];
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        all[m].a = rows_c[k];
        all[m].b = cols_c[k];
        all[m].idx = k;
        ++m;
    }

    /* 3. scores of the empty positions, best n_prune of them */
    for (int64_t i = 0; i < B * out; ++i) dyf[i] = word_to_float(dY, dtype, i);
    for (int64_t i = 0; i < B * in; ++i) xf[i] = word_to_float(X, dtype, i);
    int64_t ncand = 0;
    for (int64_t r = 0; r < out; ++r)
        for (int64_t c = 0; c < in; ++c) {
            int64_t p = r * in + c;
            if ((occ[p >> 3] >> (p & 7)) & 1) continue;
            float sc = 0.0f;
            for (int64_t b = 0; b < B; ++b) sc = fmaf(dyf[b * out + r], xf[b * in + c], sc);
            if (!MUTANT(9)) sc = fabsf(sc); /* mutant 9: ranks the signed sum */
            uint32_t key;
            memcpy(&key, &sc, 4);
            if (MUTANT(9)) key ^= (key >> 31) ? 0xFFFFFFFFu : 0x80000000u; /* order of the signed value */
            cand[ncand].key = key;
            cand[ncand].pos = p;
            ++ncand;
        }
    qsort(cand, (size_t)ncand, sizeof *cand, cmp_scored);
    for (int64_t j = 0; j < n_prune; ++j) {
        all[m].a = cand[j].pos / in;
        all[m].b = cand[j].pos % in;
        all[m].idx = -1;
        ++m;
    }

    /* 4. back to canonical order */
    qsort(all, (size_t)m, sizeof *all, cmp_triple);
    for (int64_t k = 0; k < m; ++k) {
        rows_new[k] = (int32_t)all[k].a;
        cols_new[k] = (int32_t)all[k].b;
        char *dst = (char *)vals_new + k * eb;
        if (all[k].idx >= 0)
            memcpy(dst, (const char *)vals_c + all[k].idx * eb, (size_t)eb);
        else if (dtype == OR_BF16) {
            uint16_t h = (uint16_t)regrow_bits;
            memcpy(dst, &h, 2);
        } else
            memcpy(dst, &regrow_bits, 4);
    }
    free(ord);
    free(pruned);
    free(occ);
    free(all);
    free(cand);
    free(dyf);
    free(xf);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* GELU (exact erf form) and its derivative, for the two-layer MLP       */
/* workload that places GELU between two sparse layers.                  */
/*   gelu(x)  = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))                 */
/*   gelu'(x) = Phi(x) + x phi(x),  phi(x) = exp(-x^2/2) / sqrt(2 pi)     */
/* ------------------------------------------------------------------ */
void oracle_gelu(int64_t n, const double *x, double *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = 0.5 * x[i] * (1.0 + erf(x[i] / sqrt(2.0)));
}

void oracle_gelu_grad(int64_t n, const double *x, double *g)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    for (int64_t i = 0; i < n; ++i) {
        double cdf = 0.5 * (1.0 + erf(x[i] / sqrt(2.0)));
        g[i] = cdf + x[i] * inv_sqrt_2pi * exp(-0.5 * x[i] * x[i]);
    }
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }
