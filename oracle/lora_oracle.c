/*
 * Plain fp64 CPU oracle for unmerged multi-LoRA application.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no grouping):
 *
 *   "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged
 *   or alongside": with W' = W + BA (A is r x d, B is d x r), the unmerged form
 *   adds x A^T B^T to x W^T in every adapted layer.  Generalised here to
 *   A: r x d_in and B: d_out x r.
 *
 *   Same page, "Exercises" (the four-requests answer) and the self-test answer
 *   on mixing LoRAs: each request names its own adapter, each request's rows
 *   get their own x A^T B^T, and every result goes back to the row it came
 *   from; section "LoRA: merged or alongside" (comparison table, stacking
 *   row): stacked LoRAs add further computations alongside, whose results add.
 *
 *   For every request s and every row t of it, for every slot k whose index
 *   i = idx[s][k] is not -1:
 *       v[j]    = sum_c x[t][c] * A[i][j][c]                 (c ascending)
 *       acc[o] += scale[s][k] * sum_j v[j] * B[i][o][j]      (j ascending)
 *   y_ref[t] = y[t] + acc   if some slot of the request is not -1,
 *   y_ref[t] = y[t]         otherwise (the row is untouched).
 *   Rows covered by no request are untouched.
 *
 * Adapters of different ranks in one pool ("LoRA: merged or alongside": r is
 * usually 8 to 128) are stored at the pool's rank r; with a rank array, row j
 * of A_i and column j of B_i take part only for j < ranks[i] (what lies
 * beyond is never read), which is the same as zero padding.
 *
 * Readings where the pages are silent: no implicit alpha/r factor; the
 * per-slot scale defaults to 1 and multiplies the slot's contribution; an
 * index below -1 or >= n is an error here (the oracle refuses the input).
 *
 * Inputs are decoded exactly to double: float32 values, or bfloat16 bit
 * patterns widened to float32.  All arithmetic is double, in the order above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_ESHAPE = -1, OR_EINDEX = -2, OR_ESEG = -3, OR_ENOMEM = -4 };

static double elem(const void *p, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Map every row to the request that covers it (-1: none).  Requests must be
 * given by non-decreasing offsets inside [0, T]; per-token mode (seg_off NULL)
 * means request s is row s. */
static int build_row_owner(int T, int S, const int32_t *seg_off, int32_t *owner) {
    for (int t = 0; t < T; ++t) owner[t] = -1;
    if (!seg_off) {
        if (S != T) return OR_ESHAPE;
        for (int t = 0; t < T; ++t) owner[t] = t;
        return OR_OK;
    }
    if (seg_off[0] < 0 || seg_off[S] > T) return OR_ESEG;
    for (int s = 0; s < S; ++s) {
        if (seg_off[s + 1] < seg_off[s]) return OR_ESEG;
        for (int t = seg_off[s]; t < seg_off[s + 1]; ++t) owner[t] = s;
    }
    return OR_OK;
}

static int check_indices(int S, int K, const int32_t *idx, int n) {
    for (int64_t q = 0; q < (int64_t)S * K; ++q)
        if (idx[q] < -1 || idx[q] >= n) return OR_EINDEX;
    return OR_OK;
}

/* Per-adapter ranks (NULL: every adapter has rank r): each in [1, r]. */
static int check_ranks(int n, int r, const int32_t *ranks) {
    if (!ranks) return OR_OK;
    for (int i = 0; i < n; ++i)
        if (ranks[i] < 1 || ranks[i] > r) return OR_ESHAPE;
    return OR_OK;
}

static int check_common(int n, int r, int d_in, int d_out, int T, int S, int K, int64_t ldx, int64_t ldy) {
    if (n < 0 || r < 1 || d_in < 1 || d_out < 1 || T < 0 || S < 0 || K < 1) return OR_ESHAPE;
    if (ldx < d_in || ldy < d_out) return OR_ESHAPE;
    return OR_OK;
}

/*
 * y_ref for n_rows rows (rows == NULL: all T rows, in order).
 *   y_ref   [n_rows][d_out]  double
 *   touched [n_rows]         1 if some slot of the row's request is not -1
 *   routing [n_rows][K]      adapter applied in slot k, or -1
 *   macs    (optional)       multiply-adds performed
 */
int oracle_apply(int dtype, int n, int r, int d_in, int d_out, const void *A, const void *B,
                 int T, int S, const int32_t *seg_off, const int32_t *idx, int K, const float *scale,
                 const void *x, int64_t ldx, const void *y, int64_t ldy,
                 const int32_t *rows, int n_rows,
                 double *y_ref, uint8_t *touched, int32_t *routing, int64_t *macs, int nthreads,
                 const int32_t *ranks) {
    int rc = check_common(n, r, d_in, d_out, T, S, K, ldx, ldy);
    if (rc) return rc;
    if ((rc = check_ranks(n, r, ranks))) return rc;
    if ((rc = check_indices(S, K, idx, n))) return rc;
    int32_t *owner = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!owner) return OR_ENOMEM;
    if ((rc = build_row_owner(T, S, seg_off, owner))) { free(owner); return rc; }
    if (!rows) n_rows = T;
    for (int q = 0; q < n_rows; ++q) {
        int t = rows ? rows[q] : q;
        if (t < 0 || t >= T) { free(owner); return OR_ESHAPE; }
    }
    int64_t mac_total = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel reduction(+ : mac_total)
#endif
    {
        double *v = (double *)malloc(sizeof(double) * (size_t)r);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d_out);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int q = 0; q < n_rows; ++q) {
            int t = rows ? rows[q] : q;
            int s = owner[t];
            int hit = 0;
            for (int o = 0; o < d_out; ++o) acc[o] = 0.0;
            for (int k = 0; k < K; ++k) {
                int i = (s >= 0) ? idx[(int64_t)s * K + k] : -1;
                routing[(int64_t)q * K + k] = i;
                if (i == -1) continue;
                hit = 1;
                double sc = scale ? (double)scale[(int64_t)s * K + k] : 1.0;
                const int ri = ranks ? ranks[i] : r;  /* the adapter's own rank */
                for (int j = 0; j < ri; ++j) {
                    double sum = 0.0;
                    for (int c = 0; c < d_in; ++c)
                        sum += elem(x, dtype, (int64_t)t * ldx + c) *
                               elem(A, dtype, ((int64_t)i * r + j) * d_in + c);
                    v[j] = sum;
                }
                for (int o = 0; o < d_out; ++o) {
                    double sum = 0.0;
                    for (int j = 0; j < ri; ++j)
                        sum += v[j] * elem(B, dtype, ((int64_t)i * d_out + o) * r + j);
                    acc[o] += sc * sum;
                }
                mac_total += (int64_t)ri * d_in + (int64_t)d_out * ri;
            }
            touched[q] = (uint8_t)hit;
            for (int o = 0; o < d_out; ++o) {
                double y0 = elem(y, dtype, (int64_t)t * ldy + o);
                y_ref[(int64_t)q * d_out + o] = hit ? y0 + acc[o] : y0;
            }
        }
        free(v);
        free(acc);
    }
    free(owner);
    if (macs) *macs = mac_total;
    return OR_OK;
}

/*
 * The rank-r intermediate alone (the "shrink" half of x A^T B^T), per slot:
 *   v_ref[q][k*r + j] = scale[s][k] * sum_c x[t][c] * A[i][j][c]   (slot valid)
 *   v_ref[q][k*r + j] = 0                                          (slot -1)
 * touched as in oracle_apply; v_ref rows of untouched rows are all 0.
 */
int oracle_shrink(int dtype, int n, int r, int d_in, const void *A,
                  int T, int S, const int32_t *seg_off, const int32_t *idx, int K, const float *scale,
                  const void *x, int64_t ldx, const int32_t *rows, int n_rows,
                  double *v_ref, uint8_t *touched, int nthreads, const int32_t *ranks) {
    int rc = check_common(n, r, d_in, 1, T, S, K, ldx, 1);
    if (rc) return rc;
    if ((rc = check_ranks(n, r, ranks))) return rc;
    if ((rc = check_indices(S, K, idx, n))) return rc;
    int32_t *owner = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!owner) return OR_ENOMEM;
    if ((rc = build_row_owner(T, S, seg_off, owner))) { free(owner); return rc; }
    if (!rows) n_rows = T;
    for (int q = 0; q < n_rows; ++q) {
        int t = rows ? rows[q] : q;
        if (t < 0 || t >= T) { free(owner); return OR_ESHAPE; }
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int q = 0; q < n_rows; ++q) {
        int t = rows ? rows[q] : q;
        int s = owner[t];
        int hit = 0;
        for (int k = 0; k < K; ++k) {
            int i = (s >= 0) ? idx[(int64_t)s * K + k] : -1;
            double *vk = v_ref + (int64_t)q * K * r + (int64_t)k * r;
            if (i == -1) {
                for (int j = 0; j < r; ++j) vk[j] = 0.0;
                continue;
            }
            hit = 1;
            double sc = scale ? (double)scale[(int64_t)s * K + k] : 1.0;
            const int ri = ranks ? ranks[i] : r;
            for (int j = 0; j < r; ++j) {
                double sum = 0.0;
                for (int c = 0; j < ri && c < d_in; ++c)
                    sum += elem(x, dtype, (int64_t)t * ldx + c) *
                           elem(A, dtype, ((int64_t)i * r + j) * d_in + c);
                vk[j] = sc * sum;  /* 0 past the adapter's rank */
            }
        }
        touched[q] = (uint8_t)hit;
    }
    free(owner);
    return OR_OK;
}

/*
 * The "expand" half, given a float32 intermediate v [T][ldv] laid out as
 * v[t][k*r + j] (per slot, scale already folded in):
 *   y_ref[q][o] = y[t][o] + sum_{k valid} sum_j v[t][k*r + j] * B[i][o][j]
 * for touched rows; untouched rows copy y.
 */
int oracle_expand(int dtype, int n, int r, int d_out, const void *B,
                  int T, int S, const int32_t *seg_off, const int32_t *idx, int K,
                  const float *v, int64_t ldv, const void *y, int64_t ldy,
                  const int32_t *rows, int n_rows, double *y_ref, uint8_t *touched, int nthreads,
                  const int32_t *ranks) {
    int rc = check_common(n, r, 1, d_out, T, S, K, 1, ldy);
    if (rc) return rc;
    if ((rc = check_ranks(n, r, ranks))) return rc;
    if (ldv < (int64_t)K * r) return OR_ESHAPE;
    if ((rc = check_indices(S, K, idx, n))) return rc;
    int32_t *owner = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!owner) return OR_ENOMEM;
    if ((rc = build_row_owner(T, S, seg_off, owner))) { free(owner); return rc; }
    if (!rows) n_rows = T;
    for (int q = 0; q < n_rows; ++q) {
        int t = rows ? rows[q] : q;
        if (t < 0 || t >= T) { free(owner); return OR_ESHAPE; }
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int q = 0; q < n_rows; ++q) {
        int t = rows ? rows[q] : q;
        int s = owner[t];
        int hit = 0;
        for (int k = 0; k < K; ++k)
            if (s >= 0 && idx[(int64_t)s * K + k] != -1) hit = 1;
        touched[q] = (uint8_t)hit;
        for (int o = 0; o < d_out; ++o) {
            double y0 = elem(y, dtype, (int64_t)t * ldy + o);
            if (!hit) { y_ref[(int64_t)q * d_out + o] = y0; continue; }
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                int i = idx[(int64_t)s * K + k];
                if (i == -1) continue;
                const int ri = ranks ? ranks[i] : r;
                double sum = 0.0;
                for (int j = 0; j < ri; ++j)
                    sum += (double)v[(int64_t)t * ldv + (int64_t)k * r + j] *
                           elem(B, dtype, ((int64_t)i * d_out + o) * r + j);
                acc += sum;
            }
            y_ref[(int64_t)q * d_out + o] = y0 + acc;
        }
    }
    free(owner);
    return OR_OK;
}

/*
 * Merge / unmerge ("Serving several LoRAs, ControlNet and IP-Adapter", section
 * "LoRA: merged or alongside"): the merged form computes W + BA ahead of time;
 * stacked LoRAs merge as a weighted sum (comparison table, stacking row);
 * unmerging subtracts what was added.  Here, for output rows o in
 * [row_lo, row_hi) and every column c < d_in:
 *
 *   W_out[o - row_lo][c] = W[o][c]
 *       + alpha * sum_k scale[k] * sum_j B[idx[k]][o][j] * A[idx[k]][j][c]
 *
 * over the slots k with idx[k] != -1 (j ascending, then k ascending), with
 * scale NULL meaning 1.  alpha = 1 merges, alpha = -1 unmerges.  W is
 * [d_out][ldw] in the pool's type; W_out is double.
 */
int oracle_merge(int dtype, int n, int r, int d_in, int d_out, const void *A, const void *B,
                 const void *W, int64_t ldw, int K, const int32_t *idx, const float *scale, double alpha,
                 int row_lo, int row_hi, double *W_out, int nthreads) {
    if (n < 1 || r < 1 || d_in < 1 || d_out < 1 || ldw < d_in || K < 0) return OR_ESHAPE;
    if (row_lo < 0 || row_hi > d_out || row_lo > row_hi) return OR_ESHAPE;
    for (int k = 0; k < K; ++k)
        if (idx[k] < -1 || idx[k] >= n) return OR_EINDEX;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int o = row_lo; o < row_hi; ++o) {
        for (int c = 0; c < d_in; ++c) {
            double delta = 0.0;
            for (int k = 0; k < K; ++k) {
                const int i = idx[k];
                if (i == -1) continue;
                double sum = 0.0;
                for (int j = 0; j < r; ++j)
                    sum += elem(B, dtype, ((int64_t)i * d_out + o) * r + j) *
                           elem(A, dtype, ((int64_t)i * r + j) * d_in + c);
                delta += (scale ? (double)scale[k] : 1.0) * sum;
            }
            W_out[(int64_t)(o - row_lo) * d_in + c] = elem(W, dtype, (int64_t)o * ldw + c) + alpha * delta;
        }
    }
    return OR_OK;
}
