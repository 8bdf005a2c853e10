/*
 * fa_oracle.c -- plain CPU reference for scaled dot-product attention, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant with the HIP kernels.
 *
 * What it computes (the plain definition, two passes per query row):
 *
 *   "Triton Ascend Attention", section "standard attention computation flow",
 *   the three phases: scores = Q K^T * scale, attn = softmax(scores) with each
 *   row summing to one, output = attn V.
 *   FlashAttention-2 forward article (wsisp.com), the passage that defines
 *   S = Q K^T, P = softmax(S), O = P V, and the kernel epilogue that stores the
 *   per-row statistic m + log(l) (natural log) next to O.
 *
 * Causal masking ("flash-attention-kernel" skill page, pitfalls list, and the
 * FlashAttention-2 article, _attn_fwd_inner mask): query i keeps key j when
 * j <= i (the diagonal is kept), indices counted from the top-left corner.
 * Keys j >= Lk do not exist and are never visited.
 *
 * For every row (b, h, i):
 *   J    = { 0 <= j < Lk : (!causal) or j <= i }
 *   s_j  = scale * sum_d q[b,h,i,d] * k[b,h,j,d]          (j in J)
 *   m    = max_j s_j                                        (pass 1)
 *   l    = sum_j exp(s_j - m)                               (pass 2)
 *   p_j  = exp(s_j - m) / l,   p_j = 0 for j not in J
 *   o[d] = sum_j p_j * v[b,h,j,d]
 *   lse  = m + log(l)
 * A row with J empty (impossible for Lk >= 1 under top-left causal) gets
 * o = 0 and lse = -inf.
 *
 * Arithmetic is IEEE double, no fast-math; the row loop is OpenMP-parallel
 * (rows are independent, so the parallel result is identical to the serial).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One past the last visible key of query row i. */
static int64_t visible_end(int64_t i, int64_t Lk, int causal)
{
    if (!causal) return Lk;
    return (i + 1 < Lk) ? i + 1 : Lk;
}

/*
 * Probabilities of one query row.  q_row points at q[b,h,i,0]; k_head at
 * k[b,h,0,0].  Writes p[0..Lk), zero for invisible keys, and returns m and l.
 * Returns 0 when the row has no visible key (then p is all zero).
 */
static int softmax_row(const double *q_row, const double *k_head, int64_t Lk,
                       int64_t D, int64_t jend, double scale, double *p,
                       double *m_out, double *l_out)
{
    int64_t j, d;
    double m = -INFINITY, l = 0.0;

    for (j = 0; j < Lk; ++j) p[j] = 0.0;
    if (jend <= 0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return 0;
    }
    /* scores, and pass 1: the row maximum */
    for (j = 0; j < jend; ++j) {
        const double *k_row = k_head + j * D;
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += q_row[d] * k_row[d];
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
    }
    /* pass 2: exponentials relative to the maximum, and their sum */
    for (j = 0; j < jend; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (j = 0; j < jend; ++j) p[j] /= l;
    *m_out = m;
    *l_out = l;
    return 1;
}

/* o_row[d] = sum_j p[j] * v[b,h,j,d] over the visible keys. */
static void weighted_sum(const double *p, const double *v_head, int64_t jend,
                         int64_t D, double *o_row)
{
    int64_t j, d;
    for (d = 0; d < D; ++d) o_row[d] = 0.0;
    for (j = 0; j < jend; ++j) {
        const double *v_row = v_head + j * D;
        for (d = 0; d < D; ++d) o_row[d] += p[j] * v_row[d];
    }
}

static int check_shape(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D)
{
    return (B >= 0 && H >= 0 && Lq >= 0 && Lk >= 0 && D >= 1);
}

/* One row (b*H + h, i) of the output: o_row[0..D) and *lse_out. */
static void one_row(const double *q, const double *k, const double *v,
                    int64_t bh, int64_t i, int64_t Lq, int64_t Lk, int64_t D,
                    int causal, double scale, double *p, double *o_row,
                    double *lse_out)
{
    const double *q_row = q + (bh * Lq + i) * D;
    const double *k_head = k + bh * Lk * D;
    const double *v_head = v + bh * Lk * D;
    int64_t jend = visible_end(i, Lk, causal);
    double m, l;

    if (!softmax_row(q_row, k_head, Lk, D, jend, scale, p, &m, &l)) {
        int64_t d;
        for (d = 0; d < D; ++d) o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    weighted_sum(p, v_head, jend, D, o_row);
    *lse_out = m + log(l);
}

/*
 * Full forward: q [B,H,Lq,D], k and v [B,H,Lk,D], o [B,H,Lq,D], lse [B,H,Lq],
 * all contiguous row-major fp64.  Returns 0, or -1 on a bad shape or an
 * allocation failure.
 */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, int64_t B, int64_t H, int64_t Lq,
                     int64_t Lk, int64_t D, int causal, double scale)
{
    int64_t rows = B * H * Lq, r;
    int failed = 0;
    if (!check_shape(B, H, Lq, Lk, D)) return -1;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        if (!p) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (r = 0; r < rows; ++r) {
                int64_t bh = r / Lq, i = r % Lq;
                one_row(q, k, v, bh, i, Lq, Lk, D, causal, scale, p,
                        o + r * D, lse + r);
            }
        }
        free(p);
    }
    return failed ? -1 : 0;
}

/*
 * Selected rows only.  row_ids[n] = (b*H + h)*Lq + i names a query row; the
 * outputs are packed: o_rows [nrows, D], lse_rows [nrows].  Rows are
 * independent, so each selected row is exactly what oracle_attention gives.
 */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          const int64_t *row_ids, int64_t nrows,
                          double *o_rows, double *lse_rows, int64_t B,
                          int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                          int causal, double scale)
{
    int64_t n;
    int failed = 0;
    if (!check_shape(B, H, Lq, Lk, D)) return -1;
    for (n = 0; n < nrows; ++n)
        if (row_ids[n] < 0 || row_ids[n] >= B * H * Lq) return -1;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
        if (!p) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (n = 0; n < nrows; ++n) {
                int64_t r = row_ids[n];
                one_row(q, k, v, r / Lq, r % Lq, Lq, Lk, D, causal, scale, p,
                        o_rows + n * D, lse_rows + n);
            }
        }
        free(p);
    }
    return failed ? -1 : 0;
}

/*
 * The probability matrix itself: p_out [B,H,Lq,Lk], zero where masked.
 * Used by the tests to check that every row sums to one and that O = P V.
 */
int oracle_probs(const double *q, const double *k, double *p_out, int64_t B,
                 int64_t H, int64_t Lq, int64_t Lk, int64_t D, int causal,
                 double scale)
{
    int64_t rows = B * H * Lq, r;
    if (!check_shape(B, H, Lq, Lk, D)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (r = 0; r < rows; ++r) {
        int64_t bh = r / Lq, i = r % Lq;
        double m, l;
        softmax_row(q + r * D, k + bh * Lk * D, Lk, D, visible_end(i, Lk, causal),
                    scale, p_out + r * Lk, &m, &l);
    }
    return 0;
}

/* Threads the OpenMP runtime will use for the calls above. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
