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
 * Local (sliding-window) masking, one of the mask variants the article
 * leaves for later: with window_left wl >= 0 query i also drops keys
 * j < i - wl, with window_right wr >= 0 it drops keys j > i + wr; a negative
 * bound means no bound.  Causal and a window combine (both must keep j).
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

/* Visible keys of query row i: [visible_begin, visible_end). */
static int64_t visible_end(int64_t i, int64_t Lk, int causal, int64_t wr)
{
    int64_t e = Lk;
    if (causal && i + 1 < e) e = i + 1;
    if (wr >= 0 && i + wr + 1 < e) e = i + wr + 1;
    return e;
}

static int64_t visible_begin(int64_t i, int64_t wl)
{
    if (wl < 0 || i - wl <= 0) return 0;
    return i - wl;
}

/*
 * Probabilities of one query row.  q_row points at q[b,h,i,0]; k_head at
 * k[b,h,0,0].  Writes p[0..Lk), zero for invisible keys, and returns m and l.
 * Returns 0 when the row has no visible key (then p is all zero).
 */
static int softmax_row(const double *q_row, const double *k_head, int64_t Lk,
                       int64_t D, int64_t jbeg, int64_t jend, double scale,
                       double *p, double *m_out, double *l_out)
{
    int64_t j, d;
    double m = -INFINITY, l = 0.0;

    for (j = 0; j < Lk; ++j) p[j] = 0.0;
    if (jend <= jbeg) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return 0;
    }
    /* scores, and pass 1: the row maximum */
    for (j = jbeg; j < jend; ++j) {
        const double *k_row = k_head + j * D;
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += q_row[d] * k_row[d];
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
    }
    /* pass 2: exponentials relative to the maximum, and their sum */
    for (j = jbeg; j < jend; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (j = jbeg; j < jend; ++j) p[j] /= l;
    *m_out = m;
    *l_out = l;
    return 1;
}

/* o_row[d] = sum_j p[j] * v[b,h,j,d] over the visible keys. */
static void weighted_sum(const double *p, const double *v_head, int64_t jbeg,
                         int64_t jend, int64_t D, double *o_row)
{
    int64_t j, d;
    for (d = 0; d < D; ++d) o_row[d] = 0.0;
    for (j = jbeg; j < jend; ++j) {
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
                    int causal, int64_t wl, int64_t wr, double scale, double *p,
                    double *o_row, double *lse_out)
{
    const double *q_row = q + (bh * Lq + i) * D;
    const double *k_head = k + bh * Lk * D;
    const double *v_head = v + bh * Lk * D;
    int64_t jbeg = visible_begin(i, wl), jend = visible_end(i, Lk, causal, wr);
    double m, l;

    if (!softmax_row(q_row, k_head, Lk, D, jbeg, jend, scale, p, &m, &l)) {
        int64_t d;
        for (d = 0; d < D; ++d) o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    weighted_sum(p, v_head, jbeg, jend, D, o_row);
    *lse_out = m + log(l);
}

/*
 * Full forward: q [B,H,Lq,D], k and v [B,H,Lk,D], o [B,H,Lq,D], lse [B,H,Lq],
 * all contiguous row-major fp64; wl / wr are the window bounds (negative: no
 * bound).  Returns 0, or -1 on a bad shape or an allocation failure.
 */
int oracle_attention_win(const double *q, const double *k, const double *v,
                         double *o, double *lse, int64_t B, int64_t H,
                         int64_t Lq, int64_t Lk, int64_t D, int causal,
                         int64_t wl, int64_t wr, double scale)
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
                one_row(q, k, v, bh, i, Lq, Lk, D, causal, wl, wr, scale, p,
                        o + r * D, lse + r);
            }
        }
        free(p);
    }
    return failed ? -1 : 0;
}

/* The forward without a window. */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, int64_t B, int64_t H, int64_t Lq,
                     int64_t Lk, int64_t D, int causal, double scale)
{
    return oracle_attention_win(q, k, v, o, lse, B, H, Lq, Lk, D, causal, -1,
                                -1, scale);
}

/*
 * Selected rows only.  row_ids[n] = (b*H + h)*Lq + i names a query row; the
 * outputs are packed: o_rows [nrows, D], lse_rows [nrows].  Rows are
 * independent, so each selected row is exactly what oracle_attention gives.
 */
int oracle_attention_rows_win(const double *q, const double *k,
                              const double *v, const int64_t *row_ids,
                              int64_t nrows, double *o_rows, double *lse_rows,
                              int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                              int64_t D, int causal, int64_t wl, int64_t wr,
                              double scale)
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
                one_row(q, k, v, r / Lq, r % Lq, Lq, Lk, D, causal, wl, wr,
                        scale, p, o_rows + n * D, lse_rows + n);
            }
        }
        free(p);
    }
    return failed ? -1 : 0;
}

int oracle_attention_rows(const double *q, const double *k, const double *v,
                          const int64_t *row_ids, int64_t nrows,
                          double *o_rows, double *lse_rows, int64_t B,
                          int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                          int causal, double scale)
{
    return oracle_attention_rows_win(q, k, v, row_ids, nrows, o_rows,
                                     lse_rows, B, H, Lq, Lk, D, causal, -1, -1,
                                     scale);
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
        softmax_row(q + r * D, k + bh * Lk * D, Lk, D, 0,
                    visible_end(i, Lk, causal, -1), scale, p_out + r * Lk, &m,
                    &l);
    }
    return 0;
}

/*
 * Gradients of the forward above with respect to q, k and v, for an incoming
 * gradient dout of o.  The pages implement only the forward: the
 * FlashAttention-2 article's host wrapper keeps q, k, v, o and the row
 * statistic for a backward pass, and its closing remarks leave the backward
 * as future work; the same article's account of the IO-aware idea notes
 * that a backward pass may recompute the probabilities rather than store
 * them.  The backward is therefore the plain chain rule through the
 * definition in this file's header, with lse an auxiliary output that takes
 * no gradient.  Per (b, h), with p the probabilities of the forward:
 *
 *   dv_j  = sum_i p_ij dout_i
 *   dp_ij = dout_i . v_j
 *   delta_i = sum_j p_ij dp_ij
 *   ds_ij = p_ij (dp_ij - delta_i)          (softmax Jacobian; 0 if masked)
 *   dq_i  = scale * sum_j ds_ij k_j
 *   dk_j  = scale * sum_i ds_ij q_i
 *
 * Layouts as for oracle_attention; dout and dq are [B,H,Lq,D], dk and dv
 * [B,H,Lk,D]; delta [B,H,Lq] receives delta_i (may be NULL).  wl / wr: the
 * window of the forward (p is 0 outside it, so are ds and the sums).  Each head keeps p and ds as dense [Lq, Lk] fp64 matrices.
 * Rows are done in parallel (p, ds, dq), then keys (dk, dv), so no sum is
 * shared between threads.  Returns 0, or -1 on a bad shape or allocation
 * failure.
 */
int oracle_attention_bwd_win(const double *q, const double *k,
                             const double *v, const double *dout, double *dq,
                             double *dk, double *dv, double *delta_out,
                             int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                             int64_t D, int causal, int64_t wl, int64_t wr,
                             double scale)
{
    int64_t bh;
    double *p, *ds;
    if (!check_shape(B, H, Lq, Lk, D)) return -1;
    p = (double *)malloc(sizeof(double) * (size_t)(Lq * Lk > 0 ? Lq * Lk : 1));
    ds = (double *)malloc(sizeof(double) * (size_t)(Lq * Lk > 0 ? Lq * Lk : 1));
    if (!p || !ds) {
        free(p);
        free(ds);
        return -1;
    }
    for (bh = 0; bh < B * H; ++bh) {
        const double *qh = q + bh * Lq * D, *kh = k + bh * Lk * D;
        const double *vh = v + bh * Lk * D, *gh = dout + bh * Lq * D;
        double *dqh = dq + bh * Lq * D, *dkh = dk + bh * Lk * D;
        double *dvh = dv + bh * Lk * D;
        int64_t i, j;
#pragma omp parallel for schedule(dynamic, 8)
        for (i = 0; i < Lq; ++i) {
            double *pi = p + i * Lk, *dsi = ds + i * Lk;
            const double *gi = gh + i * D;
            int64_t jbeg = visible_begin(i, wl), jj, d;
            int64_t jend = visible_end(i, Lk, causal, wr);
            double m, l, delta = 0.0;
            softmax_row(qh + i * D, kh, Lk, D, jbeg, jend, scale, pi, &m, &l);
            for (jj = 0; jj < Lk; ++jj) dsi[jj] = 0.0;
            for (jj = jbeg; jj < jend; ++jj) {
                const double *vj = vh + jj * D;
                double dp = 0.0;
                for (d = 0; d < D; ++d) dp += gi[d] * vj[d];
                dsi[jj] = dp;
                delta += pi[jj] * dp;
            }
            for (jj = jbeg; jj < jend; ++jj) dsi[jj] = pi[jj] * (dsi[jj] - delta);
            if (delta_out) delta_out[bh * Lq + i] = delta;
            for (d = 0; d < D; ++d) {
                double acc = 0.0;
                for (jj = jbeg; jj < jend; ++jj) acc += dsi[jj] * kh[jj * D + d];
                dqh[i * D + d] = scale * acc;
            }
        }
#pragma omp parallel for schedule(dynamic, 8)
        for (j = 0; j < Lk; ++j) {
            int64_t ii, d;
            for (d = 0; d < D; ++d) {
                double accv = 0.0, acck = 0.0;
                for (ii = 0; ii < Lq; ++ii) {
                    accv += p[ii * Lk + j] * gh[ii * D + d];
                    acck += ds[ii * Lk + j] * qh[ii * D + d];
                }
                dvh[j * D + d] = accv;
                dkh[j * D + d] = scale * acck;
            }
        }
    }
    free(p);
    free(ds);
    return 0;
}

/* The backward without a window. */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk,
                         double *dv, double *delta_out, int64_t B, int64_t H,
                         int64_t Lq, int64_t Lk, int64_t D, int causal,
                         double scale)
{
    return oracle_attention_bwd_win(q, k, v, dout, dq, dk, dv, delta_out, B, H,
                                    Lq, Lk, D, causal, -1, -1, scale);
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
