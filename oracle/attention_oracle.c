/*
 * attention_oracle.c — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of exact attention, used by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg to judge
 * the GPU library.  Nothing in the product path may link or call it, and it
 * shares no code, header or constant with the GPU library.
 *
 * What it computes (the plain definition, not the tiled algorithm):
 *
 *   Pages "FlashAttention (HI)" and "FlashAttention (TL)", section on the
 *   problems of standard attention, print the one formula of the method:
 *       Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *   with the softmax taken along each query row.  The same pages (section on
 *   fusing all operations into one kernel) name masking as one of the fused
 *   operations; the causal mask used here lets query i see key j iff j <= i.
 *   The pages call FlashAttention exact ("online softmax" section: the result
 *   is exact; "FlashAttention-2 (BN)", performance section: exact and
 *   deterministic), so the oracle is that definition written out:
 *
 *     s_ij  = scale * sum_c q_ic k_jc
 *     A_i   = { j : 0 <= j < N and (causal == 0 or j <= i) }
 *     m_i   = max_{j in A_i} s_ij
 *     l_i   = sum_{j in A_i} exp(s_ij - m_i)
 *     o_ic  = (1 / l_i) sum_{j in A_i} exp(s_ij - m_i) v_jc
 *     lse_i = m_i + ln(l_i)          (natural-log logsumexp of the row)
 *
 *   The max subtraction only keeps exp() in range; it cancels exactly in the
 *   ratio, so the result is the textbook softmax.  The caller passes `scale`
 *   (1/sqrt(d) in the formula) so that the oracle and the GPU see the same
 *   number.
 *
 * Layout: q, k, v are contiguous [B, H, N, d] fp64 arrays (each (b, h) pair is
 * one N x d matrix of the formula); o is [B, H, N, d] and lse is [B, H, N].
 * Two passes per query row, N doubles of scratch per thread, OpenMP over rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* One output row: query i of the head whose K/V start at k, v. */
static void attend_one_row(const double *qi, const double *k, const double *v,
                           int64_t N, int64_t d, int causal, double scale,
                           int64_t i, double *s, double *o_row, double *lse_out)
{
    const int64_t nvis = causal ? (i + 1 < N ? i + 1 : N) : N; /* |A_i| */
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        const double *kj = k + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double *vj = v + j * d;
        const double p = s[j];
        for (int64_t c = 0; c < d; ++c) o_row[c] += p * vj[c];
    }
    for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
    *lse_out = m + log(l);
}

/*
 * Selected rows.  rows[r] is a flat row index (b*H + h)*N + i.  Row r of the
 * result goes to o[r*d .. r*d+d) and lse[r].  Returns 0, or -1 on a bad
 * argument / allocation failure.
 */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          int causal, double scale,
                          const int64_t *rows, int64_t nrows,
                          double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse || (nrows > 0 && !rows)) return -1;
    if (B < 1 || H < 1 || N < 1 || d < 1 || nrows < 0) return -1;
    const int64_t total = B * H * N;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t flat = rows[r];
                const int64_t bh = flat / N, i = flat % N;
                const double *kh = k + bh * N * d, *vh = v + bh * N * d;
                attend_one_row(q + flat * d, kh, vh, N, d, causal, scale, i, s,
                               o + r * d, lse + r);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* Every row: o and lse have the full [B,H,N,d] / [B,H,N] shapes. */
int oracle_attention(const double *q, const double *k, const double *v,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                     double scale, double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || H < 1 || N < 1 || d < 1) return -1;
    const int64_t total = B * H * N;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t flat = 0; flat < total; ++flat) {
                const int64_t bh = flat / N, i = flat % N;
                const double *kh = k + bh * N * d, *vh = v + bh * N * d;
                attend_one_row(q + flat * d, kh, vh, N, d, causal, scale, i, s,
                               o + flat * d, lse + flat);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
