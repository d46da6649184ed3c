/*
 * fa_ref.c -- fp64 CPU oracle for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the
 * benchmark's CPU-baseline leg call this library; the product path
 * (libfa355 and its Python binding) never loads, links or calls it, and the
 * two share no source, header, table or helper.
 *
 * What is computed (page "Mini FlashAttention", section 1 "What attention
 * is"): for one head with rows q_i, k_j, v_j of length d,
 *     s_ij = scale * <q_i, k_j>,   P_i = softmax over the allowed j of s_ij,
 *     O_i  = sum_j P_ij v_j,
 * where "allowed" is every key j < n, or, with the causal mask of the same
 * section, only j <= i.  The running statistics the pages carry (max m and
 * denominator l) give one more per-row output, the log-sum-exp
 *     lse_i = ln sum_{j allowed} exp(s_ij) = m_i + ln l_i,
 * natural log, which the pages do not print; it is defined here by that
 * formula.  A row with no allowed key (never the case for a real query of a
 * square problem) yields O_i = 0 and lse_i = -inf.
 *
 * Algorithm of fa_ref_fwd* : the plain three-pass safe softmax, one row at a
 * time (page "How Did I Write My First FlashAttention Kernel in CUDA?", the
 * passage on softmax normally needing three passes over the data: the max,
 * then the sum of exponentials, then the normalisation), followed by P.V --
 * the naive "golden reference" of the grasp.study lesson, section
 * "Verification: Does It Actually Work?".  Scores live in a length-n fp64
 * row buffer; the n x n matrix is never formed.
 *
 * fa_ref_online() is the second, independent algorithm: the chunked
 * running-state recurrence of "Mini FlashAttention", section 4 "The flash
 * trick: online softmax", including its guard that replaces a -inf running
 * max by 0 so fully masked rows cannot produce NaN.  It exists to be checked
 * against the three-pass result for every chunk size.
 *
 * All arithmetic is fp64: inputs are fp32 arrays holding exactly the values
 * the GPU sees (bf16 inputs are widened exactly), and the scale is the fp32
 * value handed to the GPU, widened to double.
 *
 * Layouts (strides in elements):
 *   fixed length : q, k, v [B, H, N, d] contiguous; o [B, H, N, d]; lse [B, H, N]
 *   packed varlen: q, k, v [T, H, d] with T = cu_seqlens[nseq]; o [T, H, d]; lse [T, H]
 *   decode       : q, o [B, H, Nq, d]; k, v [B, H, Nk, d]; lse [B, H, Nq]
 * Return value: 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Plain three-pass attention for one query row against `nkeys` allowed keys
 * (keys 0..nkeys-1; the causal mask of a square problem leaves a prefix).
 * buf must hold nkeys doubles. */
static void row_three_pass(const float *q, const float *kb, long ks,
                           const float *vb, long vs, int nkeys, int d,
                           double scale, double *buf, double *o, double *lse)
{
    int j, c;
    double m = -INFINITY, l = 0.0;

    for (c = 0; c < d; ++c)
        o[c] = 0.0;
    if (nkeys <= 0) {
        *lse = -INFINITY;
        return;
    }
    /* pass 1: scores and their maximum */
    for (j = 0; j < nkeys; ++j) {
        const float *kr = kb + (long)j * ks;
        double acc = 0.0;
        for (c = 0; c < d; ++c)
            acc += (double)q[c] * (double)kr[c];
        buf[j] = scale * acc;
        if (buf[j] > m)
            m = buf[j];
    }
    /* pass 2: shifted exponentials and their sum */
    for (j = 0; j < nkeys; ++j) {
        buf[j] = exp(buf[j] - m);
        l += buf[j];
    }
    /* pass 3: normalised weights times V */
    for (j = 0; j < nkeys; ++j) {
        const float *vr = vb + (long)j * vs;
        double w = buf[j] / l;
        for (c = 0; c < d; ++c)
            o[c] += w * (double)vr[c];
    }
    *lse = m + log(l);
}

static int allowed_keys(int i, int n, int causal)
{
    if (!causal)
        return n;
    return i + 1 < n ? i + 1 : n;
}

void fa_ref_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int fa_ref_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Fixed-length batch, all rows. */
int fa_ref_fwd(const float *q, const float *k, const float *v, double *o,
               double *lse, int B, int H, int N, int d, double scale,
               int causal)
{
    long nrows, r;
    int bad = 0;

    if (!q || !k || !v || !o || !lse || B < 0 || H < 0 || N < 0 || d <= 0)
        return -1;
    nrows = (long)B * H * N;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (N > 0 ? N : 1));
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (r = 0; r < nrows; ++r) {
            long bh = r / N;
            int i = (int)(r % N);
            const float *kb = k + bh * N * (long)d;
            const float *vb = v + bh * N * (long)d;
            if (!buf)
                continue;
            row_three_pass(q + r * d, kb, d, vb, d, allowed_keys(i, N, causal),
                           d, scale, buf, o + r * d, lse + r);
        }
        free(buf);
    }
    return bad ? -2 : 0;
}

/* Fixed-length batch, selected rows only.  rows[t] is a flat index into
 * [B, H, N]; o_rows is [nrows, d], lse_rows is [nrows]. */
int fa_ref_fwd_rows(const float *q, const float *k, const float *v,
                    int B, int H, int N, int d, double scale, int causal,
                    const long long *rows, int nrows, double *o_rows,
                    double *lse_rows)
{
    int t, bad = 0;
    long total = (long)B * H * N;

    if (!q || !k || !v || !rows || !o_rows || !lse_rows || N <= 0 || d <= 0 ||
        nrows < 0)
        return -1;
    for (t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= total)
            return -1;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * N);
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (t = 0; t < nrows; ++t) {
            long r = (long)rows[t];
            long bh = r / N;
            int i = (int)(r % N);
            if (!buf)
                continue;
            row_three_pass(q + r * d, k + bh * N * (long)d, d,
                           v + bh * N * (long)d, d, allowed_keys(i, N, causal),
                           d, scale, buf, o_rows + (long)t * d, lse_rows + t);
        }
        free(buf);
    }
    return bad ? -2 : 0;
}

static int check_cu(const int *cu, int nseq)
{
    int s;
    if (cu[0] != 0)
        return -1;
    for (s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s])
            return -1;
    return 0;
}

static int seq_of_token(const int *cu, int nseq, long t)
{
    int lo = 0, hi = nseq - 1;
    while (lo < hi) { /* last s with cu[s] <= t */
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

static int max_len(const int *cu, int nseq)
{
    int s, m = 1;
    for (s = 0; s < nseq; ++s)
        if (cu[s + 1] - cu[s] > m)
            m = cu[s + 1] - cu[s];
    return m;
}

/* Packed variable-length batch, all rows.  Each sequence s owns tokens
 * cu[s] .. cu[s+1]-1 and attends only within itself; the causal mask uses
 * positions local to the sequence. */
int fa_ref_fwd_varlen(const float *q, const float *k, const float *v,
                      double *o, double *lse, const int *cu, int nseq, int H,
                      int d, double scale, int causal)
{
    long nrows, r;
    int bad = 0, mlen;

    if (!q || !k || !v || !o || !lse || !cu || nseq <= 0 || H <= 0 || d <= 0)
        return -1;
    if (check_cu(cu, nseq))
        return -1;
    nrows = (long)cu[nseq] * H;
    mlen = max_len(cu, nseq);
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * mlen);
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (r = 0; r < nrows; ++r) {
            long tok = r / H;
            int h = (int)(r % H);
            int s = seq_of_token(cu, nseq, tok);
            long base = (long)cu[s];
            int n = cu[s + 1] - cu[s];
            int i = (int)(tok - base);
            long hs = (long)H * d;
            if (!buf)
                continue;
            row_three_pass(q + r * d, k + base * hs + (long)h * d, hs,
                           v + base * hs + (long)h * d, hs,
                           allowed_keys(i, n, causal), d, scale, buf,
                           o + r * d, lse + r);
        }
        free(buf);
    }
    return bad ? -2 : 0;
}

/* Packed variable-length batch, selected rows: rows[t] = token * H + head. */
int fa_ref_fwd_varlen_rows(const float *q, const float *k, const float *v,
                           const int *cu, int nseq, int H, int d, double scale,
                           int causal, const long long *rows, int nrows,
                           double *o_rows, double *lse_rows)
{
    int t, bad = 0, mlen;
    long total;

    if (!q || !k || !v || !cu || !rows || !o_rows || !lse_rows || nseq <= 0 ||
        H <= 0 || d <= 0 || nrows < 0)
        return -1;
    if (check_cu(cu, nseq))
        return -1;
    total = (long)cu[nseq] * H;
    for (t = 0; t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= total)
            return -1;
    mlen = max_len(cu, nseq);
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * mlen);
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (t = 0; t < nrows; ++t) {
            long r = (long)rows[t];
            long tok = r / H;
            int h = (int)(r % H);
            int s = seq_of_token(cu, nseq, tok);
            long base = (long)cu[s];
            int n = cu[s + 1] - cu[s];
            int i = (int)(tok - base);
            long hs = (long)H * d;
            if (!buf)
                continue;
            row_three_pass(q + r * d, k + base * hs + (long)h * d, hs,
                           v + base * hs + (long)h * d, hs,
                           allowed_keys(i, n, causal), d, scale, buf,
                           o_rows + (long)t * d, lse_rows + t);
        }
        free(buf);
    }
    return bad ? -2 : 0;
}

/* Decode-shaped batch: per (batch, head), Nq queries against Nk keys.
 * q, o [B, H, Nq, d]; k, v [B, H, Nk, d]; lse [B, H, Nq].  "Mini
 * FlashAttention", section 1, ties the causal mask to autoregressive decoding
 * (a token never sees a later one) without fixing the shapes of a decode
 * step; the reading taken here is that the Nq queries are the newest Nq
 * positions of an Nk-long sequence.  The mask (key j hidden from query i
 * when j > i, positions in the whole sequence) then lets query i, 0-based
 * among the Nq, see keys 0 .. Nk - Nq + i.  Without the mask every query sees all Nk keys.  A query
 * that sees no key (causal with Nq > Nk) gives O = 0 and lse = -inf. */
static int visible_keys_decode(int i, int nq, int nk, int causal)
{
    long last; /* position of the query in the whole sequence */
    if (!causal)
        return nk;
    last = (long)nk - nq + i;
    if (last < 0)
        return 0;
    return last + 1 < nk ? (int)(last + 1) : nk;
}

int fa_ref_fwd_decode(const float *q, const float *k, const float *v,
                      double *o, double *lse, int B, int H, int Nq, int Nk,
                      int d, double scale, int causal)
{
    long nrows, r;
    int bad = 0;

    if (!q || !k || !v || !o || !lse || B < 0 || H < 0 || Nq < 0 || Nk < 0 ||
        d <= 0)
        return -1;
    nrows = (long)B * H * Nq;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
        if (!buf) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (r = 0; r < nrows; ++r) {
            long bh = r / (Nq > 0 ? Nq : 1);
            int i = (int)(r % (Nq > 0 ? Nq : 1));
            if (!buf)
                continue;
            row_three_pass(q + r * d, k + bh * Nk * (long)d, d,
                           v + bh * Nk * (long)d, d,
                           visible_keys_decode(i, Nq, Nk, causal), d, scale,
                           buf, o + r * d, lse + r);
        }
        free(buf);
    }
    return bad ? -2 : 0;
}

/* The chunked running-state recurrence ("Mini FlashAttention", section 4),
 * one head [n, d], fp64.  For every row: m = -inf, l = 0, acc = 0; for each
 * chunk of `chunk` consecutive keys (restricted to the allowed ones):
 *     m_new = max(m, max_j s_j), replaced by 0 if it is -inf (ghost guard)
 *     alpha = exp(m - m_new),  p_j = exp(s_j - m_new)
 *     l = l * alpha + sum_j p_j,  acc = acc * alpha + sum_j p_j v_j,  m = m_new
 * and finally O = acc / l, lse = m + ln l (O = 0, lse = -inf when l = 0). */
int fa_ref_online(const float *q, const float *k, const float *v, double *o,
                  double *lse, int n, int d, double scale, int causal,
                  int chunk)
{
    int i, bad = 0;

    if (!q || !k || !v || !o || !lse || n < 0 || d <= 0 || chunk <= 0)
        return -1;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * chunk);
        double *acc = (double *)malloc(sizeof(double) * d);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (i = 0; i < n; ++i) {
            const float *qi = q + (long)i * d;
            int nk = allowed_keys(i, n, causal);
            double m = -INFINITY, l = 0.0;
            int j0, j, c;
            if (!s || !acc)
                continue;
            for (c = 0; c < d; ++c)
                acc[c] = 0.0;
            for (j0 = 0; j0 < n; j0 += chunk) {
                int w = (n - j0 < chunk) ? n - j0 : chunk;
                double cmax = -INFINITY, m_new, alpha, psum = 0.0;
                for (j = 0; j < w; ++j) {
                    int key = j0 + j;
                    if (key < nk) {
                        const float *kr = k + (long)key * d;
                        double dot = 0.0;
                        for (c = 0; c < d; ++c)
                            dot += (double)qi[c] * (double)kr[c];
                        s[j] = scale * dot;
                    } else {
                        s[j] = -INFINITY; /* masked key */
                    }
                    if (s[j] > cmax)
                        cmax = s[j];
                }
                m_new = m > cmax ? m : cmax;
                if (m_new == -INFINITY)
                    m_new = 0.0;
                alpha = exp(m - m_new);
                for (c = 0; c < d; ++c)
                    acc[c] *= alpha;
                for (j = 0; j < w; ++j) {
                    double p = exp(s[j] - m_new);
                    const float *vr = v + (long)(j0 + j) * d;
                    psum += p;
                    if (p != 0.0)
                        for (c = 0; c < d; ++c)
                            acc[c] += p * (double)vr[c];
                }
                l = l * alpha + psum;
                m = m_new;
            }
            for (c = 0; c < d; ++c)
                o[(long)i * d + c] = l > 0.0 ? acc[c] / l : 0.0;
            lse[i] = l > 0.0 ? m + log(l) : -INFINITY;
        }
        free(s);
        free(acc);
    }
    return bad ? -2 : 0;
}
