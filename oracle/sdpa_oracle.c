/*
 * sdpa_oracle.c -- plain fp64 CPU oracle for multi-head scaled dot-product
 * attention, forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the ground truth that the HIP path is
 * checked against.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load it.  It shares no code, header or constant with the
 * HIP library and must never be used to produce a product result.
 *
 * What it computes (one definition, written out; no blocking, no fusion, no
 * online rescaling):
 *
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *     -- page "Attention Is All You Need/paper/es", §3.2.1, Eq. (1): dot products
 *        of the query with every key, each divided by sqrt(d_k), a softmax for
 *        the weights, and the output as the weighted sum of the values (§3.2).
 *
 *   Masking: "illegal connections" get the score -infinity before the softmax
 *     -- same page, §3.2.3 (decoder self-attention may attend to every position
 *        up to and including its own).  Page "Arquitectura Transformer",
 *        section "Cómo hacerlo": a score of -infinity has exponential 0, and the
 *        triangular mask keeps the current and earlier positions, rows being
 *        queries and columns keys.
 *
 *   Restricted self-attention: each output position considers only a
 *     neighbourhood of size r of the input sequence centred on it -- same
 *     page, §4 and Table 1 (work O(r n d), path length O(n / r)).  Reading
 *     taken: the neighbourhood is given by its radius w >= 0, key j being
 *     legal for query i only when |i - j| <= w (r = 2w + 1 positions, fewer at
 *     the ends of the sequence); a negative radius means no restriction.  It
 *     combines with the two masks below.
 *
 *   Key padding (readings stated where the pages are silent):
 *     key j is illegal for every query of sequence b when j >= len_b, with
 *     len_b = clamp(key_lengths[b], 0, Lk) (Lk when key_lengths is NULL);
 *     causal masking is top-left aligned: key j is illegal for query i when j > i;
 *     a row whose every key is illegal has output 0 and all weights 0.
 *
 *   Softmax: exponentials divided by their sum (page "Arquitectura Transformer",
 *     "Cómo funciona").  The row maximum is subtracted before exponentiating;
 *     softmax is unchanged by a common shift of its inputs (page
 *     "Self-Attention คืออะไร (แบบจับต้องได้)", section on dividing by sqrt(d_k):
 *     [100,100,100] splits exactly like [0,0,0]).
 *
 * Layout: Q [B,H,Lq,d_k], K [B,H,Lk,d_k], V [B,H,Lk,d_v], O [B,H,Lq,d_v],
 * all fp64, contiguous, row-major.  Heads and batch entries are independent
 * (§3.2.2: the h heads run in parallel).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: IEEE semantics are
 * relied upon for exp(-inf) == 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Is key j a legal connection for query i of a sequence with len keys? */
static int is_legal(int64_t i, int64_t j, int64_t len, int causal, int64_t radius)
{
    if (j >= len) return 0;             /* key padding */
    if (causal && j > i) return 0;      /* future position */
    if (radius >= 0 && (j < i - radius || j > i + radius)) return 0;   /* outside the neighbourhood */
    return 1;
}

static int64_t clamp_len(const int32_t *key_lengths, int64_t b, int64_t Lk)
{
    if (!key_lengths) return Lk;
    int64_t l = key_lengths[b];
    if (l < 0) l = 0;
    if (l > Lk) l = Lk;
    return l;
}

/*
 * One query row: q[d_k] against K[Lk][d_k], V[Lk][d_v].
 *   s[j]  = (q . k_j) / sqrt(d_k), or -inf if illegal     (Eq. 1, §3.2.3)
 *   w[j]  = exp(s[j] - max_j s[j])                        (softmax numerator)
 *   p[j]  = w[j] / sum_j w[j]                             (weights, sum to 1)
 *   o[t]  = sum_j p[j] * V[j][t]                          (weighted sum of values)
 * s and w are caller-provided scratch of length Lk.  p_out (length Lk) and lse
 * (log of the softmax denominator of the scaled scores, m + log Z) are optional.
 */
static void attention_row(const double *q, const double *K, const double *V,
                          int64_t Lk, int64_t d_k, int64_t d_v, int64_t len,
                          int causal, int64_t radius, int64_t i, double *s, double *w,
                          double *o, double *p_out, double *lse)
{
    const double root_dk = sqrt((double)d_k);
    for (int64_t j = 0; j < Lk; ++j) {
        if (!is_legal(i, j, len, causal, radius)) {
            s[j] = -INFINITY;
            continue;
        }
        const double *k = K + j * d_k;
        double dot = 0.0;
        for (int64_t t = 0; t < d_k; ++t) dot += q[t] * k[t];
        s[j] = dot / root_dk;
    }

    double m = -INFINITY;
    for (int64_t j = 0; j < Lk; ++j)
        if (s[j] > m) m = s[j];

    if (m == -INFINITY) {               /* no legal key: empty weighted sum */
        for (int64_t t = 0; t < d_v; ++t) o[t] = 0.0;
        if (p_out) for (int64_t j = 0; j < Lk; ++j) p_out[j] = 0.0;
        if (lse) *lse = -INFINITY;
        return;
    }

    double Z = 0.0;
    for (int64_t j = 0; j < Lk; ++j) {
        w[j] = exp(s[j] - m);           /* exp(-inf) == 0 exactly */
        Z += w[j];
    }
    for (int64_t j = 0; j < Lk; ++j) w[j] = w[j] / Z;   /* w now holds p */

    for (int64_t t = 0; t < d_v; ++t) o[t] = 0.0;
    for (int64_t j = 0; j < Lk; ++j) {
        const double pj = w[j];
        const double *v = V + j * d_v;
        for (int64_t t = 0; t < d_v; ++t) o[t] += pj * v[t];
    }
    if (p_out) memcpy(p_out, w, (size_t)Lk * sizeof(double));
    if (lse) *lse = m + log(Z);
}

static int bad_shape(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d_k, int64_t d_v)
{
    return B < 0 || H < 0 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1;
}

/*
 * Full attention over every (b, head, i); radius < 0: no neighbourhood
 * restriction.
 *   O   [B,H,Lq,d_v]  required
 *   P   [B,H,Lq,Lk]   optional (NULL): the softmax weights
 *   LSE [B,H,Lq]      optional (NULL)
 * Returns 0 on success, 1 on a bad shape, 2 on allocation failure.
 */
int oracle_attention(const double *Q, const double *K, const double *V,
                     const int32_t *key_lengths, int causal, int64_t radius,
                     int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                     int64_t d_k, int64_t d_v,
                     double *O, double *P, double *LSE, int nthreads)
{
    if (bad_shape(B, H, Lq, Lk, d_k, d_v)) return 1;
    const int64_t nrows = B * H * Lq;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
        double *w = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
        if (!s || !w) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t i = r % Lq;
                const int64_t bh = r / Lq;
                const int64_t b = bh / H;
                const double *Kh = K + bh * Lk * d_k;
                const double *Vh = V + bh * Lk * d_v;
                attention_row(Q + r * d_k, Kh, Vh, Lk, d_k, d_v,
                              clamp_len(key_lengths, b, Lk), causal, radius, i, s, w,
                              O + r * d_v, P ? P + r * Lk : NULL,
                              LSE ? LSE + r : NULL);
            }
        }
        free(s);
        free(w);
    }
    return failed ? 2 : 0;
}

/*
 * Attention for a chosen set of rows only.  rows[n] is the flat row index
 * (b*H + head)*Lq + i.  O_rows is [nrows, d_v]; LSE_rows is optional [nrows].
 * Same definition as oracle_attention, row by row.
 */
int oracle_attention_rows(const double *Q, const double *K, const double *V,
                          const int32_t *key_lengths, int causal, int64_t radius,
                          int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                          int64_t d_k, int64_t d_v,
                          const int64_t *rows, int64_t nrows,
                          double *O_rows, double *LSE_rows, int nthreads)
{
    if (bad_shape(B, H, Lq, Lk, d_k, d_v)) return 1;
    for (int64_t n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= B * H * Lq) return 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
        double *w = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
        if (!s || !w) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t n = 0; n < nrows; ++n) {
                const int64_t r = rows[n];
                const int64_t i = r % Lq;
                const int64_t bh = r / Lq;
                const int64_t b = bh / H;
                attention_row(Q + r * d_k, K + bh * Lk * d_k, V + bh * Lk * d_v,
                              Lk, d_k, d_v, clamp_len(key_lengths, b, Lk), causal, radius, i,
                              s, w, O_rows + n * d_v, NULL,
                              LSE_rows ? LSE_rows + n : NULL);
            }
        }
        free(s);
        free(w);
    }
    return failed ? 2 : 0;
}

/*
 * Multi-head attention -- page "Attention Is All You Need/paper/es", §3.2.2:
 *
 *   MultiHead(Q, K, V) = Concat(head_1, ..., head_h) W^O
 *   head_i             = Attention(Q W_i^Q, K W_i^K, V W_i^V)
 *
 * with W_i^Q, W_i^K in R^{d_model x d_k}, W_i^V in R^{d_model x d_v} and
 * W^O in R^{h d_v x d_model}; Attention is oracle_attention above (Eq. (1) with
 * the masks).  Q is the sequence the queries come from (Xq), K = V the one the
 * keys and values come from (Xkv; the same sequence for self-attention).
 *
 * Storage, all fp64 row-major:
 *   Xq [B][Lq][d_model], Xkv [B][Lk][d_model], O [B][Lq][d_model];
 *   Wq [d_model][h*d_k]: W_i^Q is columns i*d_k .. i*d_k + d_k - 1 (Wk alike),
 *   Wv [d_model][h*d_v], Wo [h*d_v][d_model]: row i*d_v + t multiplies
 *   component t of head i in the concatenation.
 * Returns 0 on success, 1 on a bad shape, 2 on allocation failure.
 */
/* y[n] = sum_c x[c] * W[c][n] for one row x (W row-major [d_model][n_cols]):
 * the product of a row with W_i for all heads i at once.  Loops over c, then
 * n, so that W is read along its rows. */
static void row_times(const double *x, const double *W, int64_t d_model, int64_t n_cols, double *y)
{
    for (int64_t n = 0; n < n_cols; ++n) y[n] = 0.0;
    for (int64_t c = 0; c < d_model; ++c) {
        const double xc = x[c];
        const double *w = W + c * n_cols;
        for (int64_t n = 0; n < n_cols; ++n) y[n] += xc * w[n];
    }
}

/* Split a projected row y[h*d] into head-major storage P[b][h][L][d] at position i. */
static void scatter_heads(const double *y, int64_t h, int64_t d, int64_t b, int64_t L, int64_t i,
                          double *P)
{
    for (int64_t hd = 0; hd < h; ++hd)
        for (int64_t t = 0; t < d; ++t) P[((b * h + hd) * L + i) * d + t] = y[hd * d + t];
}

int oracle_multihead(const double *Xq, const double *Xkv, const double *Wq, const double *Wk,
                     const double *Wv, const double *Wo, const int32_t *key_lengths, int causal,
                     int64_t B, int64_t Lq, int64_t Lk, int64_t d_model, int64_t h,
                     int64_t d_k, int64_t d_v, double *O, int nthreads)
{
    if (B < 0 || Lq < 0 || Lk < 0 || d_model < 1 || h < 1 || d_k < 1 || d_v < 1) return 1;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#endif
    const size_t nq = (size_t)(B * h * Lq), nk = (size_t)(B * h * Lk);
    const int64_t wide = h * (d_k > d_v ? d_k : d_v);
    double *Qp = (double *)malloc((nq * d_k + 1) * sizeof(double));
    double *Kp = (double *)malloc((nk * d_k + 1) * sizeof(double));
    double *Vp = (double *)malloc((nk * d_v + 1) * sizeof(double));
    double *A = (double *)malloc((nq * d_v + 1) * sizeof(double));
    int rc = 0;
    if (!Qp || !Kp || !Vp || !A) {
        rc = 2;
        goto done;
    }

    /* The h projections of each position: row x of the source sequence times
     * W_i (Q W_i^Q etc.), stored per head as [B][h][L][d]. */
#pragma omp parallel num_threads(nthreads)
    {
        double *y = (double *)malloc((size_t)(wide > d_model ? wide : d_model) * sizeof(double));
        if (!y) {
#pragma omp atomic write
            rc = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < B * Lq; ++r) {
                row_times(Xq + r * d_model, Wq, d_model, h * d_k, y);
                scatter_heads(y, h, d_k, r / Lq, Lq, r % Lq, Qp);
            }
#pragma omp for schedule(static)
            for (int64_t r = 0; r < B * Lk; ++r) {
                row_times(Xkv + r * d_model, Wk, d_model, h * d_k, y);
                scatter_heads(y, h, d_k, r / Lk, Lk, r % Lk, Kp);
                row_times(Xkv + r * d_model, Wv, d_model, h * d_v, y);
                scatter_heads(y, h, d_v, r / Lk, Lk, r % Lk, Vp);
            }
        }
        free(y);
    }
    if (rc != 0) goto done;

    /* head_i for every head (the attention of §3.2.1 on the projections) */
    rc = oracle_attention(Qp, Kp, Vp, key_lengths, causal, -1, B, h, Lq, Lk, d_k, d_v, A, NULL,
                          NULL, nthreads);
    if (rc != 0) goto done;

    /* Concat(head_1, ..., head_h) W^O: component t of head i is column
     * i*d_v + t of the concatenation. */
#pragma omp parallel num_threads(nthreads)
    {
        double *cat = (double *)malloc((size_t)(h * d_v) * sizeof(double));
        if (!cat) {
#pragma omp atomic write
            rc = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < B * Lq; ++r) {
                const int64_t b = r / Lq, i = r % Lq;
                for (int64_t hd = 0; hd < h; ++hd)
                    for (int64_t t = 0; t < d_v; ++t)
                        cat[hd * d_v + t] = A[((b * h + hd) * Lq + i) * d_v + t];
                row_times(cat, Wo, h * d_v, d_model, O + r * d_model);
            }
        }
        free(cat);
    }

done:
    free(Qp);
    free(Kp);
    free(Vp);
    free(A);
    return rc;
}

/*
 * oracle_multihead for chosen output rows only: rows[n] = b * Lq + i.  The keys
 * and values of every batch entry involved are projected in full (a row may
 * use any of them); queries only for the chosen rows.  O_rows [nrows][d_model].
 */
int oracle_multihead_rows(const double *Xq, const double *Xkv, const double *Wq,
                          const double *Wk, const double *Wv, const double *Wo,
                          const int32_t *key_lengths, int causal, int64_t B, int64_t Lq,
                          int64_t Lk, int64_t d_model, int64_t h, int64_t d_k, int64_t d_v,
                          const int64_t *rows, int64_t nrows, double *O_rows, int nthreads)
{
    if (B < 0 || Lq < 0 || Lk < 0 || d_model < 1 || h < 1 || d_k < 1 || d_v < 1) return 1;
    for (int64_t n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= B * Lq) return 1;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#endif
    const int64_t wide = h * (d_k > d_v ? d_k : d_v);
    const size_t hk = (size_t)(h * Lk);
    double *Kp = (double *)malloc((hk * d_k + 1) * sizeof(double));
    double *Vp = (double *)malloc((hk * d_v + 1) * sizeof(double));
    int rc = 0;
    if (!Kp || !Vp) {
        rc = 2;
        goto out;
    }
    for (int64_t b = 0; b < B; ++b) {
        int used = 0;
        for (int64_t n = 0; n < nrows; ++n) used |= rows[n] / Lq == b;
        if (!used) continue;
        /* keys and values of batch entry b, as [1][h][Lk][d] */
#pragma omp parallel num_threads(nthreads)
        {
            double *y = (double *)malloc((size_t)wide * sizeof(double));
            if (!y) {
#pragma omp atomic write
                rc = 2;
            } else {
#pragma omp for schedule(static)
                for (int64_t j = 0; j < Lk; ++j) {
                    row_times(Xkv + (b * Lk + j) * d_model, Wk, d_model, h * d_k, y);
                    scatter_heads(y, h, d_k, 0, Lk, j, Kp);
                    row_times(Xkv + (b * Lk + j) * d_model, Wv, d_model, h * d_v, y);
                    scatter_heads(y, h, d_v, 0, Lk, j, Vp);
                }
            }
            free(y);
        }
        if (rc != 0) goto out;
        const int64_t len = clamp_len(key_lengths, b, Lk);
#pragma omp parallel num_threads(nthreads)
        {
            double *q = (double *)malloc((size_t)(h * d_k + 1) * sizeof(double));
            double *cat = (double *)malloc((size_t)(h * d_v + 1) * sizeof(double));
            double *sc = (double *)malloc((size_t)(Lk + 1) * sizeof(double));
            double *w = (double *)malloc((size_t)(Lk + 1) * sizeof(double));
            if (!q || !cat || !sc || !w) {
#pragma omp atomic write
                rc = 2;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t n = 0; n < nrows; ++n) {
                    if (rows[n] / Lq != b) continue;
                    const int64_t i = rows[n] % Lq;
                    row_times(Xq + rows[n] * d_model, Wq, d_model, h * d_k, q);
                    for (int64_t hd = 0; hd < h; ++hd)
                        attention_row(q + hd * d_k, Kp + hd * Lk * d_k, Vp + hd * Lk * d_v, Lk, d_k,
                                      d_v, len, causal, -1, i, sc, w, cat + hd * d_v, NULL, NULL);
                    row_times(cat, Wo, h * d_v, d_model, O_rows + n * d_model);
                }
            }
            free(q);
            free(cat);
            free(sc);
            free(w);
        }
        if (rc != 0) goto out;
    }
out:
    free(Kp);
    free(Vp);
    return rc;
}
