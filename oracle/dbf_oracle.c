/*
 * dbf_oracle.c -- plain, slow, fp64 CPU oracle for the double-binary
 * factorized linear layer.  TEST INFRASTRUCTURE ONLY: tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the product path never
 * does.  It shares no code, header, table or layout helper with the HIP
 * library.
 *
 * What it computes (read right to left, one token at a time):
 *
 *   y = sum_{i=1..L} diag(alpha_i) B1_i diag(beta_i) B2_i diag(gamma_i) x
 *
 *   - LoRDBA: Low-Rank Double-Binary Adaptation, section 2 (Metodologia),
 *     "Arquitetura Central": the weight update Delta W is a sum over the
 *     envelope rank L of diag(alpha) B1 diag(beta) B2 diag(gamma), with
 *     B1 in {+-1}^{N x R}, B2 in {+-1}^{R x M} and fp16 scale vectors.
 *   - same page, "Kernel de Inferencia": the forward is two sign-accumulate
 *     products interleaved with per-channel scaling (additions and
 *     subtractions only inside the inner products).
 *   - "Addition is almost all you need" (DBF), technical summary section 2:
 *     W ~ (a . A . m^T)(B . b^T), the L = 1 case with a = alpha, A = B1,
 *     m = beta, B = B2, b = gamma.
 *   - "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
 *     technical summary section 2, item 2: the weight is a sum of several
 *     boolean kernels, which is the L > 1 sum.
 *   - LoRDBA section 1 and 5: the adapter stays unmerged beside a frozen
 *     base weight W0, so the adapter-mode output is W0 x + Delta W x.
 *   - Multi-Boolean page, section 2, items 1 and 2, read as written: each
 *     boolean kernel is sign(W) with a rank-one scale s_out s_in^T, and the
 *     weight is the sum of several such kernels (dbf_oracle_bool_forward).
 *
 * Signs are passed unpacked, as int8 +-1 (any value > 0 is +1), so nothing
 * here depends on a bit layout.  Each inner product is a plain sequential
 * +-add in fixed order, which makes flipping a sign an exact negation.
 * Outer loops over (token, output) run under OpenMP; every output element is
 * still summed by one thread in the same order, so the result does not depend
 * on the thread count.
 *
 * The bit-packing functions at the end write the uint32 layout out from its
 * definition (bit value 1 is +1), one bit at a time.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int dbf_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (n >= 1); the results do not
 * depend on it (every output element is summed by one thread in order). */
void dbf_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One term, one token:  y_t += diag(a) B1 diag(be) B2 diag(g) x_t.
 * u, v are scratch of length M and R. */
static void term_one_token(int64_t N, int64_t M, int64_t R,
                           const int8_t *b1, const int8_t *b2,
                           const double *a, const double *be, const double *g,
                           const double *xt, double *yt, double *u, double *v)
{
    /* diag(gamma) x */
    for (int64_t m = 0; m < M; ++m)
        u[m] = g[m] * xt[m];
    /* B2 (.): a +-add over the input features, then diag(beta) */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const int8_t *row = b2 + r * M;
        double s = 0.0;
        for (int64_t m = 0; m < M; ++m)
            s += (row[m] > 0) ? u[m] : -u[m];
        v[r] = be[r] * s;
    }
    /* B1 (.): a +-add over the inner rank, then diag(alpha), summed into y */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *row = b1 + n * R;
        double s = 0.0;
        for (int64_t r = 0; r < R; ++r)
            s += (row[r] > 0) ? v[r] : -v[r];
        yt[n] += a[n] * s;
    }
}

/* y[T x N] = sum over the L terms of Delta W_i x[t] (y is overwritten).
 * b1[i]: N x R, b2[i]: R x M, alpha[i]: N, beta[i]: R, gamma[i]: M,
 * x: T x M, all row-major.  Returns 0, or -1 if scratch cannot be had. */
int dbf_oracle_forward(int L, int64_t N, int64_t M, int64_t R, int64_t T,
                       const int8_t *const *b1, const int8_t *const *b2,
                       const double *const *alpha, const double *const *beta,
                       const double *const *gamma,
                       const double *x, double *y)
{
    double *u = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double *v = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    int64_t t, n;
    int i;
    if (!u || !v) {
        free(u);
        free(v);
        return -1;
    }
    for (t = 0; t < T; ++t) {
        double *yt = y + t * N;
        for (n = 0; n < N; ++n)
            yt[n] = 0.0;
        for (i = 0; i < L; ++i)
            term_one_token(N, M, R, b1[i], b2[i], alpha[i], beta[i], gamma[i],
                           x + t * M, yt, u, v);
    }
    free(u);
    free(v);
    return 0;
}

/* The Multi-Boolean form ("Highly Efficient and Effective LLMs with
 * Multi-Boolean Architectures", technical summary, section 2, items 1 and
 * 2): kernel k is a sign matrix Wb_k in {+-1}^{N x M} carrying the rank-one
 * scale s_out_k s_in_k^T, the weight is sum_k Wb_k . (s_out_k s_in_k^T), so
 *   y[t][n] = sum_k s_out_k[n] * sum_m Wb_k[n,m] * (s_in_k[m] * x[t][m]).
 * wb[k]: N x M row-major, s_in[k]: M, s_out[k]: N, x: T x M; y (T x N) is
 * overwritten.  Returns 0, or -1 if scratch cannot be had. */
int dbf_oracle_bool_forward(int K, int64_t N, int64_t M, int64_t T,
                            const int8_t *const *wb, const double *const *s_in,
                            const double *const *s_out, const double *x, double *y)
{
    double *xs = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    int64_t t, n, m;
    int k;
    if (!xs)
        return -1;
    for (t = 0; t < T; ++t) {
        double *yt = y + t * N;
        for (n = 0; n < N; ++n)
            yt[n] = 0.0;
        for (k = 0; k < K; ++k) {
            /* diag(s_in) x */
            for (m = 0; m < M; ++m)
                xs[m] = s_in[k][m] * x[t * M + m];
            /* the boolean kernel: a +-add over the inputs, then diag(s_out) */
#pragma omp parallel for schedule(static)
            for (int64_t o = 0; o < N; ++o) {
                const int8_t *wrow = wb[k] + o * M;
                double acc = 0.0;
                for (int64_t q = 0; q < M; ++q)
                    acc += (wrow[q] > 0) ? xs[q] : -xs[q];
                yt[o] += s_out[k][o] * acc;
            }
        }
    }
    free(xs);
    return 0;
}

/* Backward of dbf_oracle_forward for a loss with gradient dy = dL/dy, by
 * the chain rule through the LoRDBA parametrization (section 2,
 * "Arquitetura Central"), read right to left per term i and token t:
 *   u = gamma . x,  s = B2 u,  w = beta . s,  z = B1 w,  y += alpha . z
 * so, going back,
 *   e = alpha . dy,  g = B1^T e,  f = beta . g,  h = B2^T f
 *   dalpha += dy . z,  dbeta += s . g,  dgamma += x . h,  dx += gamma . h
 * (B^T v is a +-add down a column of B).  Every output is overwritten;
 * token sums run in token order.  Returns 0, or -1 if scratch cannot be had. */
int dbf_oracle_backward(int L, int64_t N, int64_t M, int64_t R, int64_t T,
                        const int8_t *const *b1, const int8_t *const *b2,
                        const double *const *alpha, const double *const *beta,
                        const double *const *gamma, const double *x,
                        const double *dy, double *dx, double *dalpha,
                        double *dbeta, double *dgamma)
{
    double *u = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double *sv = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    double *z = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    int64_t t, idx;
    int i;
    if (!u || !sv || !z || !g || !h) {
        free(u); free(sv); free(z); free(g); free(h);
        return -1;
    }
    for (idx = 0; idx < T * M; ++idx)
        dx[idx] = 0.0;
    for (idx = 0; idx < (int64_t)L * N; ++idx)
        dalpha[idx] = 0.0;
    for (idx = 0; idx < (int64_t)L * R; ++idx)
        dbeta[idx] = 0.0;
    for (idx = 0; idx < (int64_t)L * M; ++idx)
        dgamma[idx] = 0.0;
    for (t = 0; t < T; ++t) {
        const double *xt = x + t * M, *dyt = dy + t * N;
        for (i = 0; i < L; ++i) {
            const int8_t *B1 = b1[i], *B2 = b2[i];
            const double *al = alpha[i], *be = beta[i], *ga = gamma[i];
            /* forward intermediates s = B2 (gamma . x) and z = B1 (beta . s) */
            for (int64_t m = 0; m < M; ++m)
                u[m] = ga[m] * xt[m];
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int64_t m = 0; m < M; ++m)
                    acc += (B2[r * M + m] > 0) ? u[m] : -u[m];
                sv[r] = acc;
            }
#pragma omp parallel for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t r = 0; r < R; ++r)
                    acc += (B1[n * R + r] > 0) ? be[r] * sv[r] : -(be[r] * sv[r]);
                z[n] = acc;
            }
            /* g = B1^T (alpha . dy): down column r of B1 */
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += (B1[n * R + r] > 0) ? al[n] * dyt[n] : -(al[n] * dyt[n]);
                g[r] = acc;
            }
            /* h = B2^T (beta . g): down column m of B2 */
#pragma omp parallel for schedule(static)
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t r = 0; r < R; ++r)
                    acc += (B2[r * M + m] > 0) ? be[r] * g[r] : -(be[r] * g[r]);
                h[m] = acc;
            }
            for (int64_t n = 0; n < N; ++n)
                dalpha[(int64_t)i * N + n] += dyt[n] * z[n];
            for (int64_t r = 0; r < R; ++r)
                dbeta[(int64_t)i * R + r] += sv[r] * g[r];
            for (int64_t m = 0; m < M; ++m) {
                dgamma[(int64_t)i * M + m] += xt[m] * h[m];
                dx[t * M + m] += ga[m] * h[m];
            }
        }
    }
    free(u); free(sv); free(z); free(g); free(h);
    return 0;
}

/* The dense base of adapter mode: y[t] += W0 x[t], W0 is N x M row-major. */
void dbf_oracle_dense(int64_t N, int64_t M, int64_t T, const double *w0,
                      const double *x, double *y)
{
    for (int64_t t = 0; t < T; ++t) {
        const double *xt = x + t * M;
        double *yt = y + t * N;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            const double *row = w0 + n * M;
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m)
                s += row[m] * xt[m];
            yt[n] += s;
        }
    }
}

/* Exact integer sign sums for int8 activations (gamma folded into x):
 *   s1[i][t][r] = sum_m B2_i[r,m] x[t,m]
 *   s2[i][t][n] = sum_r B1_i[n,r] s1[i][t][r]
 * in int64, so nothing can overflow at the shapes used here. */
void dbf_oracle_forward_int(int L, int64_t N, int64_t M, int64_t R, int64_t T,
                            const int8_t *const *b1, const int8_t *const *b2,
                            const int8_t *x, int64_t *s1, int64_t *s2)
{
    for (int i = 0; i < L; ++i) {
        for (int64_t t = 0; t < T; ++t) {
            const int8_t *xt = x + t * M;
            int64_t *o1 = s1 + ((int64_t)i * T + t) * R;
            int64_t *o2 = s2 + ((int64_t)i * T + t) * N;
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < R; ++r) {
                const int8_t *row = b2[i] + r * M;
                int64_t s = 0;
                for (int64_t m = 0; m < M; ++m)
                    s += (row[m] > 0) ? (int64_t)xt[m] : -(int64_t)xt[m];
                o1[r] = s;
            }
#pragma omp parallel for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                const int8_t *row = b1[i] + n * R;
                int64_t s = 0;
                for (int64_t q = 0; q < R; ++q)
                    s += (row[q] > 0) ? o1[q] : -o1[q];
                o2[n] = s;
            }
        }
    }
}

/*
 * Bit layout of a sign matrix S in {+-1}^{rows x K} (the storage format of
 * B1, with rows = N, K = R, and of B2, with rows = R, K = M; one bit per
 * sign as the LoRDBA and DBF pages store it).
 *
 *   bit value 1 means +1, 0 means -1 and every padding bit is 0;
 *   kw   = min(4, ceil(K / 32)) words per row per tile;
 *   a tile is 64 rows x kw words, stored row by row (kw words per row);
 *   tiles go row-tile first, then K-block:  tile (rt, kb) is number
 *   rt * nkb + kb with nkb = ceil(K / (32 kw));
 *   bit j of word w of row r in tile (rt, kb) is sign (64 rt + r,
 *   32 kw kb + 32 w + j).
 *
 * The packer below sets bit (value >= 0): 0 and -0.0 map to +1, NaN to -1.
 */
static int64_t kw_of(int64_t K)
{
    int64_t w = (K + 31) / 32;
    return w < 4 ? (w < 1 ? 1 : w) : 4;
}

int64_t dbf_oracle_packed_words(int64_t rows, int64_t K)
{
    int64_t kw = kw_of(K);
    int64_t nrt = (rows + 63) / 64;
    int64_t nkb = (K + 32 * kw - 1) / (32 * kw);
    return nrt * nkb * 64 * kw;
}

static int64_t word_index(int64_t r, int64_t k, int64_t K)
{
    int64_t kw = kw_of(K);
    int64_t nkb = (K + 32 * kw - 1) / (32 * kw);
    int64_t rt = r / 64, kb = k / (32 * kw);
    int64_t tile = rt * nkb + kb;
    int64_t w = (k % (32 * kw)) / 32;
    return tile * 64 * kw + (r % 64) * kw + w;
}

void dbf_oracle_pack(const double *v, int64_t rows, int64_t K, uint32_t *out)
{
    int64_t r, k;
    memset(out, 0, sizeof(uint32_t) * (size_t)dbf_oracle_packed_words(rows, K));
    for (r = 0; r < rows; ++r)
        for (k = 0; k < K; ++k)
            if (v[r * K + k] >= 0.0)
                out[word_index(r, k, K)] |= (uint32_t)1u << (k % 32);
}

void dbf_oracle_unpack(const uint32_t *p, int64_t rows, int64_t K, int8_t *s)
{
    int64_t r, k;
    for (r = 0; r < rows; ++r)
        for (k = 0; k < K; ++k)
            s[r * K + k] = ((p[word_index(r, k, K)] >> (k % 32)) & 1u) ? 1 : -1;
}
