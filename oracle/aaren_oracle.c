/*
 * Oracle for single-query softmax attention: plain, slow, float64, CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header or constant with the GPU library and the GPU library never calls it.
 *
 * What it computes.
 *  - Attention of one query q over keys k_1..k_n and values v_1..v_n is the
 *    weighted sum of the values whose weights are the softmax of the scores
 *    s_i = scale * <q, k_i>  ("Self-attention Does Not Need O(n^2) Memory"
 *    review, section 1 Introduction; the scale is the caller's, 1/sqrt(d) in
 *    every workload, 1 reproduces the page literally).
 *  - It is evaluated with the page's constant-memory recurrence (same review,
 *    section 2 Algorithm): a vector accumulator and a scalar accumulator, both
 *    zero at the start; each key/value pair, taken in order, adds v_i e^{s_i}
 *    to the vector and e^{s_i} to the scalar; the division by the scalar is
 *    moved to the very end by the distributive law.
 *  - The page's numerical-stability section (section 3) lost its body. It is
 *    read here as the running-maximum shift: both accumulators are held
 *    relative to e^{m}, m the largest score seen so far, and are multiplied by
 *    e^{m_old - m_new} when m grows. Every term is scaled by the same factor,
 *    so the quotient is the page's quotient.
 *  - "Attention as an RNN" (review, abstract item (3) and proposed method)
 *    asks for the many-to-many output: the attention over every prefix
 *    1..k, k = 1..n. The recurrence above yields it by emitting
 *    (vector / scalar) after each pair.
 *  - Packed variable-length batches restart the recurrence at each sequence
 *    start; the per-token RNN update absorbs exactly one pair into a stored
 *    (m, u, w) state; the many-to-one reduction keeps only the last output.
 *  - Gradients. "Attention as an RNN" (review, proposed method) presents the
 *    many-to-many form as differentiable and trained in parallel, and the
 *    memory-efficient-attention review reports differentiation (abstract;
 *    section 5.2, body lost) without a formula. The gradient used here is
 *    derived from the definition: with p_ki = e^{s_i - L_k} the weight of
 *    pair i in output k (L_k = ln sum_{j<=k} e^{s_j}) and g_k = dloss/do_k,
 *      dv_i = sum_{k>=i} p_ki g_k,
 *      ds_i = sum_{k>=i} p_ki <g_k, v_i - o_k> = <dv_i, v_i> - sum_{k>=i} p_ki <g_k, o_k>,
 *      dk_i = scale ds_i q,  dq = scale sum_i ds_i k_i.
 *    Both suffix sums are evaluated backwards from the last pair, each term
 *    weighted by e^{L_i - L_k} <= 1 relative to the current position (L is
 *    non-decreasing along the sequence), then multiplied by p_ii = e^{s_i - L_i}.
 *
 *  - Self-attention. The memory-efficient-attention review (section 2)
 *    extends the single-query algorithm to self-attention by computing the
 *    result of every query in turn, one query per token. Row i here is the
 *    single-query recurrence for query q_i over pairs 1..i (causal) or over
 *    all n pairs, so it is the same definition applied n times.
 *
 * Notation: m = running maximum score, u = scalar accumulator (sum of
 * e^{s_i - m}), w = vector accumulator (sum of e^{s_i - m} v_i). Inputs arrive
 * as float32 (bfloat16 inputs are widened exactly by the caller) and are
 * widened to double here; all arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* s = scale * <q, k> in double. */
static double score(const float *q, const float *k, int64_t d, double scale)
{
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j)
        acc += (double)q[j] * (double)k[j];
    return scale * acc;
}

/* Absorb one pair (s, v) into the state (m, u, w): the page's update
 * "w += v e^s, u += e^s", written relative to the running maximum m. */
static void absorb(double *m, double *u, double *w, int64_t d, double s, const float *v)
{
    if (s > *m) {
        /* new maximum: what was accumulated shrinks by e^{m_old - s};
         * an empty state (m = -inf) holds nothing to shrink */
        double shrink = (*m == -INFINITY) ? 0.0 : exp(*m - s);
        *u = *u * shrink + 1.0;
        for (int64_t j = 0; j < d; ++j)
            w[j] = w[j] * shrink + (double)v[j];
        *m = s;
    } else {
        double p = exp(s - *m);
        *u += p;
        for (int64_t j = 0; j < d; ++j)
            w[j] += p * (double)v[j];
    }
}

/* Emit o = w / u and, when asked, m and the log-normaliser L = m + ln u. */
static void emit(double m, double u, const double *w, int64_t d,
                 double *o, double *m_out, double *lse_out)
{
    for (int64_t j = 0; j < d; ++j)
        o[j] = w[j] / u;
    if (m_out)
        *m_out = m;
    if (lse_out)
        *lse_out = m + log(u);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of threads the loops over independent units use (timing
   only: every unit is computed the same way whatever the count). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Many-to-many scan over a dense batch.
 * q [H,d]; k, v [B,H,N,d]; o [B,H,N,d]; m_out, lse_out [B,H,N] or NULL. */
int oracle_scan(const float *q, const float *k, const float *v,
                int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                double *o, double *m_out, double *lse_out)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return 1;
    int64_t units = B * H;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < units; ++unit) {
            const float *qh = q + (unit % H) * d;
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t i = 0; i < N; ++i) {
                int64_t row = unit * N + i;
                absorb(&m, &u, w, d, score(qh, k + row * d, d, scale), v + row * d);
                emit(m, u, w, d, o + row * d, m_out ? m_out + row : NULL,
                     lse_out ? lse_out + row : NULL);
            }
        }
        free(w);
    }
    return 0;
}

/* The same many-to-many scan for inputs that are not float32 values (keys
 * and values computed in double, e.g. a projection of the inputs): q [H,d],
 * k, v [B,H,N,d] and o in double. Each pair is absorbed as above: the state
 * is rescaled by e^{m_old - s} when the score s is a new maximum, otherwise
 * the pair enters with weight e^{s - m}; o is w / u after every pair. */
int oracle_scan_f64(const double *q, const double *k, const double *v,
                    int64_t B, int64_t H, int64_t N, int64_t d, double scale, double *o)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return 1;
    int64_t units = B * H;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < units; ++unit) {
            const double *qh = q + (unit % H) * d;
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t i = 0; i < N; ++i) {
                const double *kr = k + (unit * N + i) * d, *vr = v + (unit * N + i) * d;
                double dot = 0.0;
                for (int64_t j = 0; j < d; ++j)
                    dot += qh[j] * kr[j];
                const double sc = scale * dot;
                if (sc > m) {
                    const double shrink = (m == -INFINITY) ? 0.0 : exp(m - sc);
                    u = u * shrink + 1.0;
                    for (int64_t j = 0; j < d; ++j)
                        w[j] = w[j] * shrink + vr[j];
                    m = sc;
                } else {
                    const double p = exp(sc - m);
                    u += p;
                    for (int64_t j = 0; j < d; ++j)
                        w[j] += p * vr[j];
                }
                for (int64_t j = 0; j < d; ++j)
                    o[(unit * N + i) * d + j] = w[j] / u;
            }
        }
        free(w);
    }
    return 0;
}

/* Many-to-many scan over a packed variable-length batch: each sequence is
 * scanned on its own. q [H,d]; k, v, o [T,H,d] token-major; offsets [S+1]
 * with offsets[0] = 0, non-decreasing, offsets[S] = T. */
int oracle_scan_segmented(const float *q, const float *k, const float *v,
                          const int64_t *offsets, int64_t S, int64_t T,
                          int64_t H, int64_t d, double scale,
                          double *o, double *m_out, double *lse_out)
{
    if (S < 0 || T < 0 || H < 0 || d < 1 || offsets[0] != 0 || offsets[S] != T)
        return 1;
    for (int64_t s = 0; s < S; ++s)
        if (offsets[s + 1] < offsets[s])
            return 1;
    int64_t units = S * H;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t unit = 0; unit < units; ++unit) {
            int64_t seq = unit / H, h = unit % H;
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t t = offsets[seq]; t < offsets[seq + 1]; ++t) {
                int64_t row = t * H + h;
                absorb(&m, &u, w, d, score(q + h * d, k + row * d, d, scale), v + row * d);
                emit(m, u, w, d, o + row * d, m_out ? m_out + row : NULL,
                     lse_out ? lse_out + row : NULL);
            }
        }
        free(w);
    }
    return 0;
}

/* One RNN update per (stream, head): absorb the pair (k_t, v_t) into the
 * stored state and emit o_t. q [H,d]; k_t, v_t [S,H,d]; state m, u [S,H],
 * w [S,H,d] (in/out, a fresh state is m = -inf, u = 0, w = 0); o_t [S,H,d]
 * or NULL. */
int oracle_step(const float *q, const float *k_t, const float *v_t,
                double *m, double *u, double *w, double *o_t,
                int64_t S, int64_t H, int64_t d, double scale)
{
    if (S < 0 || H < 0 || d < 1)
        return 1;
    int64_t units = S * H;
#pragma omp parallel for schedule(static)
    for (int64_t unit = 0; unit < units; ++unit) {
        const float *qh = q + (unit % H) * d;
        absorb(&m[unit], &u[unit], w + unit * d, d,
               score(qh, k_t + unit * d, d, scale), v_t + unit * d);
        if (o_t)
            emit(m[unit], u[unit], w + unit * d, d, o_t + unit * d, NULL, NULL);
    }
    return 0;
}

/* Many-to-one: the attention of q_h over all N pairs of each (b,h).
 * q [H,d]; k, v [B,H,N,d]; o [B,H,d]; m_out, lse_out [B,H] or NULL. */
int oracle_reduce(const float *q, const float *k, const float *v,
                  int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                  double *o, double *m_out, double *lse_out)
{
    if (B < 0 || H < 0 || N < 1 || d < 1)
        return 1;
    int64_t units = B * H;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < units; ++unit) {
            const float *qh = q + (unit % H) * d;
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t i = 0; i < N; ++i) {
                int64_t row = unit * N + i;
                absorb(&m, &u, w, d, score(qh, k + row * d, d, scale), v + row * d);
            }
            emit(m, u, w, d, o + unit * d, m_out ? m_out + unit : NULL,
                 lse_out ? lse_out + unit : NULL);
        }
        free(w);
    }
    return 0;
}

/* Gradients of the many-to-many output for a dense batch, given the output
 * gradient dout [B,H,N,d]: dq [H,d] (summed over the batch), dk, dv [B,H,N,d].
 * The forward values o_k and L_k are recomputed here, in double. */
int oracle_scan_backward(const float *q, const float *k, const float *v, const float *dout,
                         int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                         double *dq, double *dk, double *dv)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return 1;
    int64_t units = B * H;
    double *dq_unit = (double *)calloc((size_t)(units > 0 ? units : 1) * (size_t)d, sizeof(double));
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
        double *o = (double *)malloc((size_t)(N > 0 ? N : 1) * (size_t)d * sizeof(double));
        double *L = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *s = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double *G = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < units; ++unit) {
            const float *qh = q + (unit % H) * d;
            /* forward: o_k and L_k */
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t i = 0; i < N; ++i) {
                int64_t row = unit * N + i;
                s[i] = score(qh, k + row * d, d, scale);
                absorb(&m, &u, w, d, s[i], v + row * d);
                emit(m, u, w, d, o + i * d, NULL, &L[i]);
            }
            /* backward: suffix sums G (vector) and D (scalar) relative to e^{-L_i} */
            double D = 0.0;
            memset(G, 0, (size_t)d * sizeof(double));
            for (int64_t i = N - 1; i >= 0; --i) {
                int64_t row = unit * N + i;
                const float *g = dout + row * d;
                double shrink = (i == N - 1) ? 0.0 : exp(L[i] - L[i + 1]);
                double delta = 0.0;
                for (int64_t j = 0; j < d; ++j)
                    delta += (double)g[j] * o[i * d + j];
                D = delta + shrink * D;
                for (int64_t j = 0; j < d; ++j)
                    G[j] = (double)g[j] + shrink * G[j];
                double pii = exp(s[i] - L[i]);
                double ds = 0.0;
                for (int64_t j = 0; j < d; ++j) {
                    dv[row * d + j] = pii * G[j];
                    ds += dv[row * d + j] * (double)v[row * d + j];
                }
                ds -= pii * D;
                for (int64_t j = 0; j < d; ++j) {
                    dk[row * d + j] = scale * ds * (double)qh[j];
                    dq_unit[unit * d + j] += scale * ds * (double)k[row * d + j];
                }
            }
        }
        free(w);
        free(o);
        free(L);
        free(s);
        free(G);
    }
    for (int64_t h = 0; h < H; ++h)
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                acc += dq_unit[(b * H + h) * d + j];
            dq[h * d + j] = acc;
        }
    free(dq_unit);
    return 0;
}

/* Self-attention, one query per token: q, k, v [B,H,N,d]; rows
 * row_begin..row_end-1 of every (b,h) are computed, each as the single-query
 * recurrence of its own query over pairs 0..i (causal != 0) or 0..N-1.
 * o [B,H,row_end-row_begin,d]; lse_out [B,H,row_end-row_begin] or NULL. */
int oracle_self_attention(const float *q, const float *k, const float *v,
                          int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                          int causal, int64_t row_begin, int64_t row_end,
                          double *o, double *lse_out)
{
    if (B < 0 || H < 0 || N < 0 || d < 1 || row_begin < 0 || row_end > N ||
        row_end < row_begin)
        return 1;
    const int64_t rows = row_end - row_begin, units = B * H;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t job = 0; job < units * rows; ++job) {
            const int64_t unit = job / rows, i = row_begin + job % rows;
            const float *qi = q + (unit * N + i) * d;
            const int64_t last = causal ? i : N - 1;
            double m = -INFINITY, u = 0.0;
            memset(w, 0, (size_t)d * sizeof(double));
            for (int64_t j = 0; j <= last; ++j) {
                const int64_t row = unit * N + j;
                absorb(&m, &u, w, d, score(qi, k + row * d, d, scale), v + row * d);
            }
            const int64_t out = unit * rows + (i - row_begin);
            emit(m, u, w, d, o + out * d, NULL, lse_out ? lse_out + out : NULL);
        }
        free(w);
    }
    return 0;
}
