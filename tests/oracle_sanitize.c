/* Drives every entry point of the C oracle on small and degenerate shapes,
 * for a build with -fsanitize=address,undefined: every buffer is malloc'ed at
 * its exact size, so a read or write one element out of bounds is reported.
 * A few value checks ride along (a single pair gives its value, the
 * reduction is the scan's last row, steps reproduce the scan). Exit status 0
 * means every call returned 0 and every check held. Test infrastructure: it
 * links the oracle's source and nothing else. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_scan(const float *q, const float *k, const float *v, int64_t B, int64_t H, int64_t N,
                int64_t d, double scale, double *o, double *m_out, double *lse_out);
int oracle_scan_segmented(const float *q, const float *k, const float *v, const int64_t *offsets,
                          int64_t S, int64_t T, int64_t H, int64_t d, double scale, double *o,
                          double *m_out, double *lse_out);
int oracle_step(const float *q, const float *k_t, const float *v_t, double *m, double *u,
                double *w, double *o_t, int64_t S, int64_t H, int64_t d, double scale);
int oracle_reduce(const float *q, const float *k, const float *v, int64_t B, int64_t H, int64_t N,
                  int64_t d, double scale, double *o, double *m_out, double *lse_out);
int oracle_scan_backward(const float *q, const float *k, const float *v, const float *dout,
                         int64_t B, int64_t H, int64_t N, int64_t d, double scale, double *dq,
                         double *dk, double *dv);
int oracle_self_attention(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                          int64_t N, int64_t d, double scale, int causal, int64_t row_begin,
                          int64_t row_end, double *o, double *lse_out);

static int failures = 0;
#define CHECK(cond, ...)                                       \
    do {                                                       \
        if (!(cond)) {                                         \
            fprintf(stderr, "check failed: " __VA_ARGS__);     \
            fprintf(stderr, "\n");                             \
            ++failures;                                        \
        }                                                      \
    } while (0)

static uint32_t rng_state = 12345u;
static float rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)((rng_state >> 8) / 16777216.0 * 2.0 - 1.0);
}
static float *fbuf(int64_t n)
{
    float *p = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}
static double *dbuf(int64_t n)
{
    return (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
}

static void scan_and_reduce(int64_t B, int64_t H, int64_t N, int64_t d)
{
    float *q = fbuf(H * d), *k = fbuf(B * H * N * d), *v = fbuf(B * H * N * d);
    double *o = dbuf(B * H * N * d), *m = dbuf(B * H * N), *l = dbuf(B * H * N);
    CHECK(oracle_scan(q, k, v, B, H, N, d, 0.5, o, m, l) == 0, "scan %lld %lld %lld %lld",
          (long long)B, (long long)H, (long long)N, (long long)d);
    if (N > 0) {
        double *r = dbuf(B * H * d), *rm = dbuf(B * H), *rl = dbuf(B * H);
        CHECK(oracle_reduce(q, k, v, B, H, N, d, 0.5, r, rm, rl) == 0, "reduce");
        for (int64_t u = 0; u < B * H; ++u)
            for (int64_t j = 0; j < d; ++j) {
                const double a = r[u * d + j], b = o[(u * N + N - 1) * d + j];
                CHECK(fabs(a - b) <= 1e-12 * (1 + fabs(b)), "reduce = last scan row");
            }
        /* the first row is its own value */
        for (int64_t u = 0; u < B * H; ++u)
            for (int64_t j = 0; j < d; ++j)
                CHECK(o[u * N * d + j] == (double)v[u * N * d + j], "first row = v");
        free(r);
        free(rm);
        free(rl);
    }
    /* gradients of the same shape */
    float *g = fbuf(B * H * N * d);
    double *dq = dbuf(H * d), *dk = dbuf(B * H * N * d), *dv = dbuf(B * H * N * d);
    CHECK(oracle_scan_backward(q, k, v, g, B, H, N, d, 0.5, dq, dk, dv) == 0, "backward");
    free(g);
    free(dq);
    free(dk);
    free(dv);
    free(q);
    free(k);
    free(v);
    free(o);
    free(m);
    free(l);
}

static void steps_against_scan(int64_t S, int64_t H, int64_t T, int64_t d)
{
    /* stream s, head h, token t: k laid out [T][S][H][d] */
    float *q = fbuf(H * d), *k = fbuf(T * S * H * d), *v = fbuf(T * S * H * d);
    double *m = dbuf(S * H), *u = dbuf(S * H), *w = dbuf(S * H * d), *o = dbuf(S * H * d);
    for (int64_t i = 0; i < S * H; ++i)
        m[i] = -INFINITY;
    float *ks = fbuf(S * H * T * d), *vs = fbuf(S * H * T * d); /* [S][H][T][d] for the scan */
    for (int64_t t = 0; t < T; ++t)
        for (int64_t sh = 0; sh < S * H; ++sh)
            for (int64_t j = 0; j < d; ++j) {
                ks[(sh * T + t) * d + j] = k[(t * S * H + sh) * d + j];
                vs[(sh * T + t) * d + j] = v[(t * S * H + sh) * d + j];
            }
    double *ref = dbuf(S * H * T * d);
    CHECK(oracle_scan(q, ks, vs, S, H, T, d, 0.25, ref, NULL, NULL) == 0, "scan for steps");
    for (int64_t t = 0; t < T; ++t) {
        CHECK(oracle_step(q, k + t * S * H * d, v + t * S * H * d, m, u, w, o, S, H, d, 0.25) == 0,
              "step");
        for (int64_t sh = 0; sh < S * H; ++sh)
            for (int64_t j = 0; j < d; ++j) {
                const double a = o[sh * d + j], b = ref[(sh * T + t) * d + j];
                CHECK(fabs(a - b) <= 1e-12 * (1 + fabs(b)), "step %lld = scan row", (long long)t);
            }
    }
    free(q);
    free(k);
    free(v);
    free(m);
    free(u);
    free(w);
    free(o);
    free(ks);
    free(vs);
    free(ref);
}

static void segmented(const int64_t *lengths, int64_t S, int64_t H, int64_t d)
{
    int64_t *off = (int64_t *)malloc((size_t)(S + 1) * sizeof(int64_t));
    off[0] = 0;
    for (int64_t s = 0; s < S; ++s)
        off[s + 1] = off[s] + lengths[s];
    const int64_t T = off[S];
    float *q = fbuf(H * d), *k = fbuf(T * H * d), *v = fbuf(T * H * d);
    double *o = dbuf(T * H * d), *m = dbuf(T * H), *l = dbuf(T * H);
    CHECK(oracle_scan_segmented(q, k, v, off, S, T, H, d, 0.5, o, m, l) == 0, "segmented");
    for (int64_t s = 0; s < S; ++s)
        if (lengths[s] > 0)
            for (int64_t j = 0; j < H * d; ++j)
                CHECK(o[off[s] * H * d + j] == (double)v[off[s] * H * d + j], "segment start = v");
    free(off);
    free(q);
    free(k);
    free(v);
    free(o);
    free(m);
    free(l);
}

static void self_attention(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int64_t a,
                           int64_t b)
{
    float *q = fbuf(B * H * N * d), *k = fbuf(B * H * N * d), *v = fbuf(B * H * N * d);
    double *o = dbuf(B * H * (b - a) * d), *l = dbuf(B * H * (b - a));
    CHECK(oracle_self_attention(q, k, v, B, H, N, d, 0.5, causal, a, b, o, l) == 0,
          "self-attention");
    free(q);
    free(k);
    free(v);
    free(o);
    free(l);
}

int main(void)
{
    const int64_t shapes[][4] = {{1, 1, 1, 1}, {1, 1, 2, 3}, {2, 3, 17, 8}, {1, 2, 65, 64},
                                 {1, 1, 1, 128}, {2, 1, 0, 4}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        scan_and_reduce(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3]);
    steps_against_scan(3, 2, 9, 5);
    steps_against_scan(1, 1, 1, 64);
    const int64_t l1[] = {1, 0, 5, 0, 0, 3};
    segmented(l1, 6, 2, 4);
    const int64_t l2[] = {40};
    segmented(l2, 1, 3, 64);
    const int64_t l3[] = {0};
    segmented(l3, 1, 1, 8);
    self_attention(1, 1, 1, 1, 1, 0, 1);
    self_attention(2, 2, 33, 16, 1, 0, 33);
    self_attention(1, 2, 33, 16, 0, 5, 30);
    self_attention(1, 1, 10, 8, 1, 4, 4);
    /* argument rejection paths */
    double dummy[4];
    float f[4] = {0, 0, 0, 0};
    CHECK(oracle_reduce(f, f, f, 1, 1, 0, 4, 1.0, dummy, NULL, NULL) != 0, "reduce N=0 rejected");
    CHECK(oracle_scan(f, f, f, -1, 1, 1, 4, 1.0, dummy, NULL, NULL) != 0, "negative B rejected");
    CHECK(oracle_self_attention(f, f, f, 1, 1, 2, 1, 1.0, 1, 1, 3, dummy, NULL) != 0,
          "rows past N rejected");
    if (failures)
        fprintf(stderr, "%d check(s) failed\n", failures);
    else
        printf("oracle under sanitizers: all calls and checks passed\n");
    return failures ? 1 : 0;
}
