/*
 * sanitize_check.c -- drives every function of the fp64 oracle (tria_oracle.c) on small seeded
 * inputs, for a build with the address and undefined-behaviour sanitizers.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by tests/test_oracle_sanitized.py).  It exercises the
 * three score forms (literal, factored, offset maximum), pre- and post-RoPE keys, the R-weighted
 * form, bf16 and fp32 keys, ragged stream lengths, budgets below and at or above N, ties and signed
 * zeros in the selection, a constant head, a non-finite score, the compaction and the calibration
 * statistics, and checks a few invariants of the results.  Exit status 0 when everything ran and
 * every invariant held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_omega(double theta, int f, int d);
void oracle_score_stream(int N, int d, int G, int dtype, const void *keys, const int32_t *pos, int64_t t,
                         const float *qc, const float *qn, const float *rb, double theta, const int64_t *off,
                         int n_off, int form, int pre_rope, int weight_r, double *s_trig, double *s_norm,
                         double *raw);
int oracle_zmax(int N, int G, const double *raw, double *z, double *F, double *mu, double *sd);
int oracle_select(int N, int B, const double *F, int32_t *kept);
void oracle_compact_rows(int nk, size_t row_bytes, unsigned char *rows, const int32_t *kept);
int oracle_prune_streams(int form, int pre_rope, int weight_r, int dtype, int S, int L, int Hkv, int G, int N, int d,
                         const void *keys, const int32_t *pos, const int64_t *t, const float *qc, const float *qn,
                         const float *rb, double theta, const int64_t *off, int n_off, int B, const int64_t *idx,
                         int n_idx, double *F_out, double *raw_out, int32_t *kept_out, int n_threads);
void oracle_calib_stats(int n_heads, int n_cal, int d, int dtype, const void *q, double *qc_out, double *qn_out,
                        double *r_out);
int oracle_max_threads(int n_threads);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void)   /* uniform in [0, 1), xorshift64* */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) * 0x1p-53;
}
static uint16_t bf16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static int failures = 0;
#define CHECK(c, msg)                                           \
    do {                                                        \
        if (!(c)) {                                             \
            fprintf(stderr, "check failed: %s (%s)\n", msg, #c); \
            ++failures;                                         \
        }                                                       \
    } while (0)

static void check_kept(const int32_t *kept, int nk, int N)
{
    for (int i = 0; i < nk; ++i) {
        CHECK(kept[i] >= 0 && kept[i] < N, "kept index in range");
        if (i) CHECK(kept[i] > kept[i - 1], "kept ascending");
    }
}

int main(void)
{
    enum { d = 128, half = 64, S = 2, L = 2, Hkv = 2, G = 3, N = 37, n_off = 17 };
    const int Hq = Hkv * G, streams = S * L * Hkv;
    const double theta = 1e6;
    int64_t off[n_off];
    for (int i = 0; i < n_off; ++i) off[i] = (int64_t)1 << i;
    for (int f = 0; f < half; ++f) CHECK(oracle_omega(theta, f, d) > 0.0, "omega positive");

    float *qc = malloc(sizeof(float) * L * Hq * d), *qn = malloc(sizeof(float) * L * Hq * half),
          *rb = malloc(sizeof(float) * L * Hq * half);
    for (int i = 0; i < L * Hq * d; ++i) qc[i] = (float)(2.0 * urand() - 1.0);
    for (int i = 0; i < L * Hq * half; ++i) {
        rb[i] = (float)(0.6 + 0.39 * urand());
        qn[i] = (float)(0.5 + urand());
    }
    float *k32 = malloc(sizeof(float) * streams * N * d);
    uint16_t *k16 = malloc(sizeof(uint16_t) * streams * N * d);
    for (int i = 0; i < streams * N * d; ++i) {
        k32[i] = (float)(4.0 * urand() - 2.0);
        k16[i] = bf16_bits(k32[i]);
    }
    int32_t *pos = malloc(sizeof(int32_t) * streams * N);
    for (int s = 0; s < streams; ++s)
        for (int j = 0; j < N; ++j) pos[s * N + j] = 3 * j + (int32_t)(2.0 * urand());
    int64_t t[S] = {200, 4000};
    int64_t idx[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    double *F = malloc(sizeof(double) * streams * N), *raw = malloc(sizeof(double) * streams * G * N);
    int32_t *kept = malloc(sizeof(int32_t) * streams * N);

    /* the prune over every stream, in every form, both dtypes, budgets below and at or above N */
    const int budgets[3] = {10, N, N + 13};
    for (int form = 0; form < 3; ++form)
        for (int pre = 0; pre < 2; ++pre)
            for (int wr = 0; wr < 2; ++wr)
                for (int dt = 0; dt < 2; ++dt)
                    for (int b = 0; b < 3; ++b) {
                        const int B = budgets[b], nk = B < N ? B : N;
                        const int rc = oracle_prune_streams(form, pre, wr, dt, S, L, Hkv, G, N, d,
                                                            dt == 0 ? (const void *)k16 : (const void *)k32, pos, t,
                                                            qc, qn, rb, theta, off, n_off, B, idx, streams, F, raw,
                                                            kept, 2);
                        CHECK(rc == 0, "prune returns 0 on finite input");
                        for (int s = 0; s < streams; ++s) check_kept(kept + (size_t)s * nk, nk, N);
                    }
    /* without the optional outputs (the oracle then allocates its own scratch) */
    CHECK(oracle_prune_streams(1, 0, 0, 0, S, L, Hkv, G, N, d, k16, pos, t, qc, qn, rb, theta, off, n_off, 10, idx,
                               streams, NULL, NULL, NULL, 1) == 0,
          "prune with no outputs");

    /* one stream scored on its own, every output */
    double *st = malloc(sizeof(double) * G * N), *sn = malloc(sizeof(double) * G * N);
    oracle_score_stream(N, d, G, 1, k32, pos, 500, qc, qn, rb, theta, off, n_off, 0, 0, 0, st, sn, raw);
    for (int i = 0; i < G * N; ++i) CHECK(fabs(raw[i] - (st[i] + sn[i])) <= 1e-9 * (1.0 + fabs(raw[i])), "s = trig + norm");

    /* z-score: a constant head gives z = 0; a non-finite score is reported */
    double *z = malloc(sizeof(double) * G * N), mu[G], sd[G];
    for (int j = 0; j < N; ++j) raw[j] = 1.5;
    CHECK(oracle_zmax(N, G, raw, z, F, mu, sd) == 0, "zmax finite");
    CHECK(sd[0] == 0.0, "constant head has std 0");
    for (int j = 0; j < N; ++j) CHECK(z[j] == 0.0, "constant head has z 0");
    raw[N + 5] = NAN;
    CHECK(oracle_zmax(N, G, raw, z, F, mu, sd) < 0, "non-finite score reported");

    /* selection: ties and signed zeros, every budget */
    double Fs[N];
    for (int j = 0; j < N; ++j) Fs[j] = (j % 5 == 0) ? 0.25 : (j % 7 == 0 ? -0.0 : (j % 3 == 0 ? 0.0 : urand() - 0.5));
    for (int B = 1; B <= N + 2; ++B) {
        const int nk = B < N ? B : N;
        CHECK(oracle_select(N, B, Fs, kept) == nk, "select count");
        check_kept(kept, nk, N);
    }

    /* compaction of a stream's rows */
    unsigned char *rows = malloc((size_t)N * 256);
    for (int i = 0; i < N * 256; ++i) rows[i] = (unsigned char)(i * 7);
    CHECK(oracle_select(N, 11, Fs, kept) == 11, "select for compaction");
    unsigned char *copy = malloc((size_t)N * 256);
    memcpy(copy, rows, (size_t)N * 256);
    oracle_compact_rows(11, 256, rows, kept);
    for (int i = 0; i < 11; ++i) CHECK(memcmp(rows + (size_t)i * 256, copy + (size_t)kept[i] * 256, 256) == 0, "compacted row");

    /* calibration statistics, both dtypes, a band that is zero in every query */
    enum { n_heads = 3, n_cal = 5 };
    float *q32 = malloc(sizeof(float) * n_heads * n_cal * d);
    uint16_t *q16 = malloc(sizeof(uint16_t) * n_heads * n_cal * d);
    for (int i = 0; i < n_heads * n_cal * d; ++i) {
        const int dim = i % d;
        q32[i] = (dim == 3 || dim == 3 + half) ? 0.0f : (float)(2.0 * urand() - 1.0);
        q16[i] = bf16_bits(q32[i]);
    }
    double *cq = malloc(sizeof(double) * n_heads * d), *cn = malloc(sizeof(double) * n_heads * half),
           *cr = malloc(sizeof(double) * n_heads * half);
    for (int dt = 0; dt < 2; ++dt) {
        oracle_calib_stats(n_heads, n_cal, d, dt, dt == 0 ? (const void *)q16 : (const void *)q32, cq, cn, cr);
        for (int i = 0; i < n_heads * half; ++i) CHECK(cr[i] >= 0.0 && cr[i] <= 1.0 + 1e-12, "0 <= R <= 1");
        CHECK(cr[3] == 0.0, "a band zero in every query has R = 0");
    }
    CHECK(oracle_max_threads(2) >= 1, "threads");

    free(qc); free(qn); free(rb); free(k32); free(k16); free(pos); free(F); free(raw); free(kept);
    free(st); free(sn); free(z); free(rows); free(copy); free(q32); free(q16); free(cq); free(cn); free(cr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}
