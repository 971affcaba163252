/*
 * tria_oracle.c -- plain, slow, fp64 CPU oracle for the TriAttention KV-cache prune step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it computes, per stream (one sequence, one layer, one KV head) of N cached keys and the
 * G query heads that share that KV head.  Sources are the pages about "TriAttention: Efficient
 * Long Reasoning with Trigonometric KV Compression" (arXiv 2604.04921):
 *
 *   [p1] "TriAttention深度解析：用三角函数革命性压缩KV Cache..." (chenxutan.com/d/2624)
 *   [p3] "旋转舞台上的追光者——TriAttention如何用三角函数破解长文本推理的内存困局" (zhichai.net)
 *   [p4] the 10100.com summary article (section "TriAttention方法")
 *   [p5] "TriAttention：面向长文本推理的高效KV缓存压缩..." (watermelonwater.tech),
 *        section "TriAttention 方案设计"
 *
 *  - RoPE in the half-split layout: band f (0 <= f < d/2) is the complex number
 *    v[f] + i*v[f+d/2]; RoPE at position p multiplies band f by exp(i*w_f*p)
 *    ([p3] section "技术细节补充 / RoPE回顾"; [p1] section 1.3).
 *    w_f = fl32(theta^(-2f/d)): the fp64 power rounded once to fp32, then used exactly.
 *  - Cached keys are post-RoPE.  The pre-RoPE key band is recovered as
 *    k_f = ktilde_f * exp(-i*w_f*p_j).  A cache that stores keys before RoPE (the layout the
 *    library serves with a flag) gives k_f directly; the score is the same function of k_f.
 *  - Trigonometric score ([p3] section "TriAttention：把理论变成算法" item 1, [p1] section 3.1):
 *      S_trig(j) = mean over d in D of sum_f |qbar_f| |k_f| cos(w_f*(t+d-p_j) + arg qbar_f - arg k_f)
 *    with the future-offset set D = {1, 2, 4, ..., 2^16} ([p1] section 3.3).  The offsets are
 *    combined by the mean (the expected attention of future queries, [p4] "TriAttention方法").
 *  - Norm score ([p3] same section, item 2): S_norm(j) = sum_f (1 - R_f) * E|q_f| * |k_f|,
 *    the (1-R) weight of [p4] "TriAttention方法" applied per band.
 *  - Raw score: s = S_trig + S_norm, the two parts simply added ([p4] "TriAttention方法").
 *  - Per query head: z = (s - mean)/std over the N keys of the stream (population std); the
 *    final key score is the max of z over the G query heads of the GQA group
 *    ([p4] "TriAttention方法" last paragraph; [p5] "TriAttention 方案设计" item 4).
 *    The pages do not say what a head whose scores are all equal contributes; such a head
 *    carries no ranking information, so its z is 0.  Scores that are mathematically equal
 *    differ by rounding, so a head whose scores span at most 2^-16 of their largest magnitude
 *    counts as constant (std reported as 0, z := 0).
 *  - Keep the top B keys by (final score descending, index ascending), output ascending
 *    ([p1] section 4.2, prune_kv_cache: topk then sort to keep the order).
 *  - Compaction: row i of K, V and positions takes row kept[i], i < min(B, N).
 *
 * Two forms of the trigonometric score are provided:
 *   lit : the definition above, a |D| x d/2 cosine sum per key and head.
 *   fac : the same sum with the offset mean taken first:
 *           mean_d cos(A + w d) = C_f cos A - S_f sin A,  C_f = mean_d cos(w_f d), S_f = mean_d sin(w_f d)
 *         with A = w_f (t - p_j) + arg qbar_f - arg k_f.  Pinned against lit by the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_HALF 256

/* w_f: theta^(-2f/d) computed in fp64 and rounded once to fp32 (the value used everywhere). */
double oracle_omega(double theta, int f, int d)
{
    float w = (float)pow(theta, -2.0 * (double)f / (double)d);
    return (double)w;
}

/* Input element loader: dtype 0 = bf16 (uint16 bit patterns), 1 = fp32.  Both convert to
 * double exactly. */
static double load_elem(const void *base, int dtype, size_t idx)
{
    if (dtype == 0) {
        uint16_t b = ((const uint16_t *)base)[idx];
        uint32_t u = (uint32_t)b << 16;
        float x;
        memcpy(&x, &u, 4);
        return (double)x;
    } else {
        return (double)((const float *)base)[idx];
    }
}

/*
 * Score one stream.
 *   keys   : [N][d] post-RoPE keys (dtype 0 bf16 bits / 1 fp32)
 *   pos    : [N]    key positions
 *   t      : current position (the newest cached token)
 *   qc     : [G][d]    pre-RoPE query centres qbar (half-split layout)
 *   qn     : [G][d/2]  E|q_f|
 *   rb     : [G][d/2]  R_f
 *   off    : [n_off]   future offsets D
 *   form   : 0 = lit, 1 = fac, 2 = max: the largest of the per-offset series instead of their mean
 *            (chenxutan.com/d/2624 section 3.3: the final trigonometric score is the maximum over
 *            the offsets; evaluated literally, offset by offset)
 *   pre_rope: 0 = keys are post-RoPE (ktilde), 1 = keys are the pre-RoPE bands k_f themselves
 *   weight_r: 0 = s = S_trig + S_norm; 1 = the trigonometric term of band f is weighted by R_f,
 *             s = sum_f R_f * (band f of S_trig) + S_norm, the convex R / (1 - R) mix of zhichai.net
 *             section "TriAttention：把理论变成算法" item 3 taken per band
 * Outputs (each [G][N], any may be NULL): s_trig (R-weighted with weight_r), s_norm, raw = s_trig + s_norm.
 */
void oracle_score_stream(int N, int d, int G, int dtype, const void *keys, const int32_t *pos,
                         int64_t t, const float *qc, const float *qn, const float *rb,
                         double theta, const int64_t *off, int n_off, int form, int pre_rope, int weight_r,
                         double *s_trig, double *s_norm, double *raw)
{
    const int half = d / 2;
    double w[ORACLE_MAX_HALF], Cf[ORACLE_MAX_HALF], Sf[ORACLE_MAX_HALF];
    for (int f = 0; f < half; ++f) {
        w[f] = oracle_omega(theta, f, d);
        double c = 0.0, s = 0.0;
        for (int m = 0; m < n_off; ++m) {
            c += cos(w[f] * (double)off[m]);
            s += sin(w[f] * (double)off[m]);
        }
        Cf[f] = c / n_off;
        Sf[f] = s / n_off;
    }
    double *kmag = (double *)malloc(sizeof(double) * half);
    double *karg = (double *)malloc(sizeof(double) * half);
    for (int j = 0; j < N; ++j) {
        const double p = (double)pos[j];
        for (int f = 0; f < half; ++f) {
            double x = load_elem(keys, dtype, (size_t)j * d + f);
            double y = load_elem(keys, dtype, (size_t)j * d + f + half);
            double kr = x, ki = y;
            if (!pre_rope) {
                double a = w[f] * p;             /* exact: 24-bit w times |p| < 2^31 */
                double ca = cos(a), sa = sin(a);
                kr = x * ca + y * sa;            /* (x + i y) * exp(-i a) */
                ki = y * ca - x * sa;
            }
            kmag[f] = sqrt(kr * kr + ki * ki);
            karg[f] = atan2(ki, kr);
        }
        for (int h = 0; h < G; ++h) {
            const float *q = qc + (size_t)h * d;
            double trig = 0.0, nrm = 0.0;
            if (form == 0 || form == 2) {
                for (int m = 0; m < n_off; ++m) {
                    double acc = 0.0;
                    for (int f = 0; f < half; ++f) {
                        double qr = q[f], qi = q[f + half];
                        double qmag = sqrt(qr * qr + qi * qi);
                        double qarg = atan2(qi, qr);
                        double dist = (double)(t + off[m]) - p;
                        double wr = weight_r ? (double)rb[(size_t)h * half + f] : 1.0;
                        acc += wr * qmag * kmag[f] * cos(w[f] * dist + qarg - karg[f]);
                    }
                    if (form == 0)
                        trig += acc;
                    else
                        trig = (m == 0 || acc > trig) ? acc : trig;
                }
                if (form == 0) trig /= n_off;
            } else {
                for (int f = 0; f < half; ++f) {
                    double qr = q[f], qi = q[f + half];
                    double qmag = sqrt(qr * qr + qi * qi);
                    double qarg = atan2(qi, qr);
                    double A = w[f] * ((double)t - p) + qarg - karg[f];
                    double wr = weight_r ? (double)rb[(size_t)h * half + f] : 1.0;
                    trig += wr * qmag * kmag[f] * (Cf[f] * cos(A) - Sf[f] * sin(A));
                }
            }
            for (int f = 0; f < half; ++f)
                nrm += (1.0 - (double)rb[(size_t)h * half + f]) * (double)qn[(size_t)h * half + f] * kmag[f];
            if (s_trig) s_trig[(size_t)h * N + j] = trig;
            if (s_norm) s_norm[(size_t)h * N + j] = nrm;
            if (raw) raw[(size_t)h * N + j] = trig + nrm;
        }
    }
    free(kmag);
    free(karg);
}

/*
 * z-score per head and max over the G heads.
 *   raw [G][N] -> z [G][N] (may be NULL), F [N], mu [G], sd [G] (may be NULL).
 * Population mean and std over the N keys.  A head whose raw scores span at most 2^-16 of
 * their largest magnitude is constant: std 0 and z = 0.  Returns 0, or -1 if any raw score is
 * not finite.
 */
int oracle_zmax(int N, int G, const double *raw, double *z, double *F, double *mu, double *sd)
{
    for (int j = 0; j < N; ++j) F[j] = -INFINITY;
    for (int h = 0; h < G; ++h) {
        const double *s = raw + (size_t)h * N;
        double sum = 0.0, lo = INFINITY, hi = -INFINITY;
        for (int j = 0; j < N; ++j) {
            if (!isfinite(s[j])) return -1;
            sum += s[j];
            if (s[j] < lo) lo = s[j];
            if (s[j] > hi) hi = s[j];
        }
        double m = sum / N;
        double var = 0.0;
        for (int j = 0; j < N; ++j) var += (s[j] - m) * (s[j] - m);
        double big = fabs(lo) > fabs(hi) ? fabs(lo) : fabs(hi);
        int constant = (hi - lo) <= ldexp(big, -16);
        double sig = constant ? 0.0 : sqrt(var / N);
        if (mu) mu[h] = m;
        if (sd) sd[h] = sig;
        for (int j = 0; j < N; ++j) {
            double zz = (sig == 0.0) ? 0.0 : (s[j] - m) / sig;
            if (z) z[(size_t)h * N + j] = zz;
            if (zz > F[j]) F[j] = zz;
        }
    }
    return 0;
}

/* ---- top-B selection by full sort ------------------------------------------------------ */
typedef struct { double v; int32_t j; } oracle_kv;

static int cmp_desc_then_index(const void *a, const void *b)
{
    const oracle_kv *x = (const oracle_kv *)a, *y = (const oracle_kv *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;          /* -0 and +0 compare equal here */
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_int32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Keep min(B, N) keys with the largest F (ties to the lower index); kept[] ascending.
 * Returns the number kept, or -1 if a score is not finite. */
int oracle_select(int N, int B, const double *F, int32_t *kept)
{
    int nk = B < N ? B : N;
    oracle_kv *a = (oracle_kv *)malloc(sizeof(oracle_kv) * (size_t)(N > 0 ? N : 1));
    for (int j = 0; j < N; ++j) {
        if (!isfinite(F[j])) { free(a); return -1; }
        a[j].v = F[j];
        a[j].j = j;
    }
    qsort(a, (size_t)N, sizeof(oracle_kv), cmp_desc_then_index);
    for (int i = 0; i < nk; ++i) kept[i] = a[i].j;
    qsort(kept, (size_t)nk, sizeof(int32_t), cmp_int32);
    free(a);
    return nk;
}

/* Out-of-place reference compaction of one stream's rows: row i <- row kept[i]. */
void oracle_compact_rows(int nk, size_t row_bytes, unsigned char *rows, const int32_t *kept)
{
    unsigned char *tmp = (unsigned char *)malloc(row_bytes * (size_t)(nk > 0 ? nk : 1));
    for (int i = 0; i < nk; ++i) memcpy(tmp + (size_t)i * row_bytes, rows + (size_t)kept[i] * row_bytes, row_bytes);
    memcpy(rows, tmp, row_bytes * (size_t)nk);
    free(tmp);
}

/*
 * Whole prune step over a list of streams (OpenMP over streams).  Layouts:
 *   keys  [n_idx][N][d]   the listed streams' keys, packed (dtype 0 bf16 bits / 1 fp32)
 *   pos   [n_idx][N]
 *   t     [S]
 *   qc    [L][Hq][d], qn and rb [L][Hq][d/2]   (query head h uses KV head h / G)
 * idx[i] is the global id (s*L + l)*Hkv + g of the i-th listed stream; it selects t[s] and the
 * calibration rows of layer l, heads g*G .. g*G+G-1.  Outputs are written at row i:
 * F_out [n_idx][N] (may be NULL), raw_out [n_idx][G][N] (may be NULL),
 * kept_out [n_idx][min(B,N)] (may be NULL).
 * Returns 0, or -1 if a non-finite score was met.
 */
int oracle_prune_streams(int form, int pre_rope, int weight_r, int dtype, int S, int L, int Hkv, int G, int N, int d,
                         const void *keys, const int32_t *pos, const int64_t *t,
                         const float *qc, const float *qn, const float *rb, double theta,
                         const int64_t *off, int n_off, int B,
                         const int64_t *idx, int n_idx,
                         double *F_out, double *raw_out, int32_t *kept_out, int n_threads)
{
    (void)S;
    const int half = d / 2;
    const int Hq = Hkv * G;
    const int nk = B < N ? B : N;
    const size_t esz = dtype == 0 ? 2 : 4;
    int bad = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int i = 0; i < n_idx; ++i) {
        int64_t sid = idx[i];
        int64_t g = sid % Hkv;
        int64_t l = (sid / Hkv) % L;
        int64_t s = sid / ((int64_t)Hkv * L);
        const unsigned char *kb = (const unsigned char *)keys + (size_t)i * N * d * esz;
        const int32_t *pb = pos + (size_t)i * N;
        size_t h0 = (size_t)l * Hq + (size_t)g * G;
        double *raw = raw_out ? raw_out + (size_t)i * G * N : (double *)malloc(sizeof(double) * (size_t)G * N);
        double *F = F_out ? F_out + (size_t)i * N : (double *)malloc(sizeof(double) * (size_t)N);
        oracle_score_stream(N, d, G, dtype, kb, pb, t[s], qc + h0 * d, qn + h0 * half, rb + h0 * half,
                            theta, off, n_off, form, pre_rope, weight_r, NULL, NULL, raw);
        int rc = oracle_zmax(N, G, raw, NULL, F, NULL, NULL);
        if (rc == 0 && kept_out) rc = oracle_select(N, B, F, kept_out + (size_t)i * nk) < 0 ? -1 : 0;
        if (rc != 0) bad |= 1;
        if (!raw_out) free(raw);
        if (!F_out) free(F);
    }
    return bad ? -1 : 0;
}

/*
 * Calibration statistics of the captured pre-RoPE queries of every (layer, query head)
 * (chenxutan.com/d/2624 section 3.4: centre vector, mean norm and concentration per head;
 * zhichai.net section "破局之道": R as the ratio of the norm of the mean to the mean norm;
 * watermelonwater.tech "TriAttention 方案设计" item 1: the Q centre and the expected norm).
 * Per band f (the complex number q[f] + i q[f + d/2]):
 *   qbar_f = mean_n q_{n,f}             (written back in the half-split layout)
 *   E|q_f| = mean_n |q_{n,f}|
 *   R_f    = |qbar_f| / E|q_f|          (0 when E|q_f| = 0)
 *   q      : [n_heads][n_cal][d] (dtype 0 bf16 bits / 1 fp32), n_heads = L * Hq
 *   qc_out : [n_heads][d];  qn_out, r_out : [n_heads][d/2]   (fp64)
 */
void oracle_calib_stats(int n_heads, int n_cal, int d, int dtype, const void *q, double *qc_out,
                        double *qn_out, double *r_out)
{
    const int half = d / 2;
    for (int hh = 0; hh < n_heads; ++hh) {
        for (int f = 0; f < half; ++f) {
            double sr = 0.0, si = 0.0, sn = 0.0;
            for (int n = 0; n < n_cal; ++n) {
                const size_t row = ((size_t)hh * n_cal + n) * d;
                const double x = load_elem(q, dtype, row + f);
                const double y = load_elem(q, dtype, row + f + half);
                sr += x;
                si += y;
                sn += sqrt(x * x + y * y);
            }
            const double mr = sr / n_cal, mi = si / n_cal, mn = sn / n_cal;
            qc_out[(size_t)hh * d + f] = mr;
            qc_out[(size_t)hh * d + f + half] = mi;
            qn_out[(size_t)hh * half + f] = mn;
            r_out[(size_t)hh * half + f] = mn > 0.0 ? sqrt(mr * mr + mi * mi) / mn : 0.0;
        }
    }
}

/* Number of threads an OpenMP parallel region actually uses (for the CPU baseline record). */
int oracle_max_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
    int n = 0;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    (void)n_threads;
    return 1;
#endif
}
