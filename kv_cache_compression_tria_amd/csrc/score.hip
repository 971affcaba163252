// score.hip -- query rotation, key scoring, per-head z-score and GQA max (gfx950).
//
// Score of key j for query head h (TriAttention pages: zhichai.net section
// "TriAttention：把理论变成算法" items 1-2; chenxutan.com/d/2624 sections 3.1 and 3.3;
// 10100.com "TriAttention方法" for the (1-R) weight and the sum of the two parts):
//
//   s_h(j) = mean_{d in D} sum_f |qbar_f||k_f| cos(w_f (t+d-p_j) + arg qbar_f - arg k_f)
//          + sum_f (1 - R_f) E|q_f| |k_f|
//
// With the keys cached after RoPE (band f of the cached key is k_f exp(i w_f p_j)) the first
// sum is the real part of sum_f Q_f conj(ktilde_f) with Q_f = qbar_f exp(i w_f t) C(f),
// C(f) = mean_d exp(i w_f d): the key's own phase cancels, so scoring a key is a 128-long dot
// product with the rotated query plus 64 band norms against the norm weights.
// Q is built once per (sequence, layer, head) from t with an exact integer range reduction
// (t * w_f/2pi mod 1 from a 64-bit fixed-point turn fraction) and fp64 sin/cos.
//
// Normalisation (10100.com "TriAttention方法"; watermelonwater.tech "TriAttention 方案设计"
// item 4): per head, z = (s - mean)/std over the stream's N keys (population std, fp64
// accumulation, deterministic order); F(j) = max over the G heads of the group.  A head whose
// scores are equal up to rounding has std 0 and z = 0.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

tria_score_ws score_ws_layout(const tria_calib *c, tria_dtype dt, int n_seq, int N, unsigned flags)
{
    tria_score_ws w{};
    const size_t streams = (size_t)n_seq * c->L * c->Hkv;
    const size_t heads = streams * c->G;
    const size_t fused_lds = (size_t)c->G * (size_t)N * 4 + (size_t)c->G * 192 * 4;
    w.tiled = fused_lds > (size_t)kFusedLdsMax;
    w.tiles = (N + kTileKeys - 1) / kTileKeys;
    // pre-RoPE bf16 keys on the staged clusters (streams too long for one block, or 256 or more
    // streams): turned to their positions inside the kernel; the other per-key forms on the
    // vector ALU
    w.rot = dt == TRIA_BF16 && (flags & TRIA_KEYS_PRE_ROPE) && (w.tiled || streams >= kStageShortStreams) &&
            !(flags & (TRIA_OFFSET_MAX | TRIA_SCORE_TILED | TRIA_TRIG_WEIGHT_R)) && stage_path_applies(c->G, N);
    const bool perkey = (flags & (TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE)) != 0 && !w.rot;
    const bool mfma = dt == TRIA_BF16 && !perkey;          // the matrix-core operand prologue runs
    // long bf16 streams: stream clusters when the device offers them; streams that fit one block
    // too when there are enough of them to fill the chip
    const bool free_path = mfma && !(flags & (TRIA_OFFSET_MAX | TRIA_SCORE_TILED));
    w.cluster = free_path && (w.tiled ? cluster_path_applies(c->G, N)
                                      : streams >= kStageShortStreams && stage_path_applies(c->G, N));
    // raw scores staged in HBM: the per-key and offset-max kernels always, the other long streams
    // unless a stream cluster keeps them on chip
    w.has_raw = perkey || (flags & TRIA_OFFSET_MAX) || (w.tiled && !w.cluster);
    size_t off = 0;
    w.err_off = 0;
    off = 256;
    if (!mfma) {
        // rotated queries of every head (the matrix-core prologue keeps its own in LDS)
        w.qrot_off = off;
        off += align256(heads * TRIA_D * sizeof(float));
    }
    if (mfma) {
        // matrix-core operands of every stream in lane layout, and the per-head pivots
        w.ops_off = off;
        off += align256(streams * (size_t)mfma_ops_per_stream(c->G) * 64 * 16);
        w.pivot_off = off;
        off += align256(heads * sizeof(float));
    }
    if (w.cluster) {
        // partial sums exchanged inside stream clusters (two round slots per block), the clusters'
        // arrival counters (one per cluster) or flags (one per block)
        w.xpart_off = off;
        off += align256((size_t)kClusterMaxBlocks * 2 * TRIA_MAX_G * 4 * sizeof(double));
        w.arrive_off = off;
        off += align256((size_t)kClusterMaxBlocks * sizeof(uint32_t));
        // the side copy of every kSampleStride-th F, which the selection samples
        w.samp_off = off;
        off += align256(streams * (size_t)((N + kSampleStride - 1) / kSampleStride) * sizeof(float));
    }
    if (w.has_raw) {
        // raw scores [streams][G][N], tile partials and per-head mean / 1/std
        w.raw_off = off;
        off += align256(heads * (size_t)N * sizeof(float));
        w.part_off = off;
        off += align256(streams * (size_t)w.tiles * c->G * 4 * sizeof(double));
        w.zst_off = off;
        off += align256(heads * 2 * sizeof(float));
    }
    w.total = off;
    return w;
}

// ---- a2: rotated queries --------------------------------------------------------------------
// qrot[s][l][h][f] = Re Q_f, qrot[..][64+f] = Im Q_f with Q_f = P_f * exp(i w_f t_s) and
// P_f = qbar_f * mean_d exp(i w_f d) precomputed in fp64 at table load; with R (the
// R-weighted variant) Q_f is scaled by R_f.
__global__ __launch_bounds__(256) void rotate_queries_kernel(const double2 *__restrict__ P,
                                                             const uint64_t *__restrict__ nu,
                                                             const int32_t *__restrict__ t, int LHq,
                                                             int total, const float *__restrict__ R,
                                                             float *__restrict__ qrot,
                                                             int *__restrict__ err)
{
    // clear the non-finite flag of this call (no memset node)
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
    const int gh = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int f = threadIdx.x & 63;
    if (gh >= total) return;
    const int s = gh / LHq;
    const int lh = gh - s * LHq;
    const int64_t tt = t[s];
    const uint64_t turns = (uint64_t)tt * nu[f];                // t * w_f / 2pi mod 1, exact
    const double r = (double)(int64_t)turns * 0x1p-64;           // in [-1/2, 1/2) turns
    double sn, cs;
    sincospi(2.0 * r, &sn, &cs);
    const double2 p = P[(size_t)lh * TRIA_HALF + f];
    const double wr = R ? (double)R[(size_t)lh * TRIA_HALF + f] : 1.0;
    qrot[(size_t)gh * TRIA_D + f] = (float)(wr * (p.x * cs - p.y * sn));
    qrot[(size_t)gh * TRIA_D + TRIA_HALF + f] = (float)(wr * (p.x * sn + p.y * cs));
}

hipError_t launch_rotate(const tria_calib *c, const int32_t *t, int n_seq, float *qrot, int *err, bool weight_r,
                         hipStream_t st)
{
    const int total = n_seq * c->L * c->Hq;
    const int LHq = c->L * c->Hq;
    rotate_queries_kernel<<<(total + 3) / 4, 256, 0, st>>>(c->P, c->nu, t, LHq, total, weight_r ? c->R : nullptr,
                                                           qrot, err);
    return hipGetLastError();
}

// ---- a3: score one key (one lane per key) ---------------------------------------------------
// qw (LDS, 16-byte aligned) holds, per head, 48 float4: [0,32) the rotated query (dims 0..127)
// and [32,48) the norm weights (bands 0..63).
template <bool BF16, int G>
__device__ __forceinline__ void score_key(const uint4 *__restrict__ row, const float4 *qw, float (&s)[G])
{
    constexpr int RV = BF16 ? 16 : 32;   // 16-byte words per 128-dim row
    uint4 r[RV];
#pragma unroll
    for (int i = 0; i < RV; ++i) r[i] = row[i];
    // Re-read the per-head constants from LDS for every key: an opaque zero offset keeps the
    // compiler from hoisting G*192 values into registers across the key loop.
    int lds_off = 0;
    asm volatile("" : "+s"(lds_off));
    qw += lds_off;
    float a[G], b[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { a[h] = 0.f; b[h] = 0.f; }
#pragma unroll
    for (int c = 0; c < 8; ++c) {        // bands 8c .. 8c+7
        float re[8], im[8], n[8];
        if (BF16) {
            const uint4 x = r[c], y = r[8 + c];
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                re[2 * i] = bf16_lo(xs[i]); re[2 * i + 1] = bf16_hi(xs[i]);
                im[2 * i] = bf16_lo(ys[i]); im[2 * i + 1] = bf16_hi(ys[i]);
            }
        } else {
            const uint4 x0 = r[2 * c], x1 = r[2 * c + 1], y0 = r[16 + 2 * c], y1 = r[16 + 2 * c + 1];
            re[0] = __uint_as_float(x0.x); re[1] = __uint_as_float(x0.y);
            re[2] = __uint_as_float(x0.z); re[3] = __uint_as_float(x0.w);
            re[4] = __uint_as_float(x1.x); re[5] = __uint_as_float(x1.y);
            re[6] = __uint_as_float(x1.z); re[7] = __uint_as_float(x1.w);
            im[0] = __uint_as_float(y0.x); im[1] = __uint_as_float(y0.y);
            im[2] = __uint_as_float(y0.z); im[3] = __uint_as_float(y0.w);
            im[4] = __uint_as_float(y1.x); im[5] = __uint_as_float(y1.y);
            im[6] = __uint_as_float(y1.z); im[7] = __uint_as_float(y1.w);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) n[i] = __builtin_amdgcn_sqrtf(fmaf(re[i], re[i], im[i] * im[i]));
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float4 *q = qw + h * 48;
            const float4 qa0 = q[2 * c], qa1 = q[2 * c + 1];
            const float4 qb0 = q[16 + 2 * c], qb1 = q[16 + 2 * c + 1];
            const float qa[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
            const float qb[8] = {qb0.x, qb0.y, qb0.z, qb0.w, qb1.x, qb1.y, qb1.z, qb1.w};
            const float4 w0 = q[32 + 2 * c], w1 = q[32 + 2 * c + 1];
            const float qw8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a[h] = fmaf(qa[i], re[i], a[h]);
                a[h] = fmaf(qb[i], im[i], a[h]);
                b[h] = fmaf(qw8[i], n[i], b[h]);
            }
            // keep the scheduler from pulling every head's constants forward at once
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = a[h] + b[h];
}

template <int G>
__device__ __forceinline__ void load_qw(float *qw, const float *__restrict__ qrot,
                                        const float *__restrict__ W, size_t qhead0, size_t whead0)
{
    for (int i = threadIdx.x; i < G * 192; i += blockDim.x) {
        const int hh = i / 192, c = i - hh * 192;
        qw[i] = c < 128 ? qrot[(qhead0 + hh) * TRIA_D + c] : W[(whead0 + hh) * TRIA_HALF + (c - 128)];
    }
}

// Block-wide reductions over kScoreThreads threads (4 waves) of G values, fixed order.
template <int G>
__device__ __forceinline__ void block_sum_g(double (&v)[G], double *red /* [4][G] */)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < G; ++h) v[h] = wave_sum(v[h]);
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) red[wid * G + h] = v[h];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) v[h] = ((red[h] + red[G + h]) + red[2 * G + h]) + red[3 * G + h];
    __syncthreads();
}

template <int G>
__device__ __forceinline__ void block_minmax_g(float (&mn)[G], float (&mx)[G], float *red /* [4][2G] */)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < G; ++h) { mn[h] = wave_min(mn[h]); mx[h] = wave_max(mx[h]); }
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) { red[wid * 2 * G + h] = mn[h]; red[wid * 2 * G + G + h] = mx[h]; }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mn[h] = fminf(fminf(red[h], red[2 * G + h]), fminf(red[4 * G + h], red[6 * G + h]));
        mx[h] = fmaxf(fmaxf(red[G + h], red[3 * G + h]), fmaxf(red[5 * G + h], red[7 * G + h]));
    }
    __syncthreads();
}

// A head whose scores span at most 2^-16 of their largest magnitude is constant (scores equal up
// to rounding): it carries no ranking information, std := 0 and z := 0.
__device__ __forceinline__ bool flat_head(double mn, double mx)
{
    return (mx - mn) <= ldexp(fmax(fabs(mn), fabs(mx)), -16);
}

// ---- fused path: one block per stream, raw scores kept in LDS --------------------------------
template <bool BF16, int G>
__global__ __launch_bounds__(kScoreThreads) void score_fused_kernel(
    const uint4 *__restrict__ k, const float *__restrict__ qrot, const float *__restrict__ W, int L,
    int Hkv, int N, float *__restrict__ F, float *__restrict__ raw_out, float *__restrict__ stats,
    int *__restrict__ err)
{
    constexpr int RV = BF16 ? 16 : 32;
    extern __shared__ float4 smem4[];
    float4 *qw = smem4;                           // [G][48] float4
    float *raw = (float *)(smem4 + G * 48);       // [G][N]
    __shared__ double redd[4 * G];
    __shared__ float redf[8 * G];
    __shared__ float zmu[G], zinv[G];

    const int sid = blockIdx.x;                       // (s*L + l)*Hkv + g
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    load_qw<G>((float *)qw, qrot, W, (size_t)sid * G, ((size_t)l * Hkv + g) * G);
    __syncthreads();

    const uint4 *kb = k + (size_t)sid * N * RV;
#pragma unroll 1
    for (int j = threadIdx.x; j < N; j += kScoreThreads) {
        float s[G];
        score_key<BF16, G>(kb + (size_t)j * RV, qw, s);
#pragma unroll
        for (int h = 0; h < G; ++h) raw[h * N + j] = s[h];
    }
    __syncthreads();
    if (raw_out)
        for (int i = threadIdx.x; i < G * N; i += kScoreThreads) raw_out[(size_t)sid * G * N + i] = raw[i];

    double sum[G];
    float mn[G], mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { sum[h] = 0.0; mn[h] = INFINITY; mx[h] = -INFINITY; }
    bool bad = false;
    for (int j = threadIdx.x; j < N; j += kScoreThreads)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float v = raw[h * N + j];
            bad |= !isfinite(v);
            sum[h] += (double)v;
            mn[h] = fminf(mn[h], v);
            mx[h] = fmaxf(mx[h], v);
        }
    if (bad) atomicOr(err, 1);
    block_sum_g<G>(sum, redd);
    block_minmax_g<G>(mn, mx, redf);
    double mean[G], m2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { mean[h] = sum[h] / (double)N; m2[h] = 0.0; }
    for (int j = threadIdx.x; j < N; j += kScoreThreads)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const double dv = (double)raw[h * N + j] - mean[h];
            m2[h] = fma(dv, dv, m2[h]);
        }
    block_sum_g<G>(m2, redd);
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const double sd = flat_head((double)mn[h], (double)mx[h]) ? 0.0 : sqrt(m2[h] / (double)N);
        zmu[h] = (float)mean[h];
        zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
        if (stats) {
            stats[((size_t)sid * G + h) * 2 + 0] = (float)mean[h];
            stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
        }
    }
    __syncthreads();
    float *fo = F + (size_t)sid * N;
    for (int j = threadIdx.x; j < N; j += kScoreThreads) {
        float z = -INFINITY;
#pragma unroll
        for (int h = 0; h < G; ++h) z = fmaxf(z, (raw[h * N + j] - zmu[h]) * zinv[h]);
        fo[j] = z;
    }
}

// ---- tiled path: raw scores through the workspace, per-tile partial moments ------------------
constexpr int kKeysPerThread = kTileKeys / kScoreThreads;

template <bool BF16, int G>
__global__ __launch_bounds__(kScoreThreads) void score_tile_kernel(
    const uint4 *__restrict__ k, const float *__restrict__ qrot, const float *__restrict__ W, int L,
    int Hkv, int N, int tiles, float *__restrict__ raw, double *__restrict__ part, int *__restrict__ err)
{
    constexpr int RV = BF16 ? 16 : 32;
    __shared__ float4 qw[G * 48];
    __shared__ double redd[4 * G];
    __shared__ float redf[8 * G];
    const int sid = blockIdx.x / tiles;
    const int tile = blockIdx.x - sid * tiles;
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    load_qw<G>((float *)qw, qrot, W, (size_t)sid * G, ((size_t)l * Hkv + g) * G);
    __syncthreads();

    const int j0 = tile * kTileKeys;
    const int nt = min(kTileKeys, N - j0);
    const uint4 *kb = k + (size_t)sid * N * RV;
    float sv[kKeysPerThread][G];
    bool bad = false;
#pragma unroll
    for (int kk = 0; kk < kKeysPerThread; ++kk) {
        const int j = j0 + kk * kScoreThreads + threadIdx.x;
        if (j < N) {
            score_key<BF16, G>(kb + (size_t)j * RV, qw, sv[kk]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                raw[((size_t)sid * G + h) * N + j] = sv[kk][h];
                bad |= !isfinite(sv[kk][h]);
            }
        }
    }
    if (bad) atomicOr(err, 1);

    double sum[G];
    float mn[G], mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { sum[h] = 0.0; mn[h] = INFINITY; mx[h] = -INFINITY; }
#pragma unroll
    for (int kk = 0; kk < kKeysPerThread; ++kk) {
        const int j = j0 + kk * kScoreThreads + threadIdx.x;
        if (j < N)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                sum[h] += (double)sv[kk][h];
                mn[h] = fminf(mn[h], sv[kk][h]);
                mx[h] = fmaxf(mx[h], sv[kk][h]);
            }
    }
    block_sum_g<G>(sum, redd);
    block_minmax_g<G>(mn, mx, redf);
    double mean[G], m2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { mean[h] = sum[h] / (double)nt; m2[h] = 0.0; }
#pragma unroll
    for (int kk = 0; kk < kKeysPerThread; ++kk) {
        const int j = j0 + kk * kScoreThreads + threadIdx.x;
        if (j < N)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const double dv = (double)sv[kk][h] - mean[h];
                m2[h] = fma(dv, dv, m2[h]);
            }
    }
    block_sum_g<G>(m2, redd);
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        double *p = part + (((size_t)sid * tiles + tile) * G + h) * 4;
        p[0] = mean[h];
        p[1] = m2[h];
        p[2] = (double)mn[h];
        p[3] = (double)mx[h];
    }
}

template <int G>
__global__ __launch_bounds__(kScoreThreads) void zmax_tile_kernel(const float *__restrict__ raw,
                                                                   const double *__restrict__ part,
                                                                   int N, int tiles, float *__restrict__ F,
                                                                   float *__restrict__ stats)
{
    __shared__ float zmu[G], zinv[G];
    const int sid = blockIdx.x / tiles;
    const int tile = blockIdx.x - sid * tiles;
    if (threadIdx.x < G) {
        // Chan et al. pairwise merge of the per-tile (count, mean, M2), tiles in order.
        const int h = threadIdx.x;
        double n = 0.0, mean = 0.0, m2 = 0.0, mn = INFINITY, mx = -INFINITY;
        for (int tt = 0; tt < tiles; ++tt) {
            const double *p = part + (((size_t)sid * tiles + tt) * G + h) * 4;
            const double nb = (double)min(kTileKeys, N - tt * kTileKeys);
            const double tot = n + nb;
            const double delta = p[0] - mean;
            mean += delta * (nb / tot);
            m2 += p[1] + delta * delta * (n * nb / tot);
            n = tot;
            mn = fmin(mn, p[2]);
            mx = fmax(mx, p[3]);
        }
        const double sd = flat_head(mn, mx) ? 0.0 : sqrt(m2 / (double)N);
        zmu[h] = (float)mean;
        zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
        if (stats && tile == 0) {
            stats[((size_t)sid * G + h) * 2 + 0] = (float)mean;
            stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
        }
    }
    __syncthreads();
    const int j0 = tile * kTileKeys;
#pragma unroll
    for (int kk = 0; kk < kKeysPerThread; ++kk) {
        const int j = j0 + kk * kScoreThreads + threadIdx.x;
        if (j < N) {
            float z = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h)
                z = fmaxf(z, (raw[((size_t)sid * G + h) * N + j] - zmu[h]) * zinv[h]);
            F[(size_t)sid * N + j] = z;
        }
    }
}

hipError_t launch_zmax(int G, const float *raw, const double *part, int streams, int N, int tiles, float *F,
                       float *stats, hipStream_t st)
{
    const long long blocks = (long long)streams * tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (G) {
#define TRIA_ZMAX_CASE(GG) \
    case GG: zmax_tile_kernel<GG><<<(unsigned)blocks, kScoreThreads, 0, st>>>(raw, part, N, tiles, F, stats); break;
    TRIA_ZMAX_CASE(1) TRIA_ZMAX_CASE(2) TRIA_ZMAX_CASE(3) TRIA_ZMAX_CASE(4)
    TRIA_ZMAX_CASE(5) TRIA_ZMAX_CASE(6) TRIA_ZMAX_CASE(7) TRIA_ZMAX_CASE(8)
#undef TRIA_ZMAX_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- launch --------------------------------------------------------------------------------
template <bool BF16, int G>
static hipError_t launch_score_t(const tria_calib *c, const void *k, int n_seq, int N, const float *qrot,
                                 float *F, float *raw_out, float *stats, const tria_score_ws &lay, char *ws,
                                 hipStream_t st)
{
    const int streams = n_seq * c->L * c->Hkv;
    int *err = (int *)(ws + lay.err_off);
    if (!lay.tiled) {
        const size_t lds = (size_t)G * 192 * 4 + (size_t)G * N * 4;
        hipError_t e = allow_dynamic_lds((const void *)score_fused_kernel<BF16, G>, kFusedLdsMax + G * 192 * 4);
        if (e != hipSuccess) return e;
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        score_fused_kernel<BF16, G><<<streams, kScoreThreads, lds, st>>>(
            (const uint4 *)k, qrot, c->W, c->L, c->Hkv, N, F, raw_out, stats, err);
        return hipGetLastError();
    }
    if (!lay.has_raw) return hipErrorInvalidValue;   // the layout did not plan this path
    float *raw = raw_out ? raw_out : (float *)(ws + lay.raw_off);
    double *part = (double *)(ws + lay.part_off);
    const long long blocks = (long long)streams * lay.tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e;
    {
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        score_tile_kernel<BF16, G><<<(unsigned)blocks, kScoreThreads, 0, st>>>(
            (const uint4 *)k, qrot, c->W, c->L, c->Hkv, N, lay.tiles, raw, part, err);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    KernelTimer timer(TRIA_TIMER_NORMALISE, st);
    return launch_zmax(G, raw, part, streams, N, lay.tiles, F, stats, st);
}

template <bool BF16>
static hipError_t launch_score_d(const tria_calib *c, const void *k, int n_seq, int N, const float *qrot,
                                 float *F, float *raw, float *stats, const tria_score_ws &lay, char *ws,
                                 hipStream_t st)
{
    switch (c->G) {
    case 1: return launch_score_t<BF16, 1>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 2: return launch_score_t<BF16, 2>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 3: return launch_score_t<BF16, 3>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 4: return launch_score_t<BF16, 4>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 5: return launch_score_t<BF16, 5>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 6: return launch_score_t<BF16, 6>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 7: return launch_score_t<BF16, 7>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 8: return launch_score_t<BF16, 8>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_score(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                        const int32_t *t, int n_seq, int N, const float *qrot, float *F, float *raw,
                        float *stats, unsigned flags, const tria_score_ws &lay, char *ws, hipStream_t st)
{
    if (lay.rot) return launch_score_mfma(c, k, pos, t, n_seq, N, false, F, raw, stats, lay, ws, st);
    if (flags & (TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE))
        return launch_score_perkey(c, dt, k, pos, t, n_seq, N, flags, F, raw, stats, lay, ws, st);
    const bool weight_r = (flags & TRIA_TRIG_WEIGHT_R) != 0;
    if (flags & TRIA_OFFSET_MAX) return launch_score_maxd(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    // bf16 caches score on the matrix cores (their prologue rotates the queries itself); fp32
    // caches on the vector ALU, with the rotated queries from the workspace
    if (dt == TRIA_BF16) return launch_score_mfma(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    return launch_score_d<false>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
}

}  // namespace tria
