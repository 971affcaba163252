// score_mfma.hip -- key scoring of bf16 caches on the matrix cores (gfx950, wave64).
//
// For one stream the G raw scores of key j are (see score.hip for the derivation)
//     s_h(j) = sum_d Qrot_h[d] * ktilde_j[d]  +  sum_f W_h[f] * |ktilde_{j,f}|
// i.e. a [keys x 128] x [128 x G] product plus a [keys x 64] x [64 x G] product of the band
// norms: a dense contraction with a skinny right-hand side.  It runs on
// v_mfma_f32_16x16x32_bf16 (16 keys x 16 columns x 32-deep per instruction):
//   * A = the cached bf16 key rows, used as loaded (exact), and the band norms |k_f| computed
//     in fp32 on the vector ALU and split into SPLIT bf16 terms (hi + lo [+ lo2]);
//   * B = the per-stream constants Qrot_h and W_h, each split into SPLIT bf16 terms; column
//     c = b*G + h carries term b of head h, so summing the SPLIT columns of a head recovers the
//     fp32 constant to 2^-17 (SPLIT = 2) or 2^-26 (SPLIT = 3) relative, accumulation in fp32.
//     For the norm part only the products of terms a (norm) and b (weight) with a + b < SPLIT
//     are formed (the rest are below the split's resolution).
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, element e < 8, r < 4):
//   A: row l%16, k = 8*(l/16) + e;  B: k = 8*(l/16) + e, column l%16;  D: row 4*(l/16) + r, column l%16.
// Lane l of a wave loads 16 bytes at byte offset 64*kb + 16*(l/16) (kb < 4) of key row l%16 of
// the tile: instruction kb reads 64 contiguous bytes of each of 16 rows, and the four loads give
// MFMA kb its A operand (dims 32kb + 8(l/16) + e).  The lane then also holds, for its 16 bands
// 8(l/16)+e and 32+8(l/16)+e, both halves (re = dim f, im = dim f+64) of every band: the band
// norms need no cross-lane exchange.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// term b (0-based) of the bf16 expansion x = t0 + t1 + t2 + ... (each residual is exact in fp32)
__device__ __forceinline__ float bf16_term(float x, int b)
{
    float r = x;
    for (int i = 0; i < b; ++i) r = r - (float)(__bf16)r;
    return (float)(__bf16)r;
}

template <int G, int SPLIT>
struct MfmaConsts {
    bf16x8 bt[4];              // trig part, K-block kb: dims 32kb + 8g + e
    bf16x8 bn[SPLIT][2];       // norm part, norm term a, band half: bands 32*half + 8g + e
};

// Build this lane's B operands for one stream (qrow: Qrot of head 0 of the group, wrow: W of
// head 0; consecutive heads are 128 / 64 floats apart).
template <int G, int SPLIT>
__device__ __forceinline__ void load_consts(MfmaConsts<G, SPLIT> &c, const float *__restrict__ qrow,
                                            const float *__restrict__ wrow)
{
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g = lane >> 4;
    const bool live = j < SPLIT * G;
    const int b = live ? j / G : 0, h = live ? j % G : 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = live ? qrow[h * TRIA_D + 32 * kb + 8 * g + e] : 0.f;
            c.bt[kb][e] = (__bf16)bf16_term(x, b);
        }
#pragma unroll
    for (int a = 0; a < SPLIT; ++a)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (live && a + b < SPLIT) ? wrow[h * TRIA_HALF + 32 * half + 8 * g + e] : 0.f;
                c.bn[a][half][e] = (__bf16)bf16_term(x, b);
            }
}

// Load this lane's 64 bytes of a 16-key tile (zeros for keys at or past `valid`).
__device__ __forceinline__ void load_tile(u32x4 (&ka)[4], const u32x4 *__restrict__ tile_base, int valid)
{
    const int lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
    if (row < valid) {
        const u32x4 *p = tile_base + row * 16 + g;   // row = 16 x 16 B; byte 64kb + 16g = word 4kb + g
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ka[kb] = __builtin_nontemporal_load(p + 4 * kb);
    } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ka[kb] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Raw scores of one 16-key tile.  Returns D: lane l holds, for keys 4*(l/16) + r, the sum of
// columns l%16: after combine_columns the lanes with l%16 < G hold head l%16.
template <int G, int SPLIT>
__device__ __forceinline__ floatx4 score_tile16(const u32x4 (&ka)[4], const MfmaConsts<G, SPLIT> &c)
{
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kb]), c.bt[kb], acc, 0, 0, 0);

    // band norms of bands 8g+e (re: ka[0], im: ka[2]) and 32+8g+e (re: ka[1], im: ka[3])
    float n[2][8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const u32x4 x = ka[half], y = ka[2 + half];
        const uint32_t xs[4] = {x[0], x[1], x[2], x[3]}, ys[4] = {y[0], y[1], y[2], y[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float r0 = bf16_lo(xs[i]), r1 = bf16_hi(xs[i]);
            const float i0 = bf16_lo(ys[i]), i1 = bf16_hi(ys[i]);
            n[half][2 * i] = __builtin_amdgcn_sqrtf(fmaf(r0, r0, i0 * i0));
            n[half][2 * i + 1] = __builtin_amdgcn_sqrtf(fmaf(r1, r1, i1 * i1));
        }
    }
#pragma unroll
    for (int a = 0; a < SPLIT; ++a)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 v = (__bf16)n[half][e];
                t[e] = v;
                n[half][e] -= (float)v;        // exact residual for the next term
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t, c.bn[a][half], acc, 0, 0, 0);
        }
    return acc;
}

// Sum the SPLIT columns of each head into the lanes with l%16 < G.
template <int G, int SPLIT>
__device__ __forceinline__ floatx4 combine_columns(floatx4 acc)
{
    const int lane = threadIdx.x & 63;
    floatx4 s = acc;
#pragma unroll
    for (int b = 1; b < SPLIT; ++b) {
        const int src = (lane & 48) | (((lane & 15) + b * G) & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] += __shfl(acc[r], src, 64);
    }
    return s;
}

// Running moments of one head over the values a lane sees: sums of (v - p) and (v - p)^2 in fp64
// around a pivot p (the lane's first value), so the variance does not cancel; min and max.
struct Moments {
    double n, s1, s2;
    float p, mn, mx;
    __device__ void init() { n = 0.0; s1 = 0.0; s2 = 0.0; p = 0.f; mn = INFINITY; mx = -INFINITY; }
    __device__ void add(float v)
    {
        if (n == 0.0) p = v;
        const double d = (double)v - (double)p;
        n += 1.0;
        s1 += d;
        s2 = fma(d, d, s2);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    __device__ double mean() const { return n > 0.0 ? (double)p + s1 / n : 0.0; }
    __device__ double m2() const { return n > 0.0 ? fmax(s2 - s1 * (s1 / n), 0.0) : 0.0; }
};

// (count, mean, M2, min, max) with Chan et al.'s pairwise merge.
struct Merged {
    double n, mean, m2;
    float mn, mx;
    __device__ void init() { n = 0.0; mean = 0.0; m2 = 0.0; mn = INFINITY; mx = -INFINITY; }
    __device__ void merge(double nb, double meanb, double m2b, float mnb, float mxb)
    {
        if (nb == 0.0) return;
        const double tot = n + nb;
        const double delta = meanb - mean;
        mean += delta * (nb / tot);
        m2 += m2b + delta * delta * (n * nb / tot);
        n = tot;
        mn = fminf(mn, mnb);
        mx = fmaxf(mx, mxb);
    }
};

// Merge the moments of the 4 lanes of a wave that hold the same head (lanes h, h+16, h+32, h+48).
__device__ __forceinline__ Merged wave_merge_heads(const Moments &m)
{
    Merged a;
    a.n = m.n; a.mean = m.mean(); a.m2 = m.m2(); a.mn = m.mn; a.mx = m.mx;
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
        const double nb = __shfl_xor(a.n, o, 64), meanb = __shfl_xor(a.mean, o, 64), m2b = __shfl_xor(a.m2, o, 64);
        const float mnb = __shfl_xor(a.mn, o, 64), mxb = __shfl_xor(a.mx, o, 64);
        a.merge(nb, meanb, m2b, mnb, mxb);
    }
    return a;
}

__device__ __forceinline__ bool flat_head_m(double mn, double mx)
{
    return (mx - mn) <= ldexp(fmax(fabs(mn), fabs(mx)), -16);
}

// ---- tiled path: block = (stream, 1024-key tile); raw scores to the workspace ------------------
template <int G, int SPLIT>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_tile_kernel(
    const u32x4 *__restrict__ k, const float *__restrict__ qrot, const float *__restrict__ W, int L, int Hkv,
    int N, int tiles, float *__restrict__ raw, double *__restrict__ part, int *__restrict__ err)
{
    __shared__ double sm_n[4][G], sm_mean[4][G], sm_m2[4][G];
    __shared__ float sm_mn[4][G], sm_mx[4][G];
    const int sid = blockIdx.x / tiles;
    const int tile = blockIdx.x - sid * tiles;
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;

    MfmaConsts<G, SPLIT> c;
    load_consts<G, SPLIT>(c, qrot + (size_t)sid * G * TRIA_D, W + ((size_t)l * Hkv + g) * G * TRIA_HALF);

    const int j0 = tile * kTileKeys;
    const int nkeys = min(kTileKeys, N - j0);
    const int ntiles16 = (nkeys + 15) >> 4;
    const u32x4 *kb = k + ((size_t)sid * N + j0) * 16;
    Moments m;
    m.init();
    bool bad = false;
    const bool vec4 = (N & 3) == 0 && ((uintptr_t)raw & 15) == 0;
    u32x4 cur[4];
    int t = wid;
    if (t < ntiles16) load_tile(cur, kb + (size_t)t * 16 * 16, nkeys - t * 16);
    for (; t < ntiles16; t += 4) {
        u32x4 nxt[4];
        const int tn = t + 4;
        if (tn < ntiles16) load_tile(nxt, kb + (size_t)tn * 16 * 16, nkeys - tn * 16);
        floatx4 acc = score_tile16<G, SPLIT>(cur, c);
        acc = combine_columns<G, SPLIT>(acc);
        if (col < G) {
            const int key = t * 16 + 4 * grp;                    // first of this lane's 4 keys
            float *dst = raw + ((size_t)sid * G + col) * N + j0 + key;
            const int nv = min(4, nkeys - key);
            if (nv == 4 && vec4) {
                *(float4 *)dst = make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r < nv) dst[r] = acc[r];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r < nv) {
                    bad |= !isfinite(acc[r]);
                    m.add(acc[r]);
                }
        }
        if (tn < ntiles16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
        }
    }
    if (bad) atomicOr(err, 1);
    const Merged wm = wave_merge_heads(m);
    if (lane < G) {
        sm_n[wid][lane] = wm.n; sm_mean[wid][lane] = wm.mean; sm_m2[wid][lane] = wm.m2;
        sm_mn[wid][lane] = wm.mn; sm_mx[wid][lane] = wm.mx;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        Merged t2;
        t2.init();
        for (int w = 0; w < 4; ++w) t2.merge(sm_n[w][h], sm_mean[w][h], sm_m2[w][h], sm_mn[w][h], sm_mx[w][h]);
        double *p = part + (((size_t)sid * tiles + tile) * G + h) * 4;
        p[0] = t2.mean;
        p[1] = t2.m2;
        p[2] = (double)t2.mn;
        p[3] = (double)t2.mx;
    }
}

// ---- fused path: one block per stream, raw scores kept in LDS ---------------------------------
template <int G, int SPLIT>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_fused_kernel(
    const u32x4 *__restrict__ k, const float *__restrict__ qrot, const float *__restrict__ W, int L, int Hkv,
    int N, float *__restrict__ F, float *__restrict__ raw_out, float *__restrict__ stats, int *__restrict__ err)
{
    extern __shared__ float raw[];                 // [G][NP], NP = N | 1 (odd stride: no bank conflicts)
    const int NP = N | 1;
    __shared__ double sm_n[4][G], sm_mean[4][G], sm_m2[4][G];
    __shared__ float sm_mn[4][G], sm_mx[4][G];
    __shared__ float zmu[G], zinv[G];
    const int sid = blockIdx.x;
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;

    MfmaConsts<G, SPLIT> c;
    load_consts<G, SPLIT>(c, qrot + (size_t)sid * G * TRIA_D, W + ((size_t)l * Hkv + g) * G * TRIA_HALF);

    const int ntiles16 = (N + 15) >> 4;
    const u32x4 *kb = k + (size_t)sid * N * 16;
    Moments m;
    m.init();
    bool bad = false;
    u32x4 cur[4];
    int t = wid;
    if (t < ntiles16) load_tile(cur, kb + (size_t)t * 16 * 16, N - t * 16);
    for (; t < ntiles16; t += 4) {
        u32x4 nxt[4];
        const int tn = t + 4;
        if (tn < ntiles16) load_tile(nxt, kb + (size_t)tn * 16 * 16, N - tn * 16);
        floatx4 acc = score_tile16<G, SPLIT>(cur, c);
        acc = combine_columns<G, SPLIT>(acc);
        if (col < G) {
            const int key = t * 16 + 4 * grp;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key + r < N) {
                    raw[col * NP + key + r] = acc[r];
                    bad |= !isfinite(acc[r]);
                    m.add(acc[r]);
                }
        }
        if (tn < ntiles16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
        }
    }
    if (bad) atomicOr(err, 1);
    const Merged wm = wave_merge_heads(m);
    if (lane < G) {
        sm_n[wid][lane] = wm.n; sm_mean[wid][lane] = wm.mean; sm_m2[wid][lane] = wm.m2;
        sm_mn[wid][lane] = wm.mn; sm_mx[wid][lane] = wm.mx;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        Merged t2;
        t2.init();
        for (int w = 0; w < 4; ++w) t2.merge(sm_n[w][h], sm_mean[w][h], sm_m2[w][h], sm_mn[w][h], sm_mx[w][h]);
        const double sd = flat_head_m((double)t2.mn, (double)t2.mx) ? 0.0 : sqrt(t2.m2 / (double)N);
        zmu[h] = (float)t2.mean;
        zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
        if (stats) {
            stats[((size_t)sid * G + h) * 2 + 0] = (float)t2.mean;
            stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
        }
    }
    __syncthreads();
    if (raw_out)
        for (int i = threadIdx.x; i < G * N; i += kScoreThreads)
            raw_out[(size_t)sid * G * N + i] = raw[(i / N) * NP + i % N];
    float *fo = F + (size_t)sid * N;
    for (int j = threadIdx.x; j < N; j += kScoreThreads) {
        float z = -INFINITY;
#pragma unroll
        for (int h = 0; h < G; ++h) z = fmaxf(z, (raw[h * NP + j] - zmu[h]) * zinv[h]);
        fo[j] = z;
    }
}

// ---- launch ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_mfma_g(const tria_calib *c, const void *k, int n_seq, int N, const float *qrot, float *F,
                                float *raw_out, float *stats, const tria_score_ws &lay, char *ws, hipStream_t st)
{
    constexpr int SPLIT = 3 * G <= 16 ? 3 : 2;
    const int streams = n_seq * c->L * c->Hkv;
    int *err = (int *)(ws + lay.err_off);
    if (!lay.tiled) {
        const size_t lds = (size_t)G * (N | 1) * 4;
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void *)score_mfma_fused_kernel<G, SPLIT>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLdsMax);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        score_mfma_fused_kernel<G, SPLIT><<<streams, kScoreThreads, lds, st>>>(
            (const u32x4 *)k, qrot, c->W, c->L, c->Hkv, N, F, raw_out, stats, err);
        return hipGetLastError();
    }
    float *raw = raw_out ? raw_out : (float *)(ws + lay.raw_off);
    double *part = (double *)(ws + lay.part_off);
    const long long blocks = (long long)streams * lay.tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    score_mfma_tile_kernel<G, SPLIT><<<(unsigned)blocks, kScoreThreads, 0, st>>>(
        (const u32x4 *)k, qrot, c->W, c->L, c->Hkv, N, lay.tiles, raw, part, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_zmax(c->G, raw, part, streams, N, lay.tiles, F, stats, st);
}

hipError_t launch_score_mfma(const tria_calib *c, const void *k, int n_seq, int N, const float *qrot, float *F,
                             float *raw, float *stats, const tria_score_ws &lay, char *ws, hipStream_t st)
{
    switch (c->G) {
    case 1: return launch_mfma_g<1>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 2: return launch_mfma_g<2>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 3: return launch_mfma_g<3>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 4: return launch_mfma_g<4>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 5: return launch_mfma_g<5>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 6: return launch_mfma_g<6>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 7: return launch_mfma_g<7>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    case 8: return launch_mfma_g<8>(c, k, n_seq, N, qrot, F, raw, stats, lay, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tria
