// score_perkey.hip -- key scoring with a per-key distance phase (gfx950, vector ALU).
//
// Two variants of step 1 that need each key's own phase (TriAttention pages: zhichai.net section
// "TriAttention：把理论变成算法" item 1, the series in w_f * distance; chenxutan.com/d/2624
// section 3.1):
//   * TRIA_PER_KEY_PHASE, keys cached after RoPE: the key's pre-RoPE band is recovered as
//     k_f = ktilde_f * exp(-i w_f p_j), and the series is evaluated in its literal per-key form
//       S_trig = sum_f Re[ P_f * exp(i w_f (t - p_j)) * conj(k_f) ],  P_f = qbar_f * mean_d exp(i w_f d),
//     i.e. the distance phase of every (key, band) is formed explicitly;
//   * TRIA_KEYS_PRE_ROPE, keys cached before RoPE: k_f is read directly and the same sum applies.
// The norm score is sum_f W_f |k_f| with W_f = (1 - R_f) E|q_f| (|k_f| = |ktilde_f|).
// Phases use the exact integer range reduction of the query rotation: w_f / 2pi is a 64-bit
// fraction of a turn (nu_f), n * nu_f mod 2^64 is exact for any integer n, and its top 32 bits
// give the angle in turns for the hardware sine and cosine.  Per band the key is turned by
// exp(-i w_f (t - p)) once, then every head costs three FMAs: Re[P_f conj(k e^{-i phi})] and
// W_f |k_f|.  The group's constants are wave-uniform and come through the scalar cache.
//
// One block scores one 1024-key tile of one stream (one thread per key, four keys per thread) and
// writes, like the matrix-core tile kernel, raw scores head-major [streams][G][N] and the tile's
// per-head sums (s1, s2 around 0 in fp64, min, max); the same statistics and z-max kernels
// finish the step.  Around 0 the fp64 sums lose at most (mean/std)^2 * 2^-48 of the variance.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

namespace {

// angle of n * w_f in turns, in [-1/2, 1/2): top 32 bits of the exact product n * nu_f mod 2^64
__device__ __forceinline__ float turns_of(int64_t n, uint64_t nu)
{
    const uint64_t prod = (uint64_t)n * nu;
    return (float)(int32_t)(uint32_t)(prod >> 32) * 0x1p-32f;
}

// sin and cos of 2 pi r for r in turns: the hardware sine / cosine take their argument in turns,
// and |r| <= 1/2 lies well inside their accurate range
__device__ __forceinline__ void sincos_turns(float r, float &s, float &c)
{
    s = __builtin_amdgcn_sinf(r);
    c = __builtin_amdgcn_cosf(r);
}

// Eight bands of a key row: real parts of bands f0..f0+7 and the matching imaginary parts.
template <bool BF16>
__device__ __forceinline__ void load_band_group(const char *__restrict__ row, int f0, float (&re)[8], float (&im)[8])
{
    if (BF16) {
        const uint4 *r = (const uint4 *)row;                 // 128 bf16 = 16 x 16 B
        const uint4 a = r[f0 / 8], b = r[(TRIA_HALF + f0) / 8];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            re[2 * i] = bf16_lo(aw[i]);
            re[2 * i + 1] = bf16_hi(aw[i]);
            im[2 * i] = bf16_lo(bw[i]);
            im[2 * i + 1] = bf16_hi(bw[i]);
        }
    } else {
        const float4 *r = (const float4 *)row;               // 128 fp32 = 32 x 16 B
        const float4 a0 = r[f0 / 4], a1 = r[f0 / 4 + 1];
        const float4 b0 = r[(TRIA_HALF + f0) / 4], b1 = r[(TRIA_HALF + f0) / 4 + 1];
        re[0] = a0.x; re[1] = a0.y; re[2] = a0.z; re[3] = a0.w;
        re[4] = a1.x; re[5] = a1.y; re[6] = a1.z; re[7] = a1.w;
        im[0] = b0.x; im[1] = b0.y; im[2] = b0.z; im[3] = b0.w;
        im[4] = b1.x; im[5] = b1.y; im[6] = b1.z; im[7] = b1.w;
    }
}

struct KSums {
    double s1, s2;
    float mn, mx;
};

}  // namespace

template <int G, bool BF16, bool PRE_ROPE>
__global__ __launch_bounds__(kScoreThreads) void score_perkey_tile_kernel(
    const void *__restrict__ k, const int32_t *__restrict__ pos, const int32_t *__restrict__ t,
    const float *__restrict__ PW, const uint64_t *__restrict__ nu, int L, int Hkv, int N, int tiles,
    float *__restrict__ raw, double *__restrict__ part)
{
    constexpr int RW = BF16 ? 256 : 512;     // row bytes
    __shared__ KSums red[kScoreThreads / 64][G];

    const int sid = blockIdx.x / tiles;
    const int tile = blockIdx.x - sid * tiles;
    const int s = sid / (Hkv * L);
    // the group's constants, band-major: Re P (G), Im P (G), W (G) per band.  Every lane reads the
    // same words, so they arrive through the scalar cache into scalar registers.
    const float *pw = PW + (size_t)(sid % (Hkv * L)) * TRIA_HALF * 3 * G;

    const int64_t ts = t[s];
    const int j0 = tile * kTileKeys;
    const int nkeys = min(kTileKeys, N - j0);
    KSums m[G];
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = {0.0, 0.0, INFINITY, -INFINITY};

    for (int jj = threadIdx.x; jj < nkeys; jj += kScoreThreads) {
        const size_t j = (size_t)sid * N + j0 + jj;
        const char *row = (const char *)k + j * RW;
        const int64_t p = pos[j];
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.f;
        for (int f0 = 0; f0 < TRIA_HALF; f0 += 8) {
            float re[8], im[8];
            load_band_group<BF16>(row, f0, re, im);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int f = f0 + e;
                float kr = re[e], ki = im[e];
                if (!PRE_ROPE) {
                    // recover the pre-RoPE band: k = ktilde * exp(-i w_f p)
                    float sp, cp;
                    sincos_turns(turns_of(p, nu[f]), sp, cp);
                    const float r2 = kr * cp + ki * sp, i2 = ki * cp - kr * sp;
                    kr = r2;
                    ki = i2;
                }
                const float mag = __builtin_amdgcn_sqrtf(fmaf(kr, kr, ki * ki));
                // distance phase w_f (t - p): turn the key by exp(-i phi)
                float sd, cd;
                sincos_turns(turns_of(ts - p, nu[f]), sd, cd);
                const float ur = kr * cd + ki * sd, ui = ki * cd - kr * sd;
                const float *c = pw + f * 3 * G;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    acc[h] = fmaf(c[h], ur, acc[h]);
                    acc[h] = fmaf(c[G + h], ui, acc[h]);
                    acc[h] = fmaf(c[2 * G + h], mag, acc[h]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float v = acc[h];
            raw[((size_t)sid * G + h) * N + j0 + jj] = v;
            const double dv = (double)v;
            m[h].s1 += dv;
            m[h].s2 = fma(dv, dv, m[h].s2);
            m[h].mn = fminf(m[h].mn, v);
            m[h].mx = fmaxf(m[h].mx, v);
        }
    }
    // block sums in a fixed order: lane butterfly, then the 4 waves in order
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        KSums v = m[h];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            v.s1 += __shfl_xor(v.s1, o, 64);
            v.s2 += __shfl_xor(v.s2, o, 64);
            v.mn = fminf(v.mn, __shfl_xor(v.mn, o, 64));
            v.mx = fmaxf(v.mx, __shfl_xor(v.mx, o, 64));
        }
        if (lane == 0) red[wid][h] = v;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        KSums v = red[0][h];
        for (int w = 1; w < kScoreThreads / 64; ++w) {
            v.s1 += red[w][h].s1;
            v.s2 += red[w][h].s2;
            v.mn = fminf(v.mn, red[w][h].mn);
            v.mx = fmaxf(v.mx, red[w][h].mx);
        }
        double *q = part + (((size_t)sid * tiles + tile) * G + h) * 4;
        q[0] = v.s1;
        q[1] = v.s2;
        q[2] = (double)v.mn;
        q[3] = (double)v.mx;
    }
}

template <int G, bool BF16, bool PRE_ROPE>
static hipError_t launch_perkey_t(const tria_calib *c, const void *k, const int32_t *pos, const int32_t *t,
                                  int n_seq, int N, float *raw, double *part, hipStream_t st)
{
    const int streams = n_seq * c->L * c->Hkv;
    const int tiles = (N + kTileKeys - 1) / kTileKeys;
    const long long blocks = (long long)streams * tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    score_perkey_tile_kernel<G, BF16, PRE_ROPE><<<(unsigned)blocks, kScoreThreads, 0, st>>>(
        k, pos, t, c->PW, c->nu, c->L, c->Hkv, N, tiles, raw, part);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_perkey_g(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                                  const int32_t *t, int n_seq, int N, bool pre_rope, float *raw, double *part,
                                  hipStream_t st)
{
    if (dt == TRIA_BF16)
        return pre_rope ? launch_perkey_t<G, true, true>(c, k, pos, t, n_seq, N, raw, part, st)
                        : launch_perkey_t<G, true, false>(c, k, pos, t, n_seq, N, raw, part, st);
    return pre_rope ? launch_perkey_t<G, false, true>(c, k, pos, t, n_seq, N, raw, part, st)
                    : launch_perkey_t<G, false, false>(c, k, pos, t, n_seq, N, raw, part, st);
}

hipError_t launch_score_perkey(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                               const int32_t *t, int n_seq, int N, unsigned flags, float *F, float *raw_out,
                               float *stats, const tria_score_ws &lay, char *ws, hipStream_t st)
{
    const bool pre_rope = (flags & TRIA_KEYS_PRE_ROPE) != 0;
    if (!lay.has_raw) return hipErrorInvalidValue;   // the layout did not plan this path
    float *raw = raw_out ? raw_out : (float *)(ws + lay.raw_off);
    double *part = (double *)(ws + lay.part_off);
    hipError_t e = hipSuccess;
    {
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        switch (c->G) {
        case 1: e = launch_perkey_g<1>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 2: e = launch_perkey_g<2>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 3: e = launch_perkey_g<3>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 4: e = launch_perkey_g<4>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 5: e = launch_perkey_g<5>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 6: e = launch_perkey_g<6>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 7: e = launch_perkey_g<7>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        case 8: e = launch_perkey_g<8>(c, dt, k, pos, t, n_seq, N, pre_rope, raw, part, st); break;
        default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    // statistics around 0 (no pivot) and the z-max of the matrix-core tiled path
    return launch_tile_finish(c->G, n_seq * c->L * c->Hkv, N, lay.tiles, raw, part, nullptr, F, stats, lay, ws, st);
}

}  // namespace tria
