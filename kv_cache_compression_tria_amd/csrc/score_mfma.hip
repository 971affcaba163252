// score_mfma.hip -- key scoring of bf16 caches on the matrix cores (gfx950, wave64).
//
// For one stream the G raw scores of key j are (see score.hip for the derivation)
//     s_h(j) = sum_d Qrot_h[d] * ktilde_j[d]  +  sum_f W_h[f] * |ktilde_{j,f}|
// i.e. a [G x 128] x [128 x keys] product plus a [G x 64] x [64 x keys] product with the band
// norms: a dense contraction with a skinny left-hand side.  It runs on v_mfma_f32_16x16x32_bf16
// (16 channels x 16 keys x 32-deep per instruction):
//   * A = the per-stream constants Qrot_h and W_h, each split into two bf16 terms
//     c = c0 + c1 (c0 = bf16(c), c1 = bf16(c - c0); |c - c0 - c1| <= 2^-18 |c|).  Term b of head h
//     is channel 8b + h (heads h >= G are zero rows);
//   * B = the cached bf16 key rows, used as loaded (exact), and the band norms |k_f| computed in
//     fp32 on the vector ALU and split the same way; of the four products of the two norm terms
//     with the two weight terms, the one of the two second terms (below 2^-16 relative) is
//     dropped.  Accumulation is fp32.
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, element e < 8, r < 4):
//   A: row l%16, k = 8*(l/16) + e;  B: k = 8*(l/16) + e, column l%16;  D: row 4*(l/16) + r, column l%16.
// Lane l of a wave loads 16 bytes at byte offset 64*kb + 16*(l/16) (kb < 4) of key row l%16 of a
// 16-key tile: the four loads give MFMA kb its B operand (dims 32kb + 8(l/16) + e), and the lane
// then holds, for its 16 bands 8(l/16)+e and 32+8(l/16)+e, both halves (re = dim f, im = dim
// f+64) of every band: the band norms need no cross-lane exchange.
// The two terms of a head sit in lanes l and l + 32 (channels 8b + h); one v_permlane32_swap per
// pair of accumulator registers brings them together, after which lane (g, j) = (l/16, l%16)
// owns the finished scores of key j for heads hA(g) = 4(g&1) + (g>>1) and hA(g) + 2.
//
// The per-stream A operands are built once per call by prologue_kernel in exactly this lane
// layout (one coalesced 16-byte load per lane per MFMA in the scoring kernels), together with a
// per-head pivot P_h (the fp32 score of the stream's first key; any value near the mean would do).
// Per-head moments are plain fp64 sums of (s - P_h) and (s - P_h)^2, merged by additions in a
// fixed order at every level (lane -> wave -> block -> stream): deterministic, no divisions, and
// no cancellation since P_h lies within the spread of the scores.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "common.cuh"
#include "tria_internal.h"

namespace tria {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kOps = 8;     // A operands per stream: 4 trig K-blocks, 2 norm terms x 2 band halves

int mfma_ops_per_stream(int) { return kOps; }

// the first of the two heads owned by lanes of row group g after the combine
__device__ __forceinline__ int head_a(int g) { return 4 * (g & 1) + (g >> 1); }

// term b (0 or 1) of the bf16 expansion of x
__device__ __forceinline__ float bf16_term(float x, int b)
{
    const float t0 = (float)(__bf16)x;
    return b == 0 ? t0 : (float)(__bf16)(x - t0);
}

// ---- prologue: rotated queries -> per-stream A operands (lane layout) and pivots -------------
// One wave per stream (s, l, g).  Lane f rotates band f of the group's G query heads to the
// sequence's position: Q_f = P_f exp(i w_f t) with the exact turn fraction t w_f / 2pi mod 1
// (64-bit integer product) and fp64 sin/cos, P_f = qbar_f mean_d exp(i w_f d) from the
// calibration table, optionally weighted by R_f (the R-weighted form); the G rotated queries stay
// in LDS.  Each lane then builds its operand words: ops[(sid*kOps + i)*64 + lane] is the operand of
// MFMA i (i < 4: trig K-block i; 4 + 2a + half: norm term a, band half).  The pivot of head h (the
// fp32 score of the stream's first key) is a butterfly sum of the lanes' band terms (every lane
// ends with the same bits).  Block 0 clears the error word and the blocks clear the stream
// clusters' n_arrive arrival words.  ROT (pre-RoPE keys): the pivot's key is first turned to its
// position (band f times exp(i w_f p), exact turn fraction, fp64 sincos).
template <int G, bool ROT>
__global__ __launch_bounds__(64) void prologue_kernel(const u32x4 *__restrict__ k, const double2 *__restrict__ P,
                                                      const uint64_t *__restrict__ nu, const int32_t *__restrict__ t,
                                                      const int32_t *__restrict__ pos,
                                                      const float *__restrict__ R, const float *__restrict__ W, int L,
                                                      int Hkv, int N, u32x4 *__restrict__ ops, float *__restrict__ pivot,
                                                      int *__restrict__ err, uint32_t *__restrict__ arrive, int n_arrive)
{
    __shared__ float q[G][TRIA_D];
    const int sid = blockIdx.x;
    const int lane = threadIdx.x;
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    const int s = sid / (Hkv * L);
    if (sid == 0 && lane == 0) *err = 0;   // this call's flag (no memset node: safe under graph capture)
    for (int i = sid * 64 + lane; i < n_arrive; i += gridDim.x * 64) arrive[i] = 0u;
    const size_t hh0 = ((size_t)l * Hkv + g) * G;   // (layer, first query head of the group)
    {
        const int f = lane;
        const uint64_t turns = (uint64_t)(int64_t)t[s] * nu[f];    // t * w_f / 2pi mod 1, exact
        double sn, cs;
        sincospi(2.0 * ((double)(int64_t)turns * 0x1p-64), &sn, &cs);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const double2 pf = P[(hh0 + h) * TRIA_HALF + f];
            const double wr = R ? (double)R[(hh0 + h) * TRIA_HALF + f] : 1.0;
            q[h][f] = (float)(wr * (pf.x * cs - pf.y * sn));
            q[h][TRIA_HALF + f] = (float)(wr * (pf.x * sn + pf.y * cs));
        }
    }
    __syncthreads();
    const float *wrow = W + hh0 * TRIA_HALF;
    const int j = lane & 15, grp = lane >> 4;
    const int b = j >> 3, h = j & 7;
    const bool live = h < G;
    const int hq = live ? h : 0;
    u32x4 *o = ops + (size_t)sid * kOps * 64 + lane;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)bf16_term(live ? q[hq][32 * kb + 8 * grp + e] : 0.f, b);
        o[kb * 64] = __builtin_bit_cast(u32x4, v);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (__bf16)bf16_term((live && a + b < 2) ? wrow[hq * TRIA_HALF + 32 * half + 8 * grp + e] : 0.f, b);
            o[(4 + 2 * a + half) * 64] = __builtin_bit_cast(u32x4, v);
        }
    // pivots: lane f holds band f of the stream's first key
    const uint16_t *row = (const uint16_t *)(k + (size_t)sid * N * 16);
    float re = __uint_as_float((uint32_t)row[lane] << 16), im = __uint_as_float((uint32_t)row[TRIA_HALF + lane] << 16);
    const float nrm = sqrtf(re * re + im * im);
    if (ROT) {
        const uint64_t turns = (uint64_t)(int64_t)pos[(size_t)sid * N] * nu[lane];
        double sn, cs;
        sincospi(2.0 * ((double)(int64_t)turns * 0x1p-64), &sn, &cs);
        const float r2 = (float)(re * cs - im * sn), i2 = (float)(re * sn + im * cs);
        re = r2;
        im = i2;
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float x = fmaf(q[hh][lane], re, fmaf(q[hh][TRIA_HALF + lane], im, wrow[hh * TRIA_HALF + lane] * nrm));
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) x += __shfl_xor(x, o2, 64);
        if (lane == hh) pivot[(size_t)sid * G + hh] = isfinite(x) ? x : 0.f;
    }
}

template <int G>
static hipError_t launch_prologue(const tria_calib *c, const u32x4 *kp, const int32_t *t, const int32_t *pos, int n_seq,
                                  int N, bool weight_r, u32x4 *ops, float *pivot, int *err, uint32_t *arrive,
                                  int n_arrive, hipStream_t st)
{
    const int streams = n_seq * c->L * c->Hkv;
    if (pos)
        prologue_kernel<G, true><<<streams, 64, 0, st>>>(kp, c->P, c->nu, t, pos, weight_r ? c->R : nullptr, c->W,
                                                         c->L, c->Hkv, N, ops, pivot, err, arrive, n_arrive);
    else
        prologue_kernel<G, false><<<streams, 64, 0, st>>>(kp, c->P, c->nu, t, nullptr, weight_r ? c->R : nullptr, c->W,
                                                          c->L, c->Hkv, N, ops, pivot, err, arrive, n_arrive);
    return hipGetLastError();
}

struct Ops {
    bf16x8 at[4];       // trig part, K-block kb: dims 32kb + 8g + e
    bf16x8 an[2][2];    // norm part, norm term a, band half: bands 32*half + 8g + e
};

__device__ __forceinline__ void load_ops(Ops &c, const u32x4 *__restrict__ ops_stream)
{
    const int lane = threadIdx.x & 63;
    const u32x4 *o = ops_stream + lane;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) c.at[kb] = __builtin_bit_cast(bf16x8, o[kb * 64]);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int half = 0; half < 2; ++half) c.an[a][half] = __builtin_bit_cast(bf16x8, o[(4 + 2 * a + half) * 64]);
}

// Load this lane's 64 bytes of a 16-key tile.  Rows at or past `valid` re-read row 0 of the tile
// (always a real row): their output columns are discarded, and keeping the load unconditional
// keeps the wait counts of the software pipeline exact.
__device__ __forceinline__ void load_tile(u32x4 (&ka)[4], const u32x4 *__restrict__ tile_base, int valid)
{
    const int lane = threadIdx.x & 63;
    const int row = (lane & 15) < valid ? (lane & 15) : 0, g = lane >> 4;
    const u32x4 *p = tile_base + row * 16 + g;   // row = 16 x 16 B; byte 64kb + 16g = word 4kb + g
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) ka[kb] = p[4 * kb];
}

// v_permlane32_swap: lanes 32..63 of x trade places with lanes 0..31 of y, so that afterwards
// x = (x[0..31], y[0..31]) and y = (x[32..63], y[32..63]).  Through the compiler builtin, so that
// the wait states after the matrix-core instruction that produced x and y (its result is not
// interlocked for this read) are inserted by the compiler's hazard recognizer.
__device__ __forceinline__ void permlane32_swap(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                    false, false);
    x = __builtin_bit_cast(float, (uint32_t)r[0]);
    y = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// re^2 + im^2 of a band held as a bf16 pair (re, im) in fp32 (v_dot2: products exact, one
// rounding)
__device__ __forceinline__ float band_sq(uint32_t pair)
{
    const bf16x2 p = __builtin_bit_cast(bf16x2, pair);
    return __builtin_amdgcn_fdot2_f32_bf16(p, p, 0.f, false);
}

// Two-term bf16 split of a pair of fp32 values: hi = the pair rounded to bf16 (one packed
// conversion), lo = the rounding errors x - hi, rounded to bf16 in turn (x = hi + lo to 2^-18 |x|).
// x - bf16(x) is exact in fp32, so v_dot2 of the packed hi with (-1, 0) or (0, -1), added to x,
// forms it with one rounding of an exact value: one instruction in place of the unpacking shift
// or mask and the subtraction.  The (-1, 0) pair is held in a scalar register: written as a
// constant, the compiler encodes it as the inline constant -1.0, which the hardware reads for this
// operand as the fp32 pattern 0xbf800000, i.e. (0, -1).  The (0, -1) pair is that literal.
struct Split2 {
    uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split2(float x0, float x1)
{
    uint32_t neg_lo;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(neg_lo));
    const bf16x2 h = __builtin_convertvector(float2v{x0, x1}, bf16x2);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg_lo), x0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, 0xbf800000u), x1, false);
    return {__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{r0, r1}, bf16x2))};
}

// Band-norm contraction of one 16-key tile into acc: bands 8g+e (re in ka[0], im in ka[2]) and
// 32+8g+e (re in ka[1], im in ka[3]); v_perm pairs (re, im) of a band, v_dot2 forms re^2 + im^2
// from the bf16 halves in fp32, and the two-term split of a pair of norms costs two packed
// conversions and two v_dot2.
__device__ __forceinline__ floatx4 norm_tile16(const u32x4 (&ka)[4], const Ops &c, floatx4 acc)
{
    u32x4 t0[2], t1[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const u32x4 x = ka[half], y = ka[2 + half];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t p0 = __builtin_amdgcn_perm(y[i], x[i], 0x05040100u);
            const uint32_t p1 = __builtin_amdgcn_perm(y[i], x[i], 0x07060302u);
            const Split2 n = split2(__builtin_amdgcn_sqrtf(band_sq(p0)), __builtin_amdgcn_sqrtf(band_sq(p1)));
            t0[half][i] = n.hi;
            t1[half][i] = n.lo;
        }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[0][half], __builtin_bit_cast(bf16x8, t0[half]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[1][half], __builtin_bit_cast(bf16x8, t1[half]), acc, 0, 0, 0);
    }
    return acc;
}

// lanes l < 32 hold term 0 of channels 4g + r, lanes l + 32 term 1 of the same heads: one swap per
// pair of accumulator registers adds them up
__device__ __forceinline__ void combine_terms(floatx4 acc, float (&v)[2])
{
    float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
    permlane32_swap(a0, a1);
    permlane32_swap(a2, a3);
    v[0] = a0 + a1;
    v[1] = a2 + a3;
}

// Scores of one 16-key tile: lane (g, j) returns v[0], v[1] = heads head_a(g), head_a(g) + 2 of
// key j (zero for heads >= G).
__device__ __forceinline__ void score_tile16(const u32x4 (&ka)[4], const Ops &c, float (&v)[2])
{
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.at[kb], __builtin_bit_cast(bf16x8, ka[kb]), acc, 0, 0, 0);
    combine_terms(norm_tile16(ka, c, acc), v);
}

// The same for pre-RoPE keys, which lane (g, j) first turns to key j's position p (RoPE applied on
// the fly): band f (re = dim f, im = dim f + 64) times exp(i w_f p).  The angle in turns is the
// top 32 bits of p nu_f mod 2^64, exact for any 32-bit p from two 32-bit products: with
// nu_f = hi 2^32 + lo and lo read as a signed word s (lo = s + 2^32 [lo >= 2^31]), the top word is
// p (hi + [lo >= 2^31]) + mulhi_signed(p, s) mod 2^32; nu_l holds (s, hi + [lo >= 2^31]) per band.
// The hardware sine and cosine take the angle in turns; they get 1 + top / 2^32 with the fraction
// truncated to 23 bits (angle error below 2^-23 turns).  The turned key is no longer exact in
// bf16, so it enters as two bf16 terms (x = x0 + x1, |x - x0 - x1| <= 2^-18 |x|): eight
// trigonometric MFMAs instead of four.  The band norms do not change under the turn and come from
// the loaded key: re^2 + im^2 from the unpacked halves (one product and one fused multiply-add,
// exact products and one rounding, as v_dot2 forms it on the default path), in the same loop.
__device__ __forceinline__ void score_tile16_rot(const u32x4 (&ka)[4], const Ops &c, int32_t p,
                                                 const int2 *__restrict__ nu_l, float (&v)[2])
{
    const int grp = (threadIdx.x & 63) >> 4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const u32x4 x = ka[half], y = ka[2 + half];
        u32x4 rh, rl, ih, il, nh, nl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = 32 * half + 8 * grp + 2 * i;
            const int4 nn = *(const int4 *)&nu_l[f];     // bands f and f + 1
            const float re[2] = {__uint_as_float(x[i] << 16), __uint_as_float(x[i] & 0xffff0000u)};
            const float im[2] = {__uint_as_float(y[i] << 16), __uint_as_float(y[i] & 0xffff0000u)};
            float r[2], q[2], nrm[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int s_lo = e ? nn.z : nn.x, hi = e ? nn.w : nn.y;
                const uint32_t top = (uint32_t)p * (uint32_t)hi + (uint32_t)__mulhi(p, s_lo);
                // 1 + top / 2^32 built from the bits (v_alignbit: 0x3f800000 | top >> 9): the
                // same angle modulo one turn, its fraction truncated to 23 bits
                const float a = __uint_as_float(__builtin_amdgcn_alignbit(0x7fu, top, 9));
                const float sn = __builtin_amdgcn_sinf(a), cs = __builtin_amdgcn_cosf(a);
                r[e] = fmaf(re[e], cs, -im[e] * sn);
                q[e] = fmaf(re[e], sn, im[e] * cs);
                nrm[e] = __builtin_amdgcn_sqrtf(fmaf(re[e], re[e], im[e] * im[e]));
            }
            const Split2 sr = split2(r[0], r[1]), sq = split2(q[0], q[1]), sn = split2(nrm[0], nrm[1]);
            rh[i] = sr.hi;
            rl[i] = sr.lo;
            ih[i] = sq.hi;
            il[i] = sq.lo;
            nh[i] = sn.hi;
            nl[i] = sn.lo;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.at[half], __builtin_bit_cast(bf16x8, rh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.at[half], __builtin_bit_cast(bf16x8, rl), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.at[2 + half], __builtin_bit_cast(bf16x8, ih), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.at[2 + half], __builtin_bit_cast(bf16x8, il), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[0][half], __builtin_bit_cast(bf16x8, nh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[1][half], __builtin_bit_cast(bf16x8, nl), acc, 0, 0, 0);
    }
    combine_terms(acc, v);
}

// Moments of one head around the stream pivot P: S1 = sum (v - P), S2 = sum (v - P)^2 (fp64),
// min, max.  Merging two is an addition; the count is known from the key ranges.  A non-finite
// score makes S1 or S2 non-finite.
struct Sums {
    double s1, s2;
    float mn, mx;
    __device__ void init() { s1 = 0.0; s2 = 0.0; mn = INFINITY; mx = -INFINITY; }
    __device__ void add(float v, float p)
    {
        const double d = (double)(v - p);
        s1 += d;
        s2 = fma(d, d, s2);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    __device__ void add(const Sums &o)
    {
        s1 += o.s1;
        s2 += o.s2;
        mn = fminf(mn, o.mn);
        mx = fmaxf(mx, o.mx);
    }
};

// Sum over the 16 lanes of a wave row (same l/16), fixed butterfly order: every lane of the row
// ends with the same bits (IEEE addition is commutative).
__device__ __forceinline__ void row16_sum(Sums &m)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        Sums t;
        t.s1 = __shfl_xor(m.s1, o, 64);
        t.s2 = __shfl_xor(m.s2, o, 64);
        t.mn = __shfl_xor(m.mn, o, 64);
        t.mx = __shfl_xor(m.mx, o, 64);
        m.add(t);
    }
}

// A head whose scores span at most 2^-16 of their largest magnitude is constant (scores equal up
// to rounding): std := 0, z := 0.
__device__ __forceinline__ bool flat_head_m(double mn, double mx)
{
    return (mx - mn) <= ldexp(fmax(fabs(mn), fabs(mx)), -16);
}

// mean and (population) std of n values from their sums around p
__device__ __forceinline__ void finish_moments(const Sums &m, double p, double n, double &mean, double &sd)
{
    mean = p + m.s1 / n;
    const double m2 = fmax(m.s2 - m.s1 * (m.s1 / n), 0.0);
    sd = flat_head_m((double)m.mn, (double)m.mx) ? 0.0 : sqrt(m2 / n);
}

// Per-block reduction of the lane sums: waves publish their 16-lane row sums to LDS, thread h
// (< G) adds the NW waves in order.
template <int NW>
struct BlockSumsT {
    double s1[NW][8], s2[NW][8];
    float mn[NW][8], mx[NW][8];
};
using BlockSums = BlockSumsT<4>;

template <int NW>
__device__ __forceinline__ void block_sums_stage(BlockSumsT<NW> &bs, Sums (&m)[2])
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        row16_sum(m[s]);
        const int h = head_a(g) + 2 * s;
        if (j == 0) {
            bs.s1[wid][h] = m[s].s1;
            bs.s2[wid][h] = m[s].s2;
            bs.mn[wid][h] = m[s].mn;
            bs.mx[wid][h] = m[s].mx;
        }
    }
}

template <int NW>
__device__ __forceinline__ Sums block_sums_of(const BlockSumsT<NW> &bs, int h)
{
    Sums t;
    t.init();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        Sums u;
        u.s1 = bs.s1[w][h]; u.s2 = bs.s2[w][h]; u.mn = bs.mn[w][h]; u.mx = bs.mx[w][h];
        t.add(u);
    }
    return t;
}

// Everything one wave needs to score 16-key tiles of a stream: operands, pivots of its two heads
// and running sums.
template <int G>
struct WaveScorer {
    Ops c;
    float p[2];
    Sums m[2];

    __device__ void begin(const u32x4 *__restrict__ ops, const float *__restrict__ pivot, int sid)
    {
        load_ops(c, ops + (size_t)sid * kOps * 64);
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int h = head_a(g) + 2 * s;
            p[s] = pivot[(size_t)sid * G + (h < G ? h : 0)];
            m[s].init();
        }
    }
    // the same from an LDS copy of the stream's operand words and pivots
    __device__ void begin_lds(const u32x4 *ops_l, const float *piv_l)
    {
        load_ops(c, ops_l);
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int h = head_a(g) + 2 * s;
            p[s] = piv_l[h < G ? h : 0];
            m[s].init();
        }
    }
    // score a tile; v[s] = score of key (tile row l%16) for head head_a(g) + 2s.  Rows >= nvalid
    // and heads >= G enter the sums as the pivot itself (no change to the sums; the pivot is the
    // score of key 0, so min and max keep their values): no branches in the key loop.
    __device__ void score(const u32x4 (&b)[4], int nvalid, float (&v)[2])
    {
        score_tile16(b, c, v);
        add(nvalid, v);
    }
    // the same for a tile of pre-RoPE keys, turned to their positions (lane's key at position p)
    __device__ void score_rot(const u32x4 (&b)[4], int32_t p, const int2 *nu_l, int nvalid, float (&v)[2])
    {
        score_tile16_rot(b, c, p, nu_l, v);
        add(nvalid, v);
    }
    __device__ __forceinline__ void add(int nvalid, const float (&v)[2])
    {
        const int lane = threadIdx.x & 63;
        const int j = lane & 15, ha = head_a(lane >> 4);
        const bool ok = j < nvalid;
        m[0].add((ok && ha < G) ? v[0] : p[0], p[0]);
        m[1].add((ok && ha + 2 < G) ? v[1] : p[1], p[1]);
    }
};

// Four-deep ring of tile registers, straight-line: item i of a wave lives in buffer i % 4 and is
// loaded three items ahead of its use.  issue(b, i) loads item i; compute(b, i) scores it.  The
// item count is rounded up to a multiple of four so that the loop body has no exits: items past
// the end re-read a real tile and are scored as empty (no valid rows).  With no branch between a
// load and its use the compiler cannot sink the loads next to their uses; TRIA_PIN (a scheduling
// barrier, no instruction) keeps the machine scheduler from regrouping them.
#define TRIA_PIN() __builtin_amdgcn_sched_barrier(0)
#define TRIA_RING4(nt, issue, compute)                                                         \
    do {                                                                                       \
        u32x4 b0_[4], b1_[4], b2_[4], b3_[4];                                                  \
        const int n4_ = ((nt) + 3) & ~3;                                                       \
        issue(b0_, 0);                                                                         \
        TRIA_PIN();                                                                            \
        issue(b1_, 1);                                                                         \
        TRIA_PIN();                                                                            \
        issue(b2_, 2);                                                                         \
        TRIA_PIN();                                                                            \
        for (int i_ = 0; i_ < n4_; i_ += 4) {                                                  \
            issue(b3_, i_ + 3);                                                                \
            TRIA_PIN();                                                                        \
            compute(b0_, i_);                                                                  \
            issue(b0_, i_ + 4);                                                                \
            TRIA_PIN();                                                                        \
            compute(b1_, i_ + 1);                                                              \
            issue(b1_, i_ + 5);                                                                \
            TRIA_PIN();                                                                        \
            compute(b2_, i_ + 2);                                                              \
            issue(b2_, i_ + 6);                                                                \
            TRIA_PIN();                                                                        \
            compute(b3_, i_ + 3);                                                              \
        }                                                                                      \
    } while (0)

// ---- tiled path: block = (stream, 1024-key tile); raw scores head-major through global memory --
// raw [streams][G][N] (the workspace, or the caller's raw output directly); partial sums per
// (stream, tile, head): s1, s2, min, max.

template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_tile_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ ops, const float *__restrict__ pivot, int N, int tiles,
    float *__restrict__ raw, double *__restrict__ part)
{
    __shared__ BlockSums bs;
    const int sid = blockIdx.x / tiles;
    const int tile = blockIdx.x - sid * tiles;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar loop control
    const int jj = lane & 15, ha = head_a(lane >> 4);

    WaveScorer<G> ws;
    ws.begin(ops, pivot, sid);

    const int j0 = tile * kTileKeys;
    const int nkeys = min(kTileKeys, N - j0);
    const int ntiles16 = (nkeys + 15) >> 4;
    const u32x4 *kb = k + ((size_t)sid * N + j0) * 16;
    const int nt_w = wid < ntiles16 ? (ntiles16 - wid + 3) >> 2 : 0;
    // Raw scores go out as they are made, through a buffer resource over this block's part of
    // the stream's rows: a store with an offset past the range (rows past the end of the tile,
    // heads >= G) is dropped by the hardware, so every ring step issues the same two stores and
    // the waits of the ring stay exact.  Each store writes 16 consecutive keys of 4 heads.
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        raw + (size_t)sid * G * N + j0, 0, ((G - 1) * N + nkeys) * 4, 0x00020000);
    constexpr int kDrop = 0x7fffffff;
    // item i of this wave is tile wid + 4i
    auto issue = [&](u32x4 (&b)[4], int i) {
        const int t = min(wid + 4 * i, ntiles16 - 1);
        load_tile(b, kb + (size_t)t * 16 * 16, nkeys - t * 16);
    };
    auto compute = [&](const u32x4 (&b)[4], int i) {
        const int t = wid + 4 * i;
        float v[2];
        ws.score(b, nkeys - t * 16, v);
        const int key = t * 16 + jj;
        const bool in = key < nkeys;
        const int o0 = (in && ha < G) ? (ha * N + key) * 4 : kDrop;
        const int o1 = (in && ha + 2 < G) ? ((ha + 2) * N + key) * 4 : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[0]), rsrc, o0, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[1]), rsrc, o1, 0, 0);
    };
    if (nt_w > 0) TRIA_RING4(nt_w, issue, compute);
    block_sums_stage(bs, ws.m);
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const Sums t2 = block_sums_of(bs, h);
        double *q = part + (((size_t)sid * tiles + tile) * G + h) * 4;
        q[0] = t2.s1;
        q[1] = t2.s2;
        q[2] = (double)t2.mn;
        q[3] = (double)t2.mx;
    }
}

// Per-stream statistics of the tiled path: one block per stream adds the tile partials of each
// head (wave w takes heads w and w + 4; lane l the tiles l, l + 64, ... in order, then a fixed
// butterfly) and publishes mean and 1/std per head (zst) and the optional head statistics.
template <int G>
__global__ __launch_bounds__(kScoreThreads) void tile_stats_kernel(const double *__restrict__ part,
                                                                   const float *__restrict__ pivot, int N, int tiles,
                                                                   float *__restrict__ zst, float *__restrict__ stats,
                                                                   int *__restrict__ err)
{
    const int sid = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int h = wid + 4 * s;
        if (h >= G) break;
        Sums t2;
        t2.init();
        for (int tt = lane; tt < tiles; tt += 64) {
            const double *q = part + (((size_t)sid * tiles + tt) * G + h) * 4;
            Sums u;
            u.s1 = q[0]; u.s2 = q[1]; u.mn = (float)q[2]; u.mx = (float)q[3];
            t2.add(u);
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            Sums u;
            u.s1 = __shfl_xor(t2.s1, o, 64);
            u.s2 = __shfl_xor(t2.s2, o, 64);
            u.mn = __shfl_xor(t2.mn, o, 64);
            u.mx = __shfl_xor(t2.mx, o, 64);
            t2.add(u);
        }
        if (lane == 0) {
            if (!isfinite(t2.s1) || !isfinite(t2.s2)) atomicOr(err, 1);
            double mean, sd;
            finish_moments(t2, pivot ? (double)pivot[(size_t)sid * G + h] : 0.0, (double)N, mean, sd);
            zst[((size_t)sid * G + h) * 2 + 0] = (float)mean;
            zst[((size_t)sid * G + h) * 2 + 1] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
            if (stats) {
                stats[((size_t)sid * G + h) * 2 + 0] = (float)mean;
                stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
            }
        }
    }
}

// Final scores of the tiled path: F(j) = max_h (raw_h(j) - mean_h) / std_h over the head-major
// raw rows; one block per (stream, 4096 keys), four keys per thread and step.
constexpr int kZmaxKeys = 4096;

template <int G>
__global__ __launch_bounds__(kScoreThreads) void zmax_tiles_kernel(const float *__restrict__ raw,
                                                                   const float *__restrict__ zst, int N, int chunks,
                                                                   float *__restrict__ F)
{
    const int sid = blockIdx.x / chunks;
    const int c = blockIdx.x - sid * chunks;
    float mu[G], inv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mu[h] = zst[((size_t)sid * G + h) * 2 + 0];
        inv[h] = zst[((size_t)sid * G + h) * 2 + 1];
    }
    const int j0 = c * kZmaxKeys;
    const int nk = min(kZmaxKeys, N - j0);
    const float *r = raw + (size_t)sid * G * N + j0;
    float *fo = F + (size_t)sid * N + j0;
    if ((N & 3) == 0 && ((uintptr_t)raw & 15) == 0 && ((uintptr_t)F & 15) == 0) {
        for (int q = threadIdx.x; q < (nk >> 2); q += kScoreThreads) {
            float4 z = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float4 x = *(const float4 *)(r + (size_t)h * N + 4 * q);
                z.x = fmaxf(z.x, (x.x - mu[h]) * inv[h]);
                z.y = fmaxf(z.y, (x.y - mu[h]) * inv[h]);
                z.z = fmaxf(z.z, (x.z - mu[h]) * inv[h]);
                z.w = fmaxf(z.w, (x.w - mu[h]) * inv[h]);
            }
            *(float4 *)(fo + 4 * q) = z;
        }
    } else {
        for (int j = threadIdx.x; j < nk; j += kScoreThreads) {
            float z = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h) z = fmaxf(z, (r[(size_t)h * N + j] - mu[h]) * inv[h]);
            fo[j] = z;
        }
    }
}

// ---- fused path: one block per stream, raw scores kept in LDS ---------------------------------
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_mfma_fused_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ ops, const float *__restrict__ pivot, int N,
    float *__restrict__ F, float *__restrict__ raw_out, float *__restrict__ stats, int *__restrict__ err)
{
    extern __shared__ float raw[];                 // [G][NP], NP = N | 1 (odd stride: no bank conflicts)
    const int NP = N | 1;
    __shared__ BlockSums bs;
    __shared__ float zmu[G], zinv[G];
    const int sid = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jj = lane & 15, ha = head_a(lane >> 4);

    WaveScorer<G> ws;
    ws.begin(ops, pivot, sid);

    const int ntiles16 = (N + 15) >> 4;
    const u32x4 *kb = k + (size_t)sid * N * 16;
    const int nt_w = wid < ntiles16 ? (ntiles16 - wid + 3) >> 2 : 0;
    auto issue = [&](u32x4 (&b)[4], int i) {
        const int t = min(wid + 4 * i, ntiles16 - 1);
        load_tile(b, kb + (size_t)t * 16 * 16, N - t * 16);
    };
    auto compute = [&](const u32x4 (&b)[4], int i) {
        const int t = wid + 4 * i;
        float v[2];
        ws.score(b, N - t * 16, v);
        const int key = t * 16 + jj;
        if (key < N) {
            if (ha < G) raw[ha * NP + key] = v[0];
            if (ha + 2 < G) raw[(ha + 2) * NP + key] = v[1];
        }
    };
    if (nt_w > 0) TRIA_RING4(nt_w, issue, compute);
    block_sums_stage(bs, ws.m);
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const Sums t2 = block_sums_of(bs, h);
        if (!isfinite(t2.s1) || !isfinite(t2.s2)) atomicOr(err, 1);
        double mean, sd;
        finish_moments(t2, (double)pivot[(size_t)sid * G + h], (double)N, mean, sd);
        zmu[h] = (float)mean;
        zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
        if (stats) {
            stats[((size_t)sid * G + h) * 2 + 0] = (float)mean;
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

// ---- cluster path: the raw scores of a stream stay on chip ----------------------------------
// A stream too long for one block's LDS is split over a cluster of Ps blocks (Ps a power of two),
// each keeping the raw scores of its Kb keys in LDS ([Kb][GP] floats, key-major, GP = G rounded up
// to even).  After scoring, every block publishes its per-head partial sums and moves on to the
// next stream; after the first four items of that stream (scores held in registers) it waits
// until the cluster's Ps partials of the previous round are there, adds them in part order (every
// block gets the same bits), and writes the final scores of its keys straight from LDS: the raw
// scores never travel through HBM, and the wait for the slowest block of the cluster is covered
// by scoring.  The grid is one block per CU, launched cooperatively so that all blocks are
// resident at once; a block loops over rounds, cluster c scoring streams c, c + C, c + 2C, ...
// The Ps blocks of a cluster sit on one XCD (workgroups are dealt to the 8 XCDs in turn).  The
// exchanged words are agent-scope atomics, coherent across the device without cache
// maintenance.  Partial sums are double-buffered by round parity: a block publishes round r + 2
// only after the whole cluster has published round r + 1, and every block has gathered round r
// before it publishes round r + 1.  The wait is bounded: past the bound the block sets bit 2 of
// the error flag and carries on (wrong scores, but no hang), and every other waiting block then
// stops at once.
constexpr int kClusterWaves = 8;
constexpr int kClusterDefer = 4;            // groups of four items scored before a round is finished
constexpr unsigned kSpinLimit = 1u << 20;   // polls of about a microsecond each

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void score_mfma_cluster_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ ops, const float *__restrict__ pivot, int N,
    int streams, int Ps, int Kb, int cpx, int C, double *__restrict__ xpart, uint32_t *__restrict__ arrive,
    float *__restrict__ F, float *__restrict__ samp, float *__restrict__ raw_out, float *__restrict__ stats,
    int *__restrict__ err)
{
    constexpr int GP = (G + 1) & ~1;
    extern __shared__ float lraw[];                // [Kb][GP]
    __shared__ BlockSumsT<NW> bs;
    __shared__ float zmu[8], zinv[8];
    __shared__ double xs[32 * 8 * 4];              // the cluster's partials of a round, gathered
    __shared__ u32x4 ops_l[kOps * 64];             // the next stream's operand words ...
    __shared__ float piv_l[8];                     // ... and pivots, fetched during a round
    static_assert(NW == kOps, "one operand word per thread");
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int cl = x * cpx + y / Ps, part = y % Ps;
    const int rounds = cl < streams ? (streams - cl + C - 1) / C : 0;
    if (rounds == 0) return;                       // the whole cluster has no stream
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jj = lane & 15, ha = head_a(lane >> 4);
    const int j0 = part * Kb;
    const int nkeys = max(0, min(Kb, N - j0));
    const int ntiles16 = (nkeys + 15) >> 4;
    // Every wave takes the same number of items per round, a multiple of four (empty items re-read
    // a real tile and score nothing), so that the four-deep ring runs on across rounds: the loads
    // of the next round's first tiles are in flight while a round ends (statistics, publication).
    const int nt = (max(1, (ntiles16 + NW - 1) / NW) + 3) & ~3;
    const int total = rounds * nt;

    WaveScorer<G> ws;
    ws.begin(ops, pivot, cl);
    auto issue = [&](u32x4 (&b)[4], int i) {
        const int ic = min(i, total - 1);
        const int r = ic / nt;
        const int sid = cl + r * C;
        const int t = min(wid + NW * (ic - r * nt), ntiles16 - 1);
        if (t >= 0)
            load_tile(b, k + ((size_t)sid * N + j0 + t * 16) * 16, nkeys - t * 16);
        else
            load_tile(b, k + (size_t)sid * N * 16, 0);   // a part with no keys: row 0, scored as empty
    };
    // raw scores of item li of this wave into LDS
    auto put = [&](int li, const float (&v)[2]) {
        const int key = (wid + NW * li) * 16 + jj;
        if (key < nkeys) {
            if (ha < GP) lraw[key * GP + ha] = v[0];
            if (ha + 2 < GP) lraw[key * GP + ha + 2] = v[1];
        }
    };
    auto compute = [&](const u32x4 (&b)[4], int li) {
        float v[2];
        ws.score(b, nkeys - (wid + NW * li) * 16, v);
        put(li, v);
    };
    // round r's partial sums: wave 0 of every block stores its per-head sums as agent-scope atomics
    // (coherent across the device without cache maintenance), waits for the stores, and counts its
    // arrival.  Nothing waits for the other blocks here.
    auto publish = [&](int r) {
        if (wid != 0) return;
        double *xr = xpart + ((size_t)cl * 2 + (r & 1)) * Ps * G * 4;
        if (lane < G) {
            const Sums t2 = block_sums_of(bs, lane);
            double *q = xr + ((size_t)part * G + lane) * 4;
            __hip_atomic_store(q + 0, t2.s1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(q + 1, t2.s2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(q + 2, (double)t2.mn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(q + 3, (double)t2.mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(&arrive[cl], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // round r's final scores: wave 0 waits (bounded) until the whole cluster has published round
    // r, fetches the Ps partials at once and lanes h < G add head h's in part order (every block
    // gets the same bits); then the block writes F for its keys straight from LDS.
    auto finish = [&](int r) {
        const int sid = cl + r * C;
        if (wid == 0) {
            const double *xr = xpart + ((size_t)cl * 2 + (r & 1)) * Ps * G * 4;
            if (lane == 0) {
                const uint32_t target = (uint32_t)(r + 1) * (uint32_t)Ps;
                unsigned spins = 0;
                while (__hip_atomic_load(&arrive[cl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                    // give up past the bound, or at once when another block already gave up
                    if (++spins > kSpinLimit ||
                        (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2)) {
                        atomicOr(err, 2);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
            for (int q = lane; q < Ps * G; q += 64) {
                const double *src = xr + (size_t)q * 4;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xs[q * 4 + c] = __hip_atomic_load(src + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_wave_barrier();
            if (lane < G) {
                const int h = lane;
                Sums t2;
                t2.init();
                for (int pp = 0; pp < Ps; ++pp) {
                    const double *q = xs + ((size_t)pp * G + h) * 4;
                    Sums u;
                    u.s1 = q[0]; u.s2 = q[1]; u.mn = (float)q[2]; u.mx = (float)q[3];
                    t2.add(u);
                }
                double mean, sd;
                finish_moments(t2, (double)pivot[(size_t)sid * G + h], (double)N, mean, sd);
                zmu[h] = (float)mean;
                zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
                if (part == 0) {
                    if (!isfinite(t2.s1) || !isfinite(t2.s2)) atomicOr(err, 1);
                    if (stats) {
                        stats[((size_t)sid * G + h) * 2 + 0] = (float)mean;
                        stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
                    }
                }
            }
        }
        __syncthreads();
        float *fo = F + (size_t)sid * N + j0;
        float *so = samp + (size_t)sid * ((N + kSampleStride - 1) / kSampleStride) + j0 / kSampleStride;
        for (int j = threadIdx.x; j < nkeys; j += NW * 64) {
            float z = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h) z = fmaxf(z, (lraw[j * GP + h] - zmu[h]) * zinv[h]);
            fo[j] = z;
            if (j % kSampleStride == 0) so[j / kSampleStride] = z;   // j0 is a multiple of the stride
        }
        if (raw_out)
            for (int q = threadIdx.x; q < G * nkeys; q += NW * 64) {
                const int h = q / nkeys, j = q - h * nkeys;
                raw_out[((size_t)sid * G + h) * N + j0 + j] = lraw[j * GP + h];
            }
        __syncthreads();                           // LDS raw and zmu are reused
    };
    u32x4 b0[4], b1[4], b2[4], b3[4];
    issue(b0, 0);
    TRIA_PIN();
    issue(b1, 1);
    TRIA_PIN();
    issue(b2, 2);
    TRIA_PIN();
    for (int r = 0; r < rounds; ++r) {
        int li = 0;
        if (r > 0) {
            // The first items of a round keep their scores in registers while the previous round
            // is finished: by then every block of the cluster has long published it, so the wait
            // for the slowest block is covered by scoring instead of idling.
            constexpr int D = 4 * kClusterDefer;
            const int nd = min(D, nt);
            float dv[D][2];
#pragma unroll
            for (int q0 = 0; q0 < D; q0 += 4) {
                if (q0 < nd) {
                    const int i = r * nt + q0;
                    issue(b3, i + 3);
                    TRIA_PIN();
                    ws.score(b0, nkeys - (wid + NW * q0) * 16, dv[q0]);
                    issue(b0, i + 4);
                    TRIA_PIN();
                    ws.score(b1, nkeys - (wid + NW * (q0 + 1)) * 16, dv[q0 + 1]);
                    issue(b1, i + 5);
                    TRIA_PIN();
                    ws.score(b2, nkeys - (wid + NW * (q0 + 2)) * 16, dv[q0 + 2]);
                    issue(b2, i + 6);
                    TRIA_PIN();
                    ws.score(b3, nkeys - (wid + NW * (q0 + 3)) * 16, dv[q0 + 3]);
                    TRIA_PIN();
                }
            }
            finish(r - 1);
#pragma unroll
            for (int q = 0; q < D; ++q)
                if (q < nd) put(q, dv[q]);
            li = nd;
        }
        // the next stream's operands and pivots: fetched now, into LDS at the end of the round
        const bool more = r + 1 < rounds;
        u32x4 nxt_op = {0u, 0u, 0u, 0u};
        float nxt_pv = 0.f;
        if (more) {
            const int sn = cl + (r + 1) * C;
            nxt_op = ops[(size_t)sn * kOps * 64 + threadIdx.x];
            if (threadIdx.x < G) nxt_pv = pivot[(size_t)sn * G + threadIdx.x];
        }
        TRIA_PIN();
        for (; li < nt; li += 4) {
            const int i = r * nt + li;
            issue(b3, i + 3);
            TRIA_PIN();
            compute(b0, li);
            issue(b0, i + 4);
            TRIA_PIN();
            compute(b1, li + 1);
            issue(b1, i + 5);
            TRIA_PIN();
            compute(b2, li + 2);
            issue(b2, i + 6);
            TRIA_PIN();
            compute(b3, li + 3);
            TRIA_PIN();
        }
        // ---- end of round r: stage and publish the partial sums, switch to the next stream
        block_sums_stage(bs, ws.m);
        if (more) {
            ops_l[threadIdx.x] = nxt_op;
            if (threadIdx.x < G) piv_l[threadIdx.x] = nxt_pv;
        }
        __syncthreads();
        publish(r);
        if (more) ws.begin_lds(ops_l, piv_l);
    }
    finish(rounds - 1);
}

// ---- staged cluster path: the keys reach LDS by direct memory-to-LDS loads -------------------
// The same stream clusters and on-chip raw scores as above, with the key tiles fetched by
// global_load_lds_dwordx4 with the non-temporal hint instead of into registers: each load
// instruction covers 1 KB of consecutive key bytes (four whole rows), which streams from HBM
// faster than the matrix-core operand layout does, and the operands are then read from LDS.  Chunk
// c of row r of a tile sits at slot 16 r + (c ^ r), so the operand reads (row j, chunk
// 4 kb + g for lane (g, j)) hit distinct bank groups.  Each wave owns two 4 KB slots: item i's
// tile is read out of its slot into registers first, and the slot is then refilled with the tile
// of item i + 2, so the tiles of items i + 1 and i + 2 are in flight while item i is scored.  The
// compiler does not see these loads, so the kernel waits for them itself: vmcnt counts vector
// memory operations in issue order, every other such operation of the loop is written out and
// issued right after a tile load, and the next wait leaves exactly those outstanding.  The raw
// scores of a round take at most 64 KB of LDS (2048 keys at G = 8), so a stream of 32768 keys
// spans a cluster of 16 blocks.  The exchange of a round: wave 0 stores the block's partial sums
// after the next round's first tile load and sets the block's arrival flag after the third (a
// flag per block written by a plain store; an atomic counter completes late and holds up the
// wave's later waits), fetches the cluster's flags and partials into LDS during the deferred
// items, and stamps the heads' mean and 1/std in LDS; each wave then writes F for its own keys.
constexpr int kStageLds = 64 * 1024;   // raw scores of one block's part of a stream
constexpr int kStageDefer = 16;        // items scored before the previous round is finished
// During the deferred items wave 0 fetches the cluster's arrival flags (item kStageFlags) and, if
// every block has arrived, its partial sums (item kStageFlags + 2) into LDS; at the finish, after a
// ring wait that the last deferred item's tile load makes exact, it turns them into the mean and
// 1/std of every head, so that the finish does not wait for the cluster.
constexpr int kStageFlags = 12;

// one 16-byte-per-lane memory-to-LDS load: lane l's 16 bytes at `src` land at lds_base + 16 l
__device__ __forceinline__ void dma16(const u32x4 *src, const u32x4 *lds_base)
{
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(la)
                 : "memory", "m0");
}

// Items per wave and round of a block that holds kStageLds bytes of raw scores (a full block).
template <int G>
constexpr int stage_full_items()
{
    constexpr int GP = (G + 1) & ~1;
    constexpr int kmax = (kStageLds / (GP * 4)) & ~15;
    return ((kmax + 15) / 16 + kClusterWaves - 1) / kClusterWaves;
}

// one 4-byte-per-lane memory-to-LDS load: lane l's word at `src` lands at lds_base + 4 l
__device__ __forceinline__ void dma4(const int32_t *src, const int32_t *lds_base)
{
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(src), "s"(la)
                 : "memory", "m0");
}

// NTC > 0: every block of the launch runs exactly NTC items per wave and round (known at compile
// time, so that the item and round indices are shifts and masks, not divisions); 0: any count.
// ROT: the keys are cached before RoPE; each tile's positions (pos) come into LDS with its rows,
// and the keys are turned to them before the contraction (score_tile16_rot, band turn fractions
// nu).  Every tile is then five loads per wave instead of four.
template <int G, int NTC, bool ROT>
__global__ __launch_bounds__(kClusterWaves * 64) void score_mfma_stage_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ ops, const float *__restrict__ pivot, int N,
    int streams, int Ps, int Kb, int cpx, int C, double *__restrict__ xpart, uint32_t *__restrict__ arrive,
    float *__restrict__ F, float *__restrict__ samp, float *__restrict__ raw_out, float *__restrict__ stats,
    int *__restrict__ err, const int32_t *__restrict__ pos, const uint64_t *__restrict__ nu)
{
    constexpr int NW = kClusterWaves;
    constexpr int GP = (G + 1) & ~1;
    extern __shared__ __attribute__((aligned(16))) float lraw[];   // [Kb][GP]
    __shared__ u32x4 stg[NW][2][256];              // two 4 KB key-tile slots per wave
    __shared__ BlockSumsT<NW> bs;
    __shared__ float zmu[8], zinv[8];
    __shared__ __attribute__((aligned(16))) double xs[32 * 8 * 4];   // the cluster's partials of a round
    // the next stream's operand words and pivots, loaded into LDS during a round; two buffers by round
    // parity, so that a round's loads never overwrite what a lagging wave may still read at the
    // start of the round before (a block barrier separates the two)
    __shared__ u32x4 ops_l[2][kOps * 64];
    __shared__ float piv_l[2][8];
    __shared__ uint32_t flg[64];                   // the cluster's arrival flags, fetched by wave 0
    __shared__ float pvs[2][8];                    // pivots of the streams of rounds r and r + 1
    __shared__ uint32_t zstamp;                    // rounds whose mean and 1/std are in zmu, zinv
    __shared__ int32_t pslot[NW][2][ROT ? 64 : 1]; // ROT: positions of each slot's tile (row l & 15 at l)
    __shared__ __attribute__((aligned(16))) int2 nu_l[ROT ? TRIA_HALF : 1];   // ROT: per band, see score_tile16_rot
    static_assert(NW == kOps, "one 1 KB operand load per wave");
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int cl = x * cpx + y / Ps, part = y % Ps;
    const int rounds = cl < streams ? (streams - cl + C - 1) / C : 0;
    if (rounds == 0) return;                       // the whole cluster has no stream
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jj = lane & 15, grp = lane >> 4, ha = head_a(grp);
    const int j0 = part * Kb;
    const int nkeys = max(0, min(Kb, N - j0));
    const int ntiles16 = (nkeys + 15) >> 4;
    const int nt = NTC > 0 ? NTC : max(1, (ntiles16 + NW - 1) / NW);   // items per wave and round
    // When every part runs the same item count, block `part` scores part (part + r) mod Ps of its
    // round-r stream, so that a part that streams slower is not always the same block's (every
    // block waits for its cluster's slowest each round); partial sums are filed by part, so the
    // merge order and the results do not change.
    auto prt = [&](int r) { return NTC > 0 ? ((part + r) & (Ps - 1)) : part; };
    auto nk_of = [&](int r) { return max(0, min(Kb, N - prt(r) * Kb)); };
    const int total = rounds * nt;

    WaveScorer<G> ws;
    ws.begin(ops, pivot, cl);
    // the operand loads complete here, before the first memory-to-LDS load is counted
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) hold(__builtin_bit_cast(uint4, ws.c.at[kb]));
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int h = 0; h < 2; ++h) hold(__builtin_bit_cast(uint4, ws.c.an[a][h]));
    hold(__builtin_bit_cast(uint32_t, ws.p[0]));
    hold(__builtin_bit_cast(uint32_t, ws.p[1]));
    if (wid == 0 && lane < G) pvs[0][lane] = pivot[(size_t)cl * G + lane];
    if (threadIdx.x == 0) zstamp = 0;     // read by the other waves only after the first barrier
    if constexpr (ROT) {
        if (threadIdx.x < TRIA_HALF) {
            const uint64_t v = nu[threadIdx.x];
            const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32) + (lo >> 31);
            nu_l[threadIdx.x] = make_int2((int)lo, (int)hi);
        }
        __syncthreads();
    }

    // Item li of a round is tile tile_of(li) of the block's part: wid + NW li, or, when the item
    // count is a known even number, the pairs 2 NW (li / 2) + 2 wid + (li & 1), so that every
    // 128-byte line of F (32 keys) belongs to one wave.
    auto tile_of = [&](int li) {
        if constexpr (NTC > 0 && NTC % 2 == 0) return 2 * NW * (li >> 1) + 2 * wid + (li & 1);
        else return wid + NW * li;
    };
    // item i of this wave: tile tile_of(i mod nt) of stream cl + (i / nt) C, into slot i & 1;
    // rows at or past the tile's valid count load row 0 (always a real row) and score nothing
    auto load_item = [&](int i) {
        const int ic = min(i, total - 1);
        const int r = ic / nt;
        const int sid = cl + r * C;
        const int nkr = nk_of(r);
        const int t = min(tile_of(ic - r * nt), ((nkr + 15) >> 4) - 1);
        const u32x4 *base = t >= 0 ? k + ((size_t)sid * N + prt(r) * Kb + t * 16) * 16 : k + (size_t)sid * N * 16;
        const int valid = t >= 0 ? nkr - t * 16 : 0;
        const u32x4 *slot = &stg[wid][i & 1][0];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int row = 4 * m + (lane >> 4);
            dma16(base + (row < valid ? row : 0) * 16 + ((lane & 15) ^ row), slot + 64 * m);
        }
        if constexpr (ROT) {
            // the rows' positions: lane l takes row l & 15 (rows at or past valid: row 0)
            const int row = lane & 15;
            const int32_t *pb = t >= 0 ? pos + (size_t)sid * N + prt(r) * Kb + t * 16 : pos + (size_t)sid * N;
            dma4(pb + (row < valid ? row : 0), &pslot[wid][i & 1][0]);
        }
    };
    // Wait until every vector memory operation but the newest 4 + e has completed: the newest
    // tile's 4 loads and the e operations (all written out in this kernel, so their count is
    // exact) that followed them.  Operations complete in issue order for this count, so a load
    // or store issued just after a tile is next waited for together with the following tile.
    // (ROT: the newest tile's 5 loads)
    auto wait_ring = [&](int e) {
        if constexpr (ROT) {
            switch (e) {
            case 0: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
            case 3: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
            case 4: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
            }
        } else {
            switch (e) {
            case 0: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
            case 3: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
            case 4: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
            }
        }
    };
    // the operand words (1 KB per wave) and pivots of the stream of round rn, loaded into LDS buffer
    // rn & 1; returns the number of load instructions issued
    auto stage_ops = [&](int rn) -> int {
        const int sn = cl + rn * C;
        dma16(ops + (size_t)sn * kOps * 64 + wid * 64 + lane, &ops_l[rn & 1][wid * 64]);
        if (wid != 0) return 1;
        if (lane < G) {
            const uint32_t la = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)piv_l[rn & 1]);
            const float *src = pivot + (size_t)sn * G + lane;   // lane l -> piv_l[l]
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(la)
                         : "memory", "m0");
        }
        return 2;
    };
    auto read_item = [&](int i, u32x4 (&b)[4]) {
        const u32x4 *slot = &stg[wid][i & 1][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) b[kb] = slot[jj * 16 + ((4 * kb + grp) ^ jj)];
    };
    auto put = [&](int li, int nkr, const float (&v)[2]) {
        const int key = tile_of(li) * 16 + jj;
        if (key < nkr) {
            if (ha < GP) lraw[key * GP + ha] = v[0];
            if (ha + 2 < GP) lraw[key * GP + ha + 2] = v[1];
        }
    };
    // round r's partial sums (staged in bs): wave 0 stores its block's per-head sums (s1, s2, min,
    // max as four doubles, two 16-byte stores) and, once a ring wait has covered those stores, sets
    // the block's arrival flag to the number of rounds it has published.  Both use the cache bits of
    // an agent-scope store, as the readers load with those of an agent-scope load, and return the
    // number of instructions issued.  (A flag per block, not a shared counter: an atomic add
    // completed late and held up every later load wait of the wave.)
    auto publish = [&](int r) -> int {
        if (wid != 0) return 0;
        double *xr = xpart + ((size_t)cl * 2 + (r & 1)) * Ps * G * 4;
        if (lane < G) {
            const Sums t2 = block_sums_of(bs, lane);
            double *q = xr + ((size_t)prt(r) * G + lane) * 4;
            const u32x4 w0 = __builtin_bit_cast(u32x4, double2{t2.s1, t2.s2});
            const u32x4 w1 = __builtin_bit_cast(u32x4, double2{(double)t2.mn, (double)t2.mx});
            // (a store of more than 8 bytes reads its data after issue: one wait state before
            // the registers may be rewritten)
            asm volatile("global_store_dwordx4 %0, %1, off sc1\n\tglobal_store_dwordx4 %0, %2, off offset:16 sc1\n\ts_nop 1"
                         ::"v"(q), "v"(w0), "v"(w1) : "memory");
        }
        return 2;
    };
    auto count_arrival = [&](int r) -> int {
        if (wid != 0) return 0;
        if (lane == 0)
            asm volatile("global_store_dword %0, %1, off sc1" ::"v"(&arrive[cl * Ps + part]), "v"((uint32_t)(r + 1))
                         : "memory");
        return 1;
    };
    // score item i (item li of its round) into v: its tile was loaded two items earlier and e_prev
    // operations followed the newest tile.  Once the tile is in registers its slot takes item
    // i + 2's tile, followed by the operands of round rn_ops's stream (rn_ops >= 0), round pub_r's partial
    // sums (pub_r >= 0) and round cnt's arrival (cnt >= 0).  Returns the number of those operations.
    auto score_item = [&](int i, int li, int nkr, int e_prev, int rn_ops, int pub_r, int cnt, float (&v)[2]) -> int {
        wait_ring(e_prev);
        u32x4 b[4];
        read_item(i, b);
        const int32_t kpos = ROT ? pslot[wid][i & 1][jj] : 0;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the slot has been read
        load_item(i + 2);
        int e = 0;
        if (rn_ops >= 0) e += stage_ops(rn_ops);
        if (pub_r >= 0) e += publish(pub_r);
        if (cnt >= 0) e += count_arrival(cnt);
        if constexpr (ROT)
            ws.score_rot(b, kpos, nu_l, nkr - tile_of(li) * 16, v);
        else
            ws.score(b, nkr - tile_of(li) * 16, v);
        return e;
    };
    // ---- finishing round r: the cluster's partial sums -> mean and 1/std per head -> F
    bool early = false;                  // wave 0 fetched round r's partials during the deferred items
    auto moments = [&](int r) {          // wave 0, from the partials in xs
        const int sid = cl + r * C;
        if (lane < G) {
            const int h = lane;
            Sums t2;
            t2.init();
            for (int pp = 0; pp < Ps; ++pp) {
                const double *q = xs + ((size_t)pp * G + h) * 4;
                Sums u;
                u.s1 = q[0]; u.s2 = q[1]; u.mn = (float)q[2]; u.mx = (float)q[3];
                t2.add(u);
            }
            double mean, sd;
            finish_moments(t2, (double)pvs[r & 1][h], (double)N, mean, sd);
            zmu[h] = (float)mean;
            zinv[h] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
            if (part == 0) {
                if (!isfinite(t2.s1) || !isfinite(t2.s2)) atomicOr(err, 1);
                if (stats) {
                    stats[((size_t)sid * G + h) * 2 + 0] = (float)mean;
                    stats[((size_t)sid * G + h) * 2 + 1] = (float)sd;
                }
            }
        }
        // the stamp follows the values (a wave's LDS operations complete in order; wait anyway)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_store(&zstamp, (uint32_t)(r + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // wave 0: the cluster's arrival flags into flg (lane l <- part min(l, Ps - 1)); one load
    auto fetch_flags = [&]() -> int {
        if (wid != 0) return 0;
        const uint32_t *src = arrive + (size_t)cl * Ps + min(lane, Ps - 1);
        const uint32_t la = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)flg);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off sc1" ::"v"(src), "s"(la)
                     : "memory", "m0");
        return 1;
    };
    // wave 0: if every flag in flg shows round r, round r's partials (Ps G x 32 bytes) into xs;
    // returns the number of loads
    auto fetch_parts = [&](int r) -> int {
        if (wid != 0) return 0;
        early = __all(flg[min(lane, Ps - 1)] >= (uint32_t)(r + 1));
        if (!early) return 0;
        const u32x4 *xr = (const u32x4 *)(xpart + ((size_t)cl * 2 + (r & 1)) * Ps * G * 4);
        const int nch = Ps * G * 2;      // 16-byte chunks, at most 512
        const int ni = (nch + 63) >> 6;
        const uint32_t la = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)xs);
        for (int m = 0; m < ni; ++m) {
            const u32x4 *src = xr + min(64 * m + lane, nch - 1);
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src),
                         "s"(la + 1024u * (uint32_t)m)
                         : "memory", "m0");
        }
        return ni;
    };
    // the block's F of round r: every wave normalises the keys of its own tiles (the rows it will
    // overwrite with its held scores) as soon as wave 0 has stamped the round's mean and 1/std, so
    // no wave waits for the others
    // e: operations issued after the newest tile (the partials, if fetched, are older than it)
    auto finish = [&](int r, int e) {
        const int sid = cl + r * C;
        if (wid == 0 && early) {
            wait_ring(e);                // the partials have landed
            moments(r);
        }
        if (wid == 0 && !early) {
            const double *xr = xpart + ((size_t)cl * 2 + (r & 1)) * Ps * G * 4;
            {
                // lane p < Ps watches part p's flag (the other lanes the last part's)
                const uint32_t *fl = arrive + (size_t)cl * Ps + min(lane, Ps - 1);
                unsigned spins = 0;
                while (!__all(__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)(r + 1))) {
                    if (++spins > kSpinLimit ||
                        (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2)) {
                        if (lane == 0) atomicOr(err, 2);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __builtin_amdgcn_wave_barrier();
            // every partial of the round (lane q takes partials q, q + 64, ... of Ps G <= 256; the
            // rest re-read the last) in one batch of coherent loads, waited for once
            const int nq = Ps * G;
            const uint32_t *xq[4];
#pragma unroll
            for (int it = 0; it < 4; ++it)
                xq[it] = (const uint32_t *)(xr + (size_t)min(lane + 64 * it, nq - 1) * 4);
            u32x4 w[4][2];
            asm volatile(
                "global_load_dwordx4 %0, %8, off sc1\n\t"
                "global_load_dwordx4 %1, %8, off offset:16 sc1\n\t"
                "global_load_dwordx4 %2, %9, off sc1\n\t"
                "global_load_dwordx4 %3, %9, off offset:16 sc1\n\t"
                "global_load_dwordx4 %4, %10, off sc1\n\t"
                "global_load_dwordx4 %5, %10, off offset:16 sc1\n\t"
                "global_load_dwordx4 %6, %11, off sc1\n\t"
                "global_load_dwordx4 %7, %11, off offset:16 sc1\n\t"
                "s_waitcnt vmcnt(0)"
                : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[1][0]), "=&v"(w[1][1]), "=&v"(w[2][0]), "=&v"(w[2][1]),
                  "=&v"(w[3][0]), "=&v"(w[3][1])
                : "v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3])
                : "memory");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int q = lane + 64 * it;
                if (q < nq) {
                    u32x4 *dst = (u32x4 *)(xs + (size_t)q * 4);
                    dst[0] = w[it][0];
                    dst[1] = w[it][1];
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_wave_barrier();
            moments(r);
        }
        early = false;
        // wave 0 has stamped round r by now or stamps it without waiting for the other waves
        while (__hip_atomic_load(&zstamp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)(r + 1))
            __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");   // zmu and zinv are read after the stamp
        const int jr = prt(r) * Kb, nkr = nk_of(r);
        float *fo = F + (size_t)sid * N + jr;
        float *so = samp + (size_t)sid * ((N + kSampleStride - 1) / kSampleStride) + jr / kSampleStride;
        // a key's raw scores (GP floats from LDS; keys at or past nkr read key 0, not stored)
        auto read_raw = [&](int key, float (&x)[GP]) {
            const float2 *src = (const float2 *)(lraw + (key < nkr ? key : 0) * GP);
#pragma unroll
            for (int h2 = 0; h2 < GP / 2; ++h2) {
                const float2 t = src[h2];
                x[2 * h2] = t.x;
                x[2 * h2 + 1] = t.y;
            }
        };
        auto emit = [&](int idx, int key, const float (&x)[GP]) {
            if (key >= nkr) return;
            float z = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h) z = fmaxf(z, (x[h] - zmu[h]) * zinv[h]);
            __builtin_nontemporal_store(z, &fo[key]);   // read back by the selection, not now
            // the first key of each 16-key tile (jr is a multiple of 16) to the side sample;
            // a plain store, so that L2 merges a line's 16 samples before it is written back
            static_assert(kSampleStride == 16, "one sampled key per 16-key tile");
            if ((idx & 15) == 0) so[key >> 4] = z;
            if (raw_out)
#pragma unroll
                for (int h = 0; h < G; ++h) raw_out[((size_t)sid * G + h) * N + jr + key] = x[h];
        };
        if constexpr (NTC > 0 && NTC % 8 == 0 && GP == 8) {
            // NTC * 16 / 64 keys per lane, two at a time with both keys' reads issued together, so
            // that one LDS round trip serves two keys (not unrolled further: registers)
#pragma unroll 1
            for (int q = 0; q < NTC / 4; q += 2) {
                const int i0 = lane + 64 * q, i1 = i0 + 64;
                const int k0 = tile_of(i0 >> 4) * 16 + (i0 & 15), k1 = tile_of(i1 >> 4) * 16 + (i1 & 15);
                float x0[GP], x1[GP];
                read_raw(k0, x0);
                read_raw(k1, x1);
                emit(i0, k0, x0);
                emit(i1, k1, x1);
            }
        } else {
            for (int idx = lane; idx < nt * 16; idx += 64) {
                const int key = tile_of(idx >> 4) * 16 + (idx & 15);
                float x[GP];
                read_raw(key, x);
                emit(idx, key, x);
            }
        }
    };

    load_item(0);
    load_item(1);
    const int ops_li = max(nt - 3, 0);   // the item that loads the next stream's operands
    int e = 0;                           // operations issued after the newest tile
    for (int r = 0; r < rounds; ++r) {
        const bool more = r + 1 < rounds;
        const int rn = more ? r + 1 : -1;    // the round whose operands this round stages
        const int nkr = nk_of(r);
        int li = 0;
        if (r > 0) {
            // The first items of a round (all 16 in a full block) keep their scores in registers
            // while the previous round is finished (its wait for the slowest block is covered by
            // scoring).  The previous round's partial sums are stored after
            // the first item's tile load, and the arrival is counted at the third item, whose
            // ring wait covers those stores; with fewer items, after waiting for everything.
            const int nd = min(kStageDefer, nt);
            // room for the early fetch: the partials' loads must precede the last deferred tile's
            const bool fetch = nd > kStageFlags + 3;
            float dv[kStageDefer][2];
#pragma unroll
            for (int q = 0; q < kStageDefer; ++q)
                if (q < nd) {
                    e = score_item(r * nt + q, q, nkr, e, q == ops_li ? rn : -1, q == 0 ? r - 1 : -1,
                                   q == 2 ? r - 1 : -1, dv[q]);
                    // each step issues its loads after the item's tile; a ring wait two items
                    // later covers them
                    if (q == kStageFlags && fetch) e += fetch_flags();
                    if (q == kStageFlags + 2 && fetch) e += fetch_parts(r - 1);
                }
            if (nd < 3) {
                if (nd == 0) publish(r - 1);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                count_arrival(r - 1);
            }
            finish(r - 1, e);
            e = 0;                       // the finish's stores only make the next wait stricter
#pragma unroll
            for (int q = 0; q < kStageDefer; ++q)
                if (q < nd) put(q, nkr, dv[q]);
            li = nd;
        }
        for (; li < nt; ++li) {
            float v[2];
            e = score_item(r * nt + li, li, nkr, e, li == ops_li ? rn : -1, -1, -1, v);
            put(li, nkr, v);
        }
        // ---- end of round r: stage the partial sums, switch to the next stream
        if (more && nt < 3) {            // the operands may still be the newest loads
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            e = 0;
        }
        block_sums_stage(bs, ws.m);
        __syncthreads();
        if (more) {
            // (two calls with fixed LDS addresses rather than one with a computed one: fewer registers)
            if ((r + 1) & 1) {
                ws.begin_lds(ops_l[1], piv_l[1]);
                if (wid == 0 && lane < G) pvs[1][lane] = piv_l[1][lane];
            } else {
                ws.begin_lds(ops_l[0], piv_l[0]);
                if (wid == 0 && lane < G) pvs[0][lane] = piv_l[0][lane];
            }
        }
    }
    publish(rounds - 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last round's stores and tile loads
    count_arrival(rounds - 1);
    finish(rounds - 1, 0);
}

// Cluster geometry for a stream of N keys: one block of 8 waves per CU, each keeping the raw
// scores of Kb keys in LDS, Ps blocks per stream (a power of two <= 32, so that clusters tile the
// 32-CU XCDs).  Measured on MI355X at 32768 keys and G = 8, this beats grids of two or three
// smaller blocks per CU with larger clusters (7.2 ms against 9.9 and 8.9 ms for 34 GB of keys):
// every extra block of a cluster adds a participant to each round's exchange.  False when the
// cluster path does not apply.
struct ClusterPlan {
    int Ps, Kb, nb, cpx, C;
};

template <int G>
static bool cluster_plan(int N, ClusterPlan &pl)
{
    constexpr int NW = kClusterWaves;
    constexpr int GP = (G + 1) & ~1;
    int dev = 0, n_cu = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
        return false;
    if (!coop || n_cu <= 0) return false;
    if (allow_dynamic_lds((const void *)score_mfma_cluster_kernel<G, NW>, kClusterLds) != hipSuccess) return false;
    const int kmax = (kClusterLds / (GP * 4)) & ~15;
    int Ps = 1;
    while ((long long)Ps * kmax < N) Ps *= 2;
    if (Ps > 32) return false;
    const int Kb = ((N + Ps - 1) / Ps + 15) & ~15;
    const int nb = (n_cu / (8 * Ps)) * 8 * Ps;
    if (nb <= 0 || nb > kClusterMaxBlocks) return false;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)score_mfma_cluster_kernel<G, NW>, NW * 64,
                                                     (size_t)Kb * GP * 4) != hipSuccess || per_cu < 1)
        return false;
    pl.Ps = Ps;
    pl.Kb = Kb;
    pl.nb = nb;
    pl.cpx = nb / 8 / Ps;
    pl.C = nb / Ps;
    return true;
}

template <int G>
static hipError_t launch_cluster_g(const ClusterPlan &pl, const u32x4 *kp, const u32x4 *ops, const float *pivot,
                                   int N, int streams, float *F, float *raw_out, float *stats,
                                   const tria_score_ws &lay, char *ws, hipStream_t st)
{
    constexpr int NW = kClusterWaves;
    constexpr int GP = (G + 1) & ~1;
    const size_t lds = (size_t)pl.Kb * GP * 4;
    uint32_t *arrive = (uint32_t *)(ws + lay.arrive_off);   // one counter per cluster, cleared by the prologue
    double *xpart = (double *)(ws + lay.xpart_off);
    int *err = (int *)(ws + lay.err_off);
    float *samp = (float *)(ws + lay.samp_off);
    int n = N, S = streams, Ps = pl.Ps, Kb = pl.Kb, cpx = pl.cpx, C = pl.C;
    void *args[] = {(void *)&kp,    (void *)&ops,   (void *)&pivot, &n,
                    &S,             &Ps,            &Kb,            &cpx,
                    &C,             (void *)&xpart, (void *)&arrive, (void *)&F,
                    (void *)&samp,  (void *)&raw_out, (void *)&stats, (void *)&err};
    KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
    return hipLaunchCooperativeKernel((const void *)score_mfma_cluster_kernel<G, NW>, dim3(pl.nb), dim3(NW * 64),
                                      args, (unsigned)lds, st);
}

// Geometry of the staged cluster path (raw scores of at most kStageLds bytes per block) for
// `streams` streams of N keys; false when it does not apply.  Of the part counts Ps that fit
// (Ps Kb >= N, Ps <= 32, parts of at least kStageMinKeys keys unless one part holds the stream),
// the one with the least modelled time: rounds = ceil(streams / C) of Kb keys each, plus a fixed
// cost per round worth kStageRoundKeys keys (the finish and the exchange).  Long streams take the
// fewest parts that fit; few streams of moderate length spread over more parts, so that the
// clusters' rounds come out even.
constexpr int kStageRoundKeys = 256;
constexpr int kStageMinKeys = 512;

template <int G>
static bool stage_plan(int N, int streams, ClusterPlan &pl)
{
    constexpr int NW = kClusterWaves;
    constexpr int GP = (G + 1) & ~1;
    int dev = 0, n_cu = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
        return false;
    if (!coop || n_cu <= 0) return false;
    if (allow_dynamic_lds((const void *)score_mfma_stage_kernel<G, 0, false>, kStageLds) != hipSuccess) return false;
    const int kmax = (kStageLds / (GP * 4)) & ~15;
    int Ps0 = 1;
    while ((long long)Ps0 * kmax < N) Ps0 *= 2;
    if (Ps0 > 32) return false;
    int best = -1;
    double best_cost = 0.0;
    for (int Ps = Ps0; Ps <= 32; Ps *= 2) {
        const int Kb = ((N + Ps - 1) / Ps + 15) & ~15;
        if (Ps > Ps0 && Kb < kStageMinKeys) break;
        const int nb = (n_cu / (8 * Ps)) * 8 * Ps;
        if (nb <= 0 || nb > kClusterMaxBlocks) break;
        const int C = nb / Ps;
        const double cost = (double)((streams + C - 1) / C) * (double)(Kb + kStageRoundKeys);
        if (best < 0 || cost < best_cost) {
            best = Ps;
            best_cost = cost;
        }
    }
    if (best < 0) return false;
    const int Ps = best;
    const int Kb = ((N + Ps - 1) / Ps + 15) & ~15;
    const int nb = (n_cu / (8 * Ps)) * 8 * Ps;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)score_mfma_stage_kernel<G, 0, false>, NW * 64,
                                                     (size_t)Kb * GP * 4) != hipSuccess || per_cu < 1)
        return false;
    pl.Ps = Ps;
    pl.Kb = Kb;
    pl.nb = nb;
    pl.cpx = nb / 8 / Ps;
    pl.C = nb / Ps;
    return true;
}

// The plans above query the device (attributes, occupancy) and raise dynamic-LDS limits: host work
// of several microseconds that the GPU would otherwise wait for at every call.  Each (device, path,
// G, N, streams) is planned once and remembered (whether a path applies does not depend on the
// stream count).
template <int G>
static bool cached_plan(bool staged, int N, int streams, ClusterPlan &pl)
{
    static std::mutex mu;
    static std::map<std::tuple<int, bool, int, int>, std::pair<bool, ClusterPlan>> memo;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    const auto key = std::make_tuple(dev, staged, N, staged ? streams : 1);
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = memo.find(key);
        if (it != memo.end()) {
            pl = it->second.second;
            return it->second.first;
        }
    }
    ClusterPlan p{};
    const bool ok = staged ? stage_plan<G>(N, streams, p) : cluster_plan<G>(N, p);
    std::lock_guard<std::mutex> lock(mu);
    memo[key] = std::make_pair(ok, p);
    pl = p;
    return ok;
}

// rot: pre-RoPE keys at positions pos (band turn fractions nu)
template <int G>
static hipError_t launch_stage_g(const ClusterPlan &pl, const u32x4 *kp, const u32x4 *ops, const float *pivot,
                                 int N, int streams, float *F, float *raw_out, float *stats,
                                 const tria_score_ws &lay, char *ws, const int32_t *pos, const uint64_t *nu,
                                 bool rot, hipStream_t st)
{
    constexpr int NW = kClusterWaves;
    constexpr int GP = (G + 1) & ~1;
    const size_t lds = (size_t)pl.Kb * GP * 4;
    uint32_t *arrive = (uint32_t *)(ws + lay.arrive_off);   // one flag per block, cleared by the prologue
    double *xpart = (double *)(ws + lay.xpart_off);
    int *err = (int *)(ws + lay.err_off);
    float *samp = (float *)(ws + lay.samp_off);
    int n = N, S = streams, Ps = pl.Ps, Kb = pl.Kb, cpx = pl.cpx, C = pl.C;
    void *args[] = {(void *)&kp,    (void *)&ops,   (void *)&pivot, &n,
                    &S,             &Ps,            &Kb,            &cpx,
                    &C,             (void *)&xpart, (void *)&arrive, (void *)&F,
                    (void *)&samp,  (void *)&raw_out, (void *)&stats, (void *)&err,
                    (void *)&pos,   (void *)&nu};
    // every block full (the first and the last part of a stream run the same item count): the
    // variant with that count built in
    auto items = [](int nkeys) { return std::max(1, ((nkeys + 15) / 16 + NW - 1) / NW); };
    constexpr int full = stage_full_items<G>();
    // (turned keys with G < 7: the built-in counts of 22 to 64 items spill ~90 registers, the
    // variant with a runtime count none)
    const bool exact = items(pl.Kb) == full && items(N - (pl.Ps - 1) * pl.Kb) == full && !(rot && G < 7);
    const void *fn = rot ? (exact ? (const void *)score_mfma_stage_kernel<G, full, true>
                                  : (const void *)score_mfma_stage_kernel<G, 0, true>)
                         : (exact ? (const void *)score_mfma_stage_kernel<G, full, false>
                                  : (const void *)score_mfma_stage_kernel<G, 0, false>);
    if ((exact || rot) && allow_dynamic_lds(fn, kStageLds) != hipSuccess) return hipErrorInvalidValue;
    KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
    return hipLaunchCooperativeKernel(fn, dim3(pl.nb), dim3(NW * 64), args, (unsigned)lds, st);
}

// ---- maximum over the future offsets (TRIA_OFFSET_MAX) ------------------------------------------
// The trigonometric score as the largest of the per-offset series (chenxutan.com/d/2624 section
// 3.3): S_trig(j) = max_{d in D} sum_f Re[qbar_f e^{i w_f (t + d)} conj(ktilde_{j,f})], plus the
// unchanged norm score.  Per offset the series is a dot product of the key with a query rotated to
// t + d, so each offset is one more matrix-core contraction: |D| x 4 MFMAs per 16-key tile, whose
// A operands (the rotated queries, two bf16 terms each) a block builds once in LDS from qbar (fp64,
// exact turn fractions, optionally scaled by R_f) and reads back per tile.  The norm part uses the
// regular operands.  One block of 4 waves per (stream, kMaxdKeys-key chunk); raw scores go
// head-major to the workspace, per-chunk sums around 0 to the partials, and the statistics and
// z-max kernels of the tiled path finish.
constexpr int kMaxdKeys = 8192;
constexpr int kMaxdOffsets = kMaxdOffsetsLimit;   // offsets whose operands fit the block's LDS (4 KB each)

template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_maxd_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ ops, const double2 *__restrict__ Qc,
    const float *__restrict__ R, const uint64_t *__restrict__ nu, const int64_t *__restrict__ off, int n_off,
    const int32_t *__restrict__ t, int L, int Hkv, int N, int chunks, float *__restrict__ raw,
    double *__restrict__ part)
{
    extern __shared__ u32x4 opsd[];                // [n_off][4 K-blocks][64 lanes]
    __shared__ BlockSums bs;
    const int sid = blockIdx.x / chunks;
    const int chunk = blockIdx.x - sid * chunks;
    const int g = sid % Hkv;
    const int l = (sid / Hkv) % L;
    const int s = sid / (Hkv * L);
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jj = lane & 15, ha = head_a(lane >> 4);

    // ---- per-offset operands in LDS: zero (rows of heads >= G), then scatter the terms
    for (int i = threadIdx.x; i < n_off * 4 * 64; i += kScoreThreads) opsd[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    {
        __bf16 *ob = (__bf16 *)opsd;
        const int64_t ts = t[s];
        const size_t hh0 = ((size_t)l * Hkv + g) * G;
        for (int i = threadIdx.x; i < n_off * G * TRIA_HALF; i += kScoreThreads) {
            const int d = i / (G * TRIA_HALF);
            const int r = i - d * (G * TRIA_HALF);
            const int h = r / TRIA_HALF, f = r - h * TRIA_HALF;
            const uint64_t turns = (uint64_t)(ts + off[d]) * nu[f];     // (t + d) w_f / 2pi mod 1, exact
            double sn, cs;
            sincospi(2.0 * ((double)(int64_t)turns * 0x1p-64), &sn, &cs);
            const double2 q = Qc[(hh0 + h) * TRIA_HALF + f];
            const double wr = R ? (double)R[(hh0 + h) * TRIA_HALF + f] : 1.0;
            const float comp[2] = {(float)(wr * (q.x * cs - q.y * sn)), (float)(wr * (q.x * sn + q.y * cs))};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int dim = f + c * TRIA_HALF;          // real part at f, imaginary at f + 64
                const int kb = dim >> 5, grp = (dim >> 3) & 3, e = dim & 7;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int ln = grp * 16 + 8 * b + h;    // A row 8b + h, K chunk grp
                    ob[(((size_t)d * 4 + kb) * 64 + ln) * 8 + e] = (__bf16)bf16_term(comp[c], b);
                }
            }
        }
    }
    __syncthreads();

    Ops c;
    load_ops(c, ops + (size_t)sid * kOps * 64);
    Sums m[2];
    m[0].init();
    m[1].init();
    const int j0 = chunk * kMaxdKeys;
    const int nkeys = min(kMaxdKeys, N - j0);
    const int ntiles16 = (nkeys + 15) >> 4;
    const u32x4 *kb = k + ((size_t)sid * N + j0) * 16;
    // items of a wave: pairs of consecutive 16-key tiles 2p, 2p + 1 for p = wid, wid + 4, ...; each
    // operand read from LDS serves both tiles
    const int npairs = (ntiles16 + 1) >> 1;
    const int nt_w = wid < npairs ? (npairs - wid + 3) >> 2 : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        raw + (size_t)sid * G * N + j0, 0, ((G - 1) * N + nkeys) * 4, 0x00020000);
    constexpr int kDrop = 0x7fffffff;
    auto issue = [&](u32x4 (&bt)[2][4], int i) {
        const int pr = min(wid + 4 * i, npairs - 1);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = min(2 * pr + q, ntiles16 - 1);
            load_tile(bt[q], kb + (size_t)tt * 16 * 16, nkeys - tt * 16);
        }
    };
    // band norms of a tile against the regular norm operands (as in score_tile16)
    auto norm_part = [&](const u32x4 (&ka)[4]) {
        floatx4 accn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const u32x4 x = ka[half], y = ka[2 + half];
            u32x4 t0, t1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t p0 = __builtin_amdgcn_perm(y[q], x[q], 0x05040100u);
                const uint32_t p1 = __builtin_amdgcn_perm(y[q], x[q], 0x07060302u);
                const Split2 n = split2(__builtin_amdgcn_sqrtf(band_sq(p0)), __builtin_amdgcn_sqrtf(band_sq(p1)));
                t0[q] = n.hi;
                t1[q] = n.lo;
            }
            accn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[0][half], __builtin_bit_cast(bf16x8, t0), accn, 0, 0, 0);
            accn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.an[1][half], __builtin_bit_cast(bf16x8, t1), accn, 0, 0, 0);
        }
        return accn;
    };
    auto compute = [&](const u32x4 (&bt)[2][4], int i) {
        const int pr = wid + 4 * i;
        floatx4 accn[2] = {norm_part(bt[0]), norm_part(bt[1])};
        // trigonometric part: the largest per-offset series, both tiles per operand read
        float mx[2][2] = {{-INFINITY, -INFINITY}, {-INFINITY, -INFINITY}};
        // two offsets per step (four independent accumulator chains), so that one offset's
        // products run while the other's operands arrive and results are combined
        auto fold = [&](floatx4 (&acc)[2]) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float a0 = acc[q][0], a1 = acc[q][1], a2 = acc[q][2], a3 = acc[q][3];
                permlane32_swap(a0, a1);
                permlane32_swap(a2, a3);
                mx[q][0] = fmaxf(mx[q][0], a0 + a1);
                mx[q][1] = fmaxf(mx[q][1], a2 + a3);
            }
        };
        auto products = [&](int d, floatx4 (&acc)[2]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, opsd[(d * 4 + q) * 64 + lane]);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bt[0][q]), acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bt[1][q]), acc[1], 0, 0, 0);
            }
        };
        int d = 0;
        for (; d + 1 < n_off; d += 2) {
            floatx4 acc0[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            floatx4 acc1[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            products(d, acc0);
            products(d + 1, acc1);
            fold(acc0);
            fold(acc1);
        }
        if (d < n_off) {
            floatx4 acc0[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            products(d, acc0);
            fold(acc0);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float n0 = accn[q][0], n1 = accn[q][1], n2 = accn[q][2], n3 = accn[q][3];
            permlane32_swap(n0, n1);
            permlane32_swap(n2, n3);
            const float v0 = mx[q][0] + (n0 + n1), v1 = mx[q][1] + (n2 + n3);
            const int tt = 2 * pr + q;
            const int key = tt * 16 + jj;
            const bool in = tt < ntiles16 && key < nkeys;
            if (in && ha < G) m[0].add(v0, 0.f);
            if (in && ha + 2 < G) m[1].add(v1, 0.f);
            const int o0 = (in && ha < G) ? (ha * N + key) * 4 : kDrop;
            const int o1 = (in && ha + 2 < G) ? ((ha + 2) * N + key) * 4 : kDrop;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v0), rsrc, o0, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v1), rsrc, o1, 0, 0);
        }
    };
    if (nt_w > 0) {
        u32x4 r0[2][4], r1[2][4], r2[2][4], r3[2][4];
        const int n4 = (nt_w + 3) & ~3;
        issue(r0, 0);
        TRIA_PIN();
        issue(r1, 1);
        TRIA_PIN();
        issue(r2, 2);
        TRIA_PIN();
        for (int i = 0; i < n4; i += 4) {
            issue(r3, i + 3);
            TRIA_PIN();
            compute(r0, i);
            issue(r0, i + 4);
            TRIA_PIN();
            compute(r1, i + 1);
            issue(r1, i + 5);
            TRIA_PIN();
            compute(r2, i + 2);
            issue(r2, i + 6);
            TRIA_PIN();
            compute(r3, i + 3);
            TRIA_PIN();
        }
    }
    block_sums_stage(bs, m);
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        const Sums t2 = block_sums_of(bs, h);
        double *q = part + (((size_t)sid * chunks + chunk) * G + h) * 4;
        q[0] = t2.s1;
        q[1] = t2.s2;
        q[2] = (double)t2.mn;
        q[3] = (double)t2.mx;
    }
}

template <int G>
static hipError_t launch_maxd_g(const tria_calib *c, const void *k, const int32_t *t, int n_seq, int N,
                                bool weight_r, float *F, float *raw_out, float *stats, const tria_score_ws &lay,
                                char *ws, hipStream_t st)
{
    const int streams = n_seq * c->L * c->Hkv;
    const u32x4 *kp = (const u32x4 *)k;
    u32x4 *ops = (u32x4 *)(ws + lay.ops_off);
    float *pivot = (float *)(ws + lay.pivot_off);
    // the norm operands (the trigonometric ones are built per offset by the kernel, R-weighted there)
    hipError_t e = launch_prologue<G>(c, kp, t, nullptr, n_seq, N, false, ops, pivot, (int *)(ws + lay.err_off), nullptr, 0, st);
    if (e != hipSuccess) return e;
    e = allow_dynamic_lds((const void *)score_maxd_kernel<G>, kMaxdOffsets * 4 * 64 * 16);
    if (e != hipSuccess) return e;
    if (!lay.has_raw) return hipErrorInvalidValue;   // the layout did not plan this path
    float *raw = raw_out ? raw_out : (float *)(ws + lay.raw_off);
    double *part = (double *)(ws + lay.part_off);
    const int chunks = (N + kMaxdKeys - 1) / kMaxdKeys;
    const long long blocks = (long long)streams * chunks;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    {
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        score_maxd_kernel<G><<<(unsigned)blocks, kScoreThreads, (size_t)c->n_off * 4 * 64 * 16, st>>>(
            kp, ops, c->Qc, weight_r ? c->R : nullptr, c->nu, c->off, c->n_off, t, c->L, c->Hkv, N, chunks, raw, part);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return launch_tile_finish(G, streams, N, chunks, raw, part, nullptr, F, stats, lay, ws, st);
}

hipError_t launch_score_maxd(const tria_calib *c, const void *k, const int32_t *t, int n_seq, int N, bool weight_r, float *F, float *raw, float *stats, const tria_score_ws &lay, char *ws,
                             hipStream_t st)
{
    if (c->n_off > kMaxdOffsets) return hipErrorInvalidValue;
    switch (c->G) {
    case 1: return launch_maxd_g<1>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 2: return launch_maxd_g<2>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 3: return launch_maxd_g<3>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 4: return launch_maxd_g<4>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 5: return launch_maxd_g<5>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 6: return launch_maxd_g<6>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 7: return launch_maxd_g<7>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 8: return launch_maxd_g<8>(c, k, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    }
    return hipErrorInvalidValue;
}

// ---- launch ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_tile_finish_g(int streams, int N, int tiles, const float *raw, const double *part,
                                       const float *pivot, float *F, float *stats, const tria_score_ws &lay, char *ws,
                                       hipStream_t st)
{
    KernelTimer timer(TRIA_TIMER_NORMALISE, st);
    int *err = (int *)(ws + lay.err_off);
    float *zst = (float *)(ws + lay.zst_off);
    tile_stats_kernel<G><<<streams, kScoreThreads, 0, st>>>(part, pivot, N, tiles, zst, stats, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long blocks = (long long)streams * ((N + kZmaxKeys - 1) / kZmaxKeys);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    zmax_tiles_kernel<G><<<(unsigned)blocks, kScoreThreads, 0, st>>>(raw, zst, N, (N + kZmaxKeys - 1) / kZmaxKeys, F);
    return hipGetLastError();
}

hipError_t launch_tile_finish(int G, int streams, int N, int tiles, const float *raw, const double *part,
                              const float *pivot, float *F, float *stats, const tria_score_ws &lay, char *ws,
                              hipStream_t st)
{
    switch (G) {
    case 1: return launch_tile_finish_g<1>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 2: return launch_tile_finish_g<2>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 3: return launch_tile_finish_g<3>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 4: return launch_tile_finish_g<4>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 5: return launch_tile_finish_g<5>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 6: return launch_tile_finish_g<6>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 7: return launch_tile_finish_g<7>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    case 8: return launch_tile_finish_g<8>(streams, N, tiles, raw, part, pivot, F, stats, lay, ws, st);
    }
    return hipErrorInvalidValue;
}

template <int G>
static hipError_t launch_mfma_g(const tria_calib *c, const void *k, const int32_t *pos, const int32_t *t, int n_seq,
                                int N, bool weight_r, float *F, float *raw_out, float *stats, const tria_score_ws &lay,
                                char *ws, hipStream_t st)
{
    const int streams = n_seq * c->L * c->Hkv;
    int *err = (int *)(ws + lay.err_off);
    const u32x4 *kp = (const u32x4 *)k;
    u32x4 *ops = (u32x4 *)(ws + lay.ops_off);
    float *pivot = (float *)(ws + lay.pivot_off);
    // the path: one block per stream (on chip), staged or register-ring stream clusters, or tiled
    enum { kOnChip, kStaged, kRing, kTiled } path = kOnChip;
    ClusterPlan pl{};
    if (lay.cluster) {
        // (streams short enough for one block take the staged clusters only; the layout checked)
        if (cached_plan<G>(true, N, streams, pl)) path = kStaged;
        else if (lay.tiled && cached_plan<G>(false, N, 1, pl)) path = kRing;
        else return hipErrorInvalidValue;   // the layout planned a cluster path the device no longer offers
    } else if (lay.tiled) {
        if (!lay.has_raw) return hipErrorInvalidValue;
        path = kTiled;
    }
    // the cluster paths' arrival words (one flag per block, or one counter per cluster) are cleared
    // by the prologue
    // pre-RoPE keys are turned inside the staged kernel only (the layout planned it)
    if (lay.rot && (path != kStaged || !pos)) return hipErrorInvalidValue;
    uint32_t *arrive = (path == kStaged || path == kRing) ? (uint32_t *)(ws + lay.arrive_off) : nullptr;
    const int n_arrive = path == kStaged ? pl.nb : path == kRing ? pl.C : 0;
    hipError_t e = launch_prologue<G>(c, kp, t, lay.rot ? pos : nullptr, n_seq, N, weight_r, ops, pivot, err, arrive,
                                      n_arrive, st);
    if (e != hipSuccess) return e;
    if (path == kOnChip) {
        const size_t lds = (size_t)G * (N | 1) * 4;
        e = allow_dynamic_lds((const void *)score_mfma_fused_kernel<G>, kFusedLdsMax);
        if (e != hipSuccess) return e;
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        score_mfma_fused_kernel<G><<<streams, kScoreThreads, lds, st>>>(kp, ops, pivot, N, F, raw_out, stats, err);
        return hipGetLastError();
    }
    if (path == kStaged)
        return launch_stage_g<G>(pl, kp, ops, pivot, N, streams, F, raw_out, stats, lay, ws, pos, c->nu, lay.rot != 0,
                                 st);
    if (path == kRing) return launch_cluster_g<G>(pl, kp, ops, pivot, N, streams, F, raw_out, stats, lay, ws, st);
    // raw scores go straight into the caller's raw output when there is one (same layout)
    float *raw = raw_out ? raw_out : (float *)(ws + lay.raw_off);
    double *part = (double *)(ws + lay.part_off);
    const long long blocks = (long long)streams * lay.tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    {
        KernelTimer timer(TRIA_TIMER_SCORE_KEYS, st);
        score_mfma_tile_kernel<G><<<(unsigned)blocks, kScoreThreads, 0, st>>>(kp, ops, pivot, N, lay.tiles, raw, part);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return launch_tile_finish(G, streams, N, lay.tiles, raw, part, pivot, F, stats, lay, ws, st);
}

template <int G>
static bool cluster_applies_g(int N)
{
    ClusterPlan pl;
    return cached_plan<G>(true, N, 1, pl) || cached_plan<G>(false, N, 1, pl);
}

template <int G>
static bool stage_applies_g(int N)
{
    ClusterPlan pl;
    return cached_plan<G>(true, N, 1, pl);
}

bool stage_path_applies(int G, int N)
{
    switch (G) {
    case 1: return stage_applies_g<1>(N);
    case 2: return stage_applies_g<2>(N);
    case 3: return stage_applies_g<3>(N);
    case 4: return stage_applies_g<4>(N);
    case 5: return stage_applies_g<5>(N);
    case 6: return stage_applies_g<6>(N);
    case 7: return stage_applies_g<7>(N);
    case 8: return stage_applies_g<8>(N);
    }
    return false;
}

bool cluster_path_applies(int G, int N)
{
    switch (G) {
    case 1: return cluster_applies_g<1>(N);
    case 2: return cluster_applies_g<2>(N);
    case 3: return cluster_applies_g<3>(N);
    case 4: return cluster_applies_g<4>(N);
    case 5: return cluster_applies_g<5>(N);
    case 6: return cluster_applies_g<6>(N);
    case 7: return cluster_applies_g<7>(N);
    case 8: return cluster_applies_g<8>(N);
    }
    return false;
}

hipError_t launch_score_mfma(const tria_calib *c, const void *k, const int32_t *pos, const int32_t *t, int n_seq,
                             int N, bool weight_r, float *F, float *raw, float *stats, const tria_score_ws &lay,
                             char *ws, hipStream_t st)
{
    switch (c->G) {
    case 1: return launch_mfma_g<1>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 2: return launch_mfma_g<2>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 3: return launch_mfma_g<3>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 4: return launch_mfma_g<4>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 5: return launch_mfma_g<5>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 6: return launch_mfma_g<6>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 7: return launch_mfma_g<7>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    case 8: return launch_mfma_g<8>(c, k, pos, t, n_seq, N, weight_r, F, raw, stats, lay, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tria
