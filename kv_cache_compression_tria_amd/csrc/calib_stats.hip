// calib_stats.hip -- calibration statistics of captured pre-RoPE queries (gfx950).
//
// The offline step that feeds tria_load_calib (TriAttention pages: chenxutan.com/d/2624 section
// 3.4, the per-head centre, mean norm and concentration from about ten thousand captured
// tokens; zhichai.net section "破局之道" for R as the norm of the mean over the mean norm).  Per
// (layer, query head) and band f (the complex number q[f] + i q[f + 64]):
//   qbar_f = mean_n q_{n,f},   E|q_f| = mean_n |q_{n,f}|,   R_f = |qbar_f| / E|q_f|  (0 if E|q_f| = 0).
//
// One block per head, HBM-bound (every captured value is read once).  A 16-lane group reads one
// query row: lane c takes bands 4c..4c+3, i.e. 8 (bf16) or 16 (fp32) contiguous bytes of the real
// half and the same of the imaginary half, so each half-row is one 128- or 256-byte segment and
// a wave's load covers four whole rows.  The four row groups of wave w take rows 4w + g,
// 4w + g + 4 NW, ...; four rows per lane (eight in one-wave blocks) are in flight, with
// non-temporal loads, and added in fp32 (|q_f| itself in fp32 from the exact input values), then
// into fp64 sums, which are combined in a fixed order: the
// row groups by butterfly, then the waves in order.  The waves per block (NW) are the most with
// which every head's block is resident at once (one wave per head for the Qwen3-32B shapes, 4096
// heads; four for Qwen3-8B's 1152), so every head streams from the start and no partial last wave
// of blocks trails the launch.  |q_f| uses the hardware square root (within 1 ulp); the
// correctly rounded expansion would hold four times the registers.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Bands 4c .. 4c+3 of one query row: 8 contiguous bytes of the real half and 8 of the imaginary
// half for bf16 (16 and 16 for fp32).  Non-temporal loads: every value is read once.
template <bool BF16>
__device__ __forceinline__ void load_band4(const char *__restrict__ row, int c, float (&re)[4], float (&im)[4])
{
    if (BF16) {
        const u32x2 a = __builtin_nontemporal_load((const u32x2 *)(row + c * 8));         // dims 4c .. 4c+3
        const u32x2 b = __builtin_nontemporal_load((const u32x2 *)(row + 128 + c * 8));   // dims 64 + 4c ..
        re[0] = bf16_lo(a.x); re[1] = bf16_hi(a.x); re[2] = bf16_lo(a.y); re[3] = bf16_hi(a.y);
        im[0] = bf16_lo(b.x); im[1] = bf16_hi(b.x); im[2] = bf16_lo(b.y); im[3] = bf16_hi(b.y);
    } else {
        const f32x4 a = __builtin_nontemporal_load((const f32x4 *)(row + c * 16));
        const f32x4 b = __builtin_nontemporal_load((const f32x4 *)(row + 256 + c * 16));
        re[0] = a.x; re[1] = a.y; re[2] = a.z; re[3] = a.w;
        im[0] = b.x; im[1] = b.y; im[2] = b.z; im[3] = b.w;
    }
}

template <bool BF16, int NW>
__global__ __launch_bounds__(NW * 64) void calib_stats_kernel(const void *__restrict__ q, int n_cal,
                                                              float *__restrict__ qc, float *__restrict__ qn,
                                                              float *__restrict__ rb)
{
    constexpr int RB = BF16 ? 256 : 512;       // row bytes
    constexpr int U = NW == 1 ? 8 : 4;         // rows per lane in flight (more for one-wave blocks)
    __shared__ double red[NW][3][TRIA_HALF];
    const int hh = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;    // lane c of row group g (4 groups per wave)
    const char *base = (const char *)q + (size_t)hh * n_cal * RB;
    double sr[4], si[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sr[e] = si[e] = sn[e] = 0.0;
    const int stride = NW * 4;
    int n = wid * 4 + g;
    // U rows per lane in flight; their values are added in fp32 (U terms), then once into fp64
    for (; n + (U - 1) * stride < n_cal; n += U * stride) {
        float re[U][4], im[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) load_band4<BF16>(base + (size_t)(n + u * stride) * RB, c, re[u], im[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float ar = 0.f, ai = 0.f, an = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float x = re[u][e], y = im[u][e];
                ar += x;
                ai += y;
                an += __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
            }
            sr[e] += (double)ar;
            si[e] += (double)ai;
            sn[e] += (double)an;
        }
    }
    for (; n < n_cal; n += stride) {
        float re[4], im[4];
        load_band4<BF16>(base + (size_t)n * RB, c, re, im);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sr[e] += (double)re[e];
            si[e] += (double)im[e];
            sn[e] += (double)__builtin_amdgcn_sqrtf(fmaf(re[e], re[e], im[e] * im[e]));
        }
    }
    // row groups 0..3 of the wave: butterfly over lane bits 4..5 (fixed order)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            sr[e] += __shfl_xor(sr[e], o, 64);
            si[e] += __shfl_xor(si[e], o, 64);
            sn[e] += __shfl_xor(sn[e], o, 64);
        }
    }
    if (g == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            red[wid][0][4 * c + e] = sr[e];
            red[wid][1][4 * c + e] = si[e];
            red[wid][2][4 * c + e] = sn[e];
        }
    }
    __syncthreads();
    if (threadIdx.x < TRIA_HALF) {
        const int f = threadIdx.x;
        double tr = 0.0, ti = 0.0, tn = 0.0;
        for (int w = 0; w < NW; ++w) {
            tr += red[w][0][f];
            ti += red[w][1][f];
            tn += red[w][2][f];
        }
        const double mr = tr / n_cal, mi = ti / n_cal, mn = tn / n_cal;
        qc[(size_t)hh * TRIA_D + f] = (float)mr;
        qc[(size_t)hh * TRIA_D + TRIA_HALF + f] = (float)mi;
        qn[(size_t)hh * TRIA_HALF + f] = (float)mn;
        rb[(size_t)hh * TRIA_HALF + f] = mn > 0.0 ? (float)(sqrt(mr * mr + mi * mi) / mn) : 0.f;
    }
}

template <bool BF16, int NW>
static hipError_t launch_calib_nw(bool run, int &resident, const void *q, int n_heads, int n_cal, float *qc,
                                  float *qn, float *rb, hipStream_t st)
{
    if (!run) {
        // blocks of this variant resident per CU
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, (const void *)calib_stats_kernel<BF16, NW>,
                                                            NW * 64, 0);
    }
    calib_stats_kernel<BF16, NW><<<n_heads, NW * 64, 0, st>>>(q, n_cal, qc, qn, rb);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_calib_dt(bool run, int nw, int &resident, const void *q, int n_heads, int n_cal, float *qc,
                                  float *qn, float *rb, hipStream_t st)
{
    switch (nw) {
    case 1: return launch_calib_nw<BF16, 1>(run, resident, q, n_heads, n_cal, qc, qn, rb, st);
    case 2: return launch_calib_nw<BF16, 2>(run, resident, q, n_heads, n_cal, qc, qn, rb, st);
    case 4: return launch_calib_nw<BF16, 4>(run, resident, q, n_heads, n_cal, qc, qn, rb, st);
    case 8: return launch_calib_nw<BF16, 8>(run, resident, q, n_heads, n_cal, qc, qn, rb, st);
    default: return launch_calib_nw<BF16, 16>(run, resident, q, n_heads, n_cal, qc, qn, rb, st);
    }
}

hipError_t launch_calib_stats(tria_dtype dt, const void *q, int n_heads, int n_cal, float *qc, float *qn, float *rb,
                              hipStream_t st)
{
    const bool bf16 = dt == TRIA_BF16;
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // waves per block: the most (1 .. 16) with which every head's block is resident at once, so
    // that all heads stream together and no partial last wave of blocks trails the launch (one
    // wave per head when the heads outnumber the resident blocks); never more waves than the rows
    // give work for (four rows per wave step)
    int nw = 1;
    for (int cand = 2; cand <= 16 && 4 * cand <= n_cal; cand *= 2) {
        int resident = 0;
        e = bf16 ? launch_calib_dt<true>(false, cand, resident, q, n_heads, n_cal, qc, qn, rb, st)
                 : launch_calib_dt<false>(false, cand, resident, q, n_heads, n_cal, qc, qn, rb, st);
        if (e != hipSuccess) return e;
        if ((long long)resident * n_cu < n_heads) break;
        nw = cand;
    }
    int unused = 0;
    KernelTimer timer(TRIA_TIMER_CALIB, st);
    return bf16 ? launch_calib_dt<true>(true, nw, unused, q, n_heads, n_cal, qc, qn, rb, st)
                : launch_calib_dt<false>(true, nw, unused, q, n_heads, n_cal, qc, qn, rb, st);
}

}  // namespace tria
