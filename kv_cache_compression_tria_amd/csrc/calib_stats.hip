// calib_stats.hip -- calibration statistics of captured pre-RoPE queries (gfx950).
//
// The offline step that feeds tria_load_calib (TriAttention pages: chenxutan.com/d/2624 section
// 3.4, the per-head centre, mean norm and concentration from about ten thousand captured
// tokens; zhichai.net section "破局之道" for R as the norm of the mean over the mean norm).  Per
// (layer, query head) and band f (the complex number q[f] + i q[f + 64]):
//   qbar_f = mean_n q_{n,f},   E|q_f| = mean_n |q_{n,f}|,   R_f = |qbar_f| / E|q_f|  (0 if E|q_f| = 0).
//
// One block of four waves per head; HBM-bound (every captured value is read once).  An 8-lane
// group reads one query row: lane c takes bands 8c..8c+7, i.e. 16 (bf16) or 32 (fp32)
// contiguous bytes of the real half and the same of the imaginary half, so each half-row is one
// 128- or 256-byte segment.  The eight groups of a wave take rows 8w + g, 8w + g + 32, ...; four
// rows per lane are added in fp32 (|q_f| itself in fp32 from the exact input values), then into
// fp64 sums, which are combined in a fixed order: row groups by butterfly, then the waves in
// order.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

constexpr int kCalibThreads = 256;

// Bands 8c .. 8c+7 of one query row: 16 contiguous bytes of the real half and 16 of the
// imaginary half for bf16 (fp32 rows take two 16-byte words per half).
template <bool BF16>
__device__ __forceinline__ void load_band8(const char *__restrict__ row, int c, float (&re)[8], float (&im)[8])
{
    if (BF16) {
        const uint4 a = *(const uint4 *)(row + c * 16);           // dims 8c .. 8c+7
        const uint4 b = *(const uint4 *)(row + 128 + c * 16);     // dims 64 + 8c ..
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            re[2 * i] = bf16_lo(aw[i]);
            re[2 * i + 1] = bf16_hi(aw[i]);
            im[2 * i] = bf16_lo(bw[i]);
            im[2 * i + 1] = bf16_hi(bw[i]);
        }
    } else {
        const float4 a0 = *(const float4 *)(row + c * 32), a1 = *(const float4 *)(row + c * 32 + 16);
        const float4 b0 = *(const float4 *)(row + 256 + c * 32), b1 = *(const float4 *)(row + 256 + c * 32 + 16);
        re[0] = a0.x; re[1] = a0.y; re[2] = a0.z; re[3] = a0.w; re[4] = a1.x; re[5] = a1.y; re[6] = a1.z; re[7] = a1.w;
        im[0] = b0.x; im[1] = b0.y; im[2] = b0.z; im[3] = b0.w; im[4] = b1.x; im[5] = b1.y; im[6] = b1.z; im[7] = b1.w;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kCalibThreads) void calib_stats_kernel(const void *__restrict__ q, int n_cal,
                                                                    float *__restrict__ qc, float *__restrict__ qn,
                                                                    float *__restrict__ rb)
{
    constexpr int RB = BF16 ? 256 : 512;       // row bytes
    constexpr int NW = kCalibThreads / 64;
    constexpr int U = 4;                       // rows per lane in flight
    __shared__ double red[NW][3][TRIA_HALF];
    const int hh = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int c = lane & 7, g = lane >> 3;     // lane c of row group g (8 groups per wave)
    const char *base = (const char *)q + (size_t)hh * n_cal * RB;
    double sr[8], si[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sr[e] = si[e] = sn[e] = 0.0;
    const int stride = NW * 8;
    int n = wid * 8 + g;
    // U rows per lane in flight; their values are added in fp32 (U terms), then once into fp64
    for (; n + (U - 1) * stride < n_cal; n += U * stride) {
        float re[U][8], im[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load_band8<BF16>(base + (size_t)(n + u * stride) * RB, c, re[u], im[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float ar = 0.f, ai = 0.f, an = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float x = re[u][e], y = im[u][e];
                ar += x;
                ai += y;
                an += __builtin_sqrtf(fmaf(x, x, y * y));
            }
            sr[e] += (double)ar;
            si[e] += (double)ai;
            sn[e] += (double)an;
        }
    }
    for (; n < n_cal; n += stride) {
        float re[8], im[8];
        load_band8<BF16>(base + (size_t)n * RB, c, re, im);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sr[e] += (double)re[e];
            si[e] += (double)im[e];
            sn[e] += (double)__builtin_sqrtf(fmaf(re[e], re[e], im[e] * im[e]));
        }
    }
    // row groups 0..7 of the wave: butterfly over lane bits 3..5 (fixed order)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int o = 8; o < 64; o <<= 1) {
            sr[e] += __shfl_xor(sr[e], o, 64);
            si[e] += __shfl_xor(si[e], o, 64);
            sn[e] += __shfl_xor(sn[e], o, 64);
        }
    }
    if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[wid][0][8 * c + e] = sr[e];
            red[wid][1][8 * c + e] = si[e];
            red[wid][2][8 * c + e] = sn[e];
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

hipError_t launch_calib_stats(tria_dtype dt, const void *q, int n_heads, int n_cal, float *qc, float *qn, float *rb,
                              hipStream_t st)
{
    KernelTimer timer(TRIA_TIMER_CALIB, st);
    if (dt == TRIA_BF16)
        calib_stats_kernel<true><<<n_heads, kCalibThreads, 0, st>>>(q, n_cal, qc, qn, rb);
    else
        calib_stats_kernel<false><<<n_heads, kCalibThreads, 0, st>>>(q, n_cal, qc, qn, rb);
    return hipGetLastError();
}

}  // namespace tria
