// select.hip -- top-B selection per stream (gfx950).
//
// Keep the B keys with the largest final score, ties to the lower index, written in ascending
// index order (chenxutan.com/d/2624 section 4.2: top-k of the scores, then sorted to keep the
// cache order).  One workgroup per stream:
//   1. map each score to an order-preserving unsigned key (-0 folded onto +0);
//   2. four 8-bit radix passes with a 256-bin LDS histogram find the B-th largest key T and
//      how many keys equal to T must be taken (k);
//   3. one ordered sweep over the stream writes every index with key > T, and the first k
//      indices with key == T: output slot = #(key > T before j) + min(#(key == T before j), k).
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

__device__ __forceinline__ uint32_t order_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0u) u = 0u;                       // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool IN_LDS>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(const float *__restrict__ F, int N, int B,
                                                                int32_t *__restrict__ kept)
{
    constexpr int NT = kSelectThreads;
    extern __shared__ uint32_t keys[];                // [N] when IN_LDS
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_scratch[NT / 64 + 1];
    __shared__ uint32_t s_prefix, s_k;

    const int sid = blockIdx.x;
    const float *f = F + (size_t)sid * N;
    int32_t *out = kept + (size_t)sid * B;            // B < N on this path
    if (IN_LDS) {
        for (int j = threadIdx.x; j < N; j += NT) keys[j] = order_key(f[j]);
        __syncthreads();
    }
    auto key_at = [&](int j) -> uint32_t { return IN_LDS ? keys[j] : order_key(f[j]); };

    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)B;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
        __syncthreads();
        for (int j = threadIdx.x; j < N; j += NT) {
            const uint32_t u = key_at(j);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending); find the bin where the count of
            // larger-or-equal keys first reaches k
            const int lane = threadIdx.x;
            uint32_t c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
            const uint32_t local = c[0] + c[1] + c[2] + c[3];
            const uint32_t incl = wave_incl_scan(local);
            uint32_t excl = incl - local;
            if (excl < k && k <= incl) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (excl + c[i] >= k) {
                        s_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
                        s_k = k - excl;
                        break;
                    }
                    excl += c[i];
                }
            }
        }
        __syncthreads();
        prefix = s_prefix;
        k = s_k;
        mask |= 255u << shift;
    }
    const uint32_t T = prefix;   // the B-th largest key; k of the keys equal to T are kept

    uint32_t gt_run = 0u, eq_run = 0u;
    for (int base = 0; base < N; base += NT) {
        const int j = base + threadIdx.x;
        uint32_t gt = 0u, eq = 0u;
        if (j < N) {
            const uint32_t u = key_at(j);
            gt = u > T;
            eq = u == T;
        }
        uint32_t total;
        const uint32_t before = block_excl_scan<NT>(gt | (eq << 16), scan_scratch, &total);
        const uint32_t gt_before = gt_run + (before & 0xffffu);
        const uint32_t eq_before = eq_run + (before >> 16);
        uint32_t slot = 0xffffffffu;
        if (gt) slot = gt_before + min(eq_before, k);
        else if (eq && eq_before < k) slot = gt_before + eq_before;
        if (slot < (uint32_t)B) out[slot] = j;      // always true for a valid histogram walk
        gt_run += total & 0xffffu;
        eq_run += total >> 16;
    }
}

__global__ void identity_kernel(int32_t *__restrict__ kept, int n_streams, int N)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (size_t)n_streams * N) kept[i] = (int32_t)(i % N);
}

hipError_t launch_select(const float *F, int n_streams, int N, int B, int32_t *kept, hipStream_t st)
{
    if (B >= N) {
        const size_t n = (size_t)n_streams * N;
        identity_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(kept, n_streams, N);
        return hipGetLastError();
    }
    if (N <= kSelectLdsKeys) {
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void *)select_kernel<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kSelectLdsKeys * 4);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        select_kernel<true><<<n_streams, kSelectThreads, (size_t)N * 4, st>>>(F, N, B, kept);
    } else {
        select_kernel<false><<<n_streams, kSelectThreads, 0, st>>>(F, N, B, kept);
    }
    return hipGetLastError();
}

}  // namespace tria
