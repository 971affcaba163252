// common.cuh -- small device helpers shared by the HIP kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tria {

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Make sure a loaded value has arrived in registers (forces the wait on its load) without
// emitting any instruction of our own.
__device__ __forceinline__ void hold(uint32_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void hold(const uint4 &x)
{
    asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float wave_min(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at most 1024).
// `scratch` must hold NT/64 + 1 words of LDS.  Returns the exclusive prefix; *total gets the
// block total.  Contains barriers: every thread of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t *scratch, uint32_t *total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t incl = wave_incl_scan(x);
    if (lane == 63) scratch[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        uint32_t v = lane < NW ? scratch[lane] : 0u;
        uint32_t vi = wave_incl_scan(v);
        if (lane < NW) scratch[lane] = vi - v;
        if (lane == NW - 1) scratch[NW] = vi;
    }
    __syncthreads();
    uint32_t r = scratch[wid] + incl - x;
    *total = scratch[NW];
    __syncthreads();
    return r;
}

}  // namespace tria
