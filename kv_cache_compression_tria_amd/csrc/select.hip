// select.hip -- top-B selection per stream (gfx950).
//
// Keep the B keys with the largest final score, ties to the lower index, written in ascending
// index order (chenxutan.com/d/2624 section 4.2: top-k of the scores, then sorted to keep the
// cache order).  One workgroup of 16 waves per stream:
//   1. map each score to an order-preserving unsigned key (-0 folded onto +0), kept in LDS;
//   2. three radix digits (11, 11 and 10 bits) find the B-th largest key T and how many of the
//      keys equal to T must be taken (k): a histogram of digit 0 over all keys picks a bin, the
//      keys of that bin are copied to a candidate list, and digits 1 and 2 are resolved over the
//      candidates only.  Final scores cluster in a few exponent values, so the top digit piles
//      onto few bins: each wave first counts its heavy bins with one ballot per bin and a single
//      atomic, and only the scattered rest use per-lane atomics;
//   3. wave w owns the contiguous key range [w*N/16, (w+1)*N/16): it counts its keys > T and
//      == T, one scan over the 16 wave totals gives its output base, and it writes every index
//      with key > T and the first k indices with key == T (in index order) at
//      slot = #(key > T before j) + min(#(key == T before j), k).
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

__device__ __forceinline__ uint32_t order_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0u) u = 0u;                       // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Add the lanes' bins (where `live`) to the LDS histogram.  Bins shared by at least 8 lanes are
// counted with one atomic per bin (at most four such bins per call), the rest lane by lane.
__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t bin, bool live)
{
    const int lane = threadIdx.x & 63;
    uint64_t todo = __ballot(live);
    for (int r = 0; r < 4 && todo; ++r) {
        const int leader = __builtin_ctzll(todo);
        const uint32_t b = __builtin_amdgcn_readlane(bin, leader);
        const uint64_t same = __ballot(live && bin == b);
        const int n = __builtin_popcountll(same);
        if (n < 8) break;
        if (lane == leader) atomicAdd(&hist[b], (uint32_t)n);
        todo &= ~same;
    }
    if ((todo >> lane) & 1u) atomicAdd(&hist[bin], 1u);
}

constexpr int kBins0 = 2048;      // digit 0: the top 11 bits of the order key
constexpr int kCand = 4096;       // candidate list (keys of the chosen digit-0 bin), in LDS
static_assert(kSelectLdsKeys * 4 + (kBins0 + kCand) * 4 + 512 <= 160 * 1024, "select LDS exceeds a CU's 160 KB");

template <bool IN_LDS>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(const float *__restrict__ F, int N, int B,
                                                                int32_t *__restrict__ kept)
{
    constexpr int NT = kSelectThreads;
    constexpr int NW = NT / 64;
    extern __shared__ uint32_t keys[];                // [N] when IN_LDS
    __shared__ uint32_t hist[kBins0];
    __shared__ uint32_t cand[kCand];
    __shared__ uint32_t wgt[NW], weq[NW];
    __shared__ uint32_t s_prefix, s_k, s_ncand;

    const int sid = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const float *f = F + (size_t)sid * N;
    int32_t *out = kept + (size_t)sid * B;            // B < N on this path
    if (IN_LDS) {
        // eight independent loads in flight per thread (16-byte loads when the rows allow)
        if ((N & 3) == 0 && ((uintptr_t)F & 15) == 0) {
            const float4 *f4 = (const float4 *)f;
            const int n4 = N >> 2;
            for (int base = 0; base < n4; base += 8 * NT) {
                float4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = base + u * NT + threadIdx.x;
                    v[u] = i < n4 ? f4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = base + u * NT + threadIdx.x;
                    if (i < n4)
                        *(uint4 *)&keys[4 * i] = make_uint4(order_key(v[u].x), order_key(v[u].y), order_key(v[u].z),
                                                            order_key(v[u].w));
                }
            }
        } else {
            for (int base = 0; base < N; base += 8 * NT) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = base + u * NT + threadIdx.x;
                    v[u] = j < N ? f[j] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = base + u * NT + threadIdx.x;
                    if (j < N) keys[j] = order_key(v[u]);
                }
            }
        }
        __syncthreads();
    }
    auto key_at = [&](int j) -> uint32_t { return IN_LDS ? keys[j] : order_key(f[j]); };

    // digit 0 = bits 31..21 over every key; the keys of the chosen digit-0 bin are then copied
    // to a candidate list (when they fit) and digits 1 (bits 20..10) and 2 (bits 9..0) are
    // resolved over the candidates alone
    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)B;
    auto find_bin = [&](int shift, int nbins) {
        __syncthreads();
        if (wid == 0) {
            // lane l owns bins nbins-1-l*per .. nbins-per-l*per (descending); find the bin where
            // the count of larger-or-equal keys first reaches k
            const int per = nbins / 64;
            uint32_t local = 0u;
            for (int i = 0; i < per; ++i) local += hist[nbins - 1 - lane * per - i];
            const uint32_t incl = wave_incl_scan(local);
            uint32_t excl = incl - local;
            if (excl < k && k <= incl) {
                for (int i = 0; i < per; ++i) {
                    const int bin = nbins - 1 - lane * per - i;
                    const uint32_t c = hist[bin];
                    if (excl + c >= k) {
                        s_prefix = prefix | ((uint32_t)bin << shift);
                        s_k = k - excl;
                        break;
                    }
                    excl += c;
                }
            }
        }
        __syncthreads();
        prefix = s_prefix;
        k = s_k;
    };
    auto clear_hist = [&](int nbins) {
        for (int i = threadIdx.x; i < nbins; i += NT) hist[i] = 0u;
        __syncthreads();
    };

    clear_hist(kBins0);
    for (int base = 0; base < N; base += NT) {       // uniform trip count: ballots see the whole wave
        const int j = base + threadIdx.x;
        const uint32_t u = j < N ? key_at(j) : 0u;
        hist_add(hist, u >> 21, j < N);
    }
    find_bin(21, kBins0);
    mask = 0xffe00000u;

    // candidates: keys whose digit 0 matches
    if (threadIdx.x == 0) s_ncand = 0u;
    __syncthreads();
    const bool listed = hist[prefix >> 21] <= (uint32_t)kCand;   // read before the histogram is reused
    if (listed) {
        for (int base = 0; base < N; base += NT) {
            const int j = base + threadIdx.x;
            const uint32_t u = j < N ? key_at(j) : 0u;
            const bool m = j < N && (u & mask) == prefix;
            const uint64_t bal = __ballot(m);
            uint32_t wbase = 0u;
            if (lane == 0 && bal) wbase = atomicAdd(&s_ncand, (uint32_t)__builtin_popcountll(bal));
            wbase = __builtin_amdgcn_readfirstlane(wbase);
            if (m)
                cand[wbase + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = u;
        }
    }
    __syncthreads();
    const int ncand = (int)s_ncand;
    for (int d = 1; d <= 2; ++d) {
        const int shift = d == 1 ? 10 : 0;
        const int nbins = d == 1 ? 2048 : 1024;
        clear_hist(nbins);
        if (listed) {
            for (int base = 0; base < ncand; base += NT) {
                const int i = base + threadIdx.x;
                const uint32_t u = i < ncand ? cand[i] : 0u;
                hist_add(hist, (u >> shift) & (uint32_t)(nbins - 1), i < ncand && (u & mask) == prefix);
            }
        } else {
            for (int base = 0; base < N; base += NT) {
                const int j = base + threadIdx.x;
                const uint32_t u = j < N ? key_at(j) : 0u;
                hist_add(hist, (u >> shift) & (uint32_t)(nbins - 1), j < N && (u & mask) == prefix);
            }
        }
        find_bin(shift, nbins);
        mask |= (uint32_t)(nbins - 1) << shift;
    }
    const uint32_t T = prefix;   // the B-th largest key; k of the keys equal to T are kept

    // ordered write: wave w walks its contiguous range in 64-key steps
    const int per = (N + NW - 1) / NW;
    const int lo = min(N, wid * per), hi = min(N, lo + per);
    uint32_t ngt = 0u, neq = 0u;
    for (int b = lo; b < hi; b += 64) {
        const int j = b + lane;
        const uint32_t u = j < hi ? key_at(j) : 0u;
        ngt += __builtin_popcountll(__ballot(j < hi && u > T));
        neq += __builtin_popcountll(__ballot(j < hi && u == T));
    }
    if (lane == 0) {
        wgt[wid] = ngt;
        weq[wid] = neq;
    }
    __syncthreads();
    uint32_t gt_run = 0u, eq_run = 0u;
    for (int w = 0; w < wid; ++w) {
        gt_run += wgt[w];
        eq_run += weq[w];
    }
    for (int b = lo; b < hi; b += 64) {
        const int j = b + lane;
        const uint32_t u = j < hi ? key_at(j) : 0u;
        const bool gt = j < hi && u > T, eq = j < hi && u == T;
        const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
        const uint32_t gt_before = gt_run + __builtin_amdgcn_mbcnt_hi((uint32_t)(mgt >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mgt, 0u));
        const uint32_t eq_before = eq_run + __builtin_amdgcn_mbcnt_hi((uint32_t)(meq >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)meq, 0u));
        uint32_t slot = 0xffffffffu;
        if (gt) slot = gt_before + min(eq_before, k);
        else if (eq && eq_before < k) slot = gt_before + eq_before;
        if (slot < (uint32_t)B) out[slot] = j;      // always true for a valid histogram walk
        gt_run += __builtin_popcountll(mgt);
        eq_run += __builtin_popcountll(meq);
    }
}

__global__ void identity_kernel(int32_t *__restrict__ kept, int n_streams, int N)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (size_t)n_streams * N) kept[i] = (int32_t)(i % N);
}

hipError_t launch_select(const float *F, int n_streams, int N, int B, int32_t *kept, hipStream_t st)
{
    KernelTimer timer(TRIA_TIMER_SELECT, st);
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
