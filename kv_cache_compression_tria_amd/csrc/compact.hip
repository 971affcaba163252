// compact.hip -- in-place, order-preserving compaction of K, V and positions (gfx950): one block
// per stream (the method and its ordering argument are in compact_stream.cuh), and the
// tile-parallel form that tria_prune takes.
#include <mutex>

#include "compact_stream.cuh"
#include "tria_internal.h"

namespace tria {

template <int RV>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                  int32_t *__restrict__ pos,
                                                                  const int32_t *__restrict__ kept, int N, int nk)
{
    compact_stream<RV, kCompactThreads, kCompactRows>(blockIdx.x, k, v, pos, kept, N, nk);
}

hipError_t launch_compact(tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *kept, int n_streams,
                          int N, int B, hipStream_t st)
{
    const int nk = B < N ? B : N;
    KernelTimer timer(TRIA_TIMER_COMPACT, st);
    if (dt == TRIA_BF16)
        compact_kernel<16><<<n_streams, kCompactThreads, 0, st>>>((uint4 *)k, (uint4 *)v, pos, kept, N, nk);
    else
        compact_kernel<32><<<n_streams, kCompactThreads, 0, st>>>((uint4 *)k, (uint4 *)v, pos, kept, N, nk);
    return hipGetLastError();
}

// The tile-parallel compaction: one block of kCompactThreads per tile of T destination rows, the
// tiles of every stream in flight at once (one block per stream leaves CUs idle when there are
// about as many streams as CUs, and one CU moves a stream at a small fraction of the chip's rate;
// with many streams the tiles still keep more rows in flight than sequential per-stream passes).
//
// Tile q of a stream writes rows [qT, qT + T) and reads rows kept[i] >= i of the same index range
// (chenxutan.com/d/2624 section 4.2: the cache is indexed by the sorted kept indices).  Its
// destinations lie below the sources of every later tile of the stream, and it holds its own
// sources in registers before it writes; but its destinations may hold sources of earlier tiles
// (kept[i] >= qT for some i < qT).  So every tile publishes a flag as soon as its sources are in
// registers, before it waits for anything, and writes only once every earlier tile of its stream
// has published.  Blocks take their tile from a counter, in (stream, tile) order: the earlier
// tiles of a stream belong to blocks that are already running and publish without waiting, so
// every wait ends.  sync: [0] the counter, [1 + s tiles + q] the flags, all zero at launch (the
// selection before it clears them).  A wait that runs past its bound sets bit 4 of *err and the
// tile writes anyway (the step then reports a device error).
constexpr int kTileSpinLimit = 1 << 20;

template <int RV, int T>
__global__ __launch_bounds__(kCompactThreads) void compact_tiles_kernel(uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                        int32_t *__restrict__ pos,
                                                                        const int32_t *__restrict__ kept, int N,
                                                                        int nk, int tiles, int n_items,
                                                                        int *__restrict__ sync, int *__restrict__ err)
{
    constexpr int NT = kCompactThreads;
    constexpr int PER = T * RV / NT;                  // 16-byte words per thread per tensor
    static_assert(PER * NT == T * RV && T <= NT, "tile shape");
    __shared__ int s_item;
    if (threadIdx.x == 0) s_item = atomicAdd(&sync[0], 1);
    __syncthreads();
    const int item = s_item;
    if (item >= n_items) {                            // the counter was not cleared: nothing is safe to move
        if (threadIdx.x == 0) atomicOr(err, 4);
        return;
    }
    const int sid = item / tiles, q = item - sid * tiles;
    const int i0 = q * T;
    uint4 *kb = k + (size_t)sid * N * RV;
    uint4 *vb = v + (size_t)sid * N * RV;
    int32_t *pb = pos ? pos + (size_t)sid * N : nullptr;
    const int32_t *kp = kept + (size_t)sid * nk;
    // every kept index first (one memory latency for all of them), then every row
    int src[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int r = i0 + (int)(threadIdx.x + m * NT) / RV;
        src[m] = r < nk ? kp[r] : r;
    }
    const int pr = i0 + (int)threadIdx.x;
    const int psrc = pb && threadIdx.x < T && pr < nk ? kp[pr] : pr;
    uint4 bk[PER], bv[PER];
    bool mv[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int idx = threadIdx.x + m * NT;
        const int r = i0 + idx / RV, c = idx % RV;
        const int s = src[m];
        mv[m] = r < nk && s > r && s < N;             // valid kept[] has r <= s < N; s == r stays
        if (mv[m]) {
            const u32x4 a = __builtin_nontemporal_load((const u32x4 *)&kb[(size_t)s * RV + c]);
            const u32x4 b = __builtin_nontemporal_load((const u32x4 *)&vb[(size_t)s * RV + c]);
            bk[m] = make_uint4(a[0], a[1], a[2], a[3]);
            bv[m] = make_uint4(b[0], b[1], b[2], b[3]);
        }
    }
    int32_t pv = 0;
    bool pmv = false;
    if (pb && threadIdx.x < T && pr < nk && psrc > pr && psrc < N) {
        pmv = true;
        pv = pb[psrc];
    }
#pragma unroll
    for (int m = 0; m < PER; ++m)
        if (mv[m]) {
            hold(bk[m]);
            hold(bv[m]);
        }
    if (pmv) hold((uint32_t)pv);
    __syncthreads();   // every source row of this tile is in registers
    int *flag = sync + 1 + (size_t)sid * tiles;
    if (threadIdx.x == 0) __hip_atomic_store(&flag[q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int j = threadIdx.x; j < q; j += NT) {
        int n = 0;
        while (__hip_atomic_load(&flag[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            if (++n > kTileSpinLimit) {
                atomicOr(err, 4);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();   // every earlier tile of the stream holds its sources
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        if (mv[m]) {
            const int idx = threadIdx.x + m * NT;
            const int r = i0 + idx / RV, c = idx % RV;
            __builtin_nontemporal_store(u32x4{bk[m].x, bk[m].y, bk[m].z, bk[m].w}, (u32x4 *)&kb[(size_t)r * RV + c]);
            __builtin_nontemporal_store(u32x4{bv[m].x, bv[m].y, bv[m].z, bv[m].w}, (u32x4 *)&vb[(size_t)r * RV + c]);
        }
    }
    if (pmv) pb[i0 + threadIdx.x] = pv;
}

namespace {
std::mutex g_cu_mu;
int g_cus[64] = {};
// compute units of the current device (looked up once per device), 0 if unknown
int device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(g_cu_mu);
    if (!g_cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}
}  // namespace

int compact_tiles_per_stream(int B) { return (B + kTileCompactRows - 1) / kTileCompactRows; }

// Measured on MI355X against one fused selection-and-compaction block per stream, in the same
// process on the same cache: with fewer streams than two per CU one block per stream leaves CUs
// idle (Qwen3-8B batch 1: 0.231 -> 0.021 + 0.166 ms); with many streams of up to 8192 keys the tiles
// still move rows faster than the per-stream passes even with the selection as a launch of its own
// (Qwen3-8B batch 64: 7.42 -> 0.39 + 6.43 ms); with many long streams the fused kernel, whose
// selection hides behind other blocks' rows, stays ahead (Qwen3-32B: 2.63 against 0.25 + 2.43 ms).
bool compact_tiles_applies(int n_streams, int N, int B)
{
    if (B >= N || n_streams <= 0) return false;
    if ((long long)n_streams * compact_tiles_per_stream(B) > 0x7fffffffLL) return false;
    const int cus = device_cus();
    return cus > 0 && (n_streams < 2 * cus || N <= kTileCompactShortKeys);
}

size_t compact_tiles_sync_words(int n_streams, int B) { return 1 + (size_t)n_streams * compact_tiles_per_stream(B); }

hipError_t launch_compact_tiles(tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *kept, int n_streams,
                                int N, int B, int *sync, int *err, hipStream_t st)
{
    if (B >= N) return hipErrorInvalidValue;
    const int tiles = compact_tiles_per_stream(B);
    const long long items = (long long)n_streams * tiles;
    if (items > 0x7fffffffLL) return hipErrorInvalidValue;
    KernelTimer timer(TRIA_TIMER_COMPACT, st);
    if (dt == TRIA_BF16)
        compact_tiles_kernel<16, kTileCompactRows><<<(unsigned)items, kCompactThreads, 0, st>>>(
            (uint4 *)k, (uint4 *)v, pos, kept, N, B, tiles, (int)items, sync, err);
    else
        compact_tiles_kernel<32, kTileCompactRows><<<(unsigned)items, kCompactThreads, 0, st>>>(
            (uint4 *)k, (uint4 *)v, pos, kept, N, B, tiles, (int)items, sync, err);
    return hipGetLastError();
}

}  // namespace tria
