// compact_stream.cuh -- the in-place, order-preserving compaction of one stream by one block
// (gfx950); used by the compaction kernel and by the prune step's fused select-and-compact kernel.
//
// After selection, row i of each kept tensor takes row kept[i] (i < B) (chenxutan.com/d/2624
// section 4.2: the cache is indexed by the sorted kept indices).  kept is strictly ascending,
// so kept[i] >= i: every source lies at or after its destination.  The block walks destination
// tiles in order; within a tile every thread first loads all of its source rows into registers,
// the block synchronises, and only then are the rows written.  A tile's destinations [i0, i0+T)
// lie below every later tile's sources (>= i0+T), and earlier tiles are complete, so no row is
// overwritten before it has been read.  Rows already in place (kept[i] == i) are not touched.
#pragma once

#include "common.cuh"

namespace tria {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The compaction of stream sid by one block of NT threads, T destination rows per tile.  RV:
// 16-byte words per row (16 for bf16, 32 for fp32; head_dim 128).  Thread x handles words x + m NT
// (m < PER) of a tile.  The kept indices of the next tile are loaded while the current tile's rows
// are in flight (a load of an index and then of the row it names would otherwise be two memory
// latencies per tile), and rows move with non-temporal loads and stores: nothing here is read again
// soon.  Every thread of the block must call it.
template <int RV, int NT, int T>
__device__ __forceinline__ void compact_stream(int sid, uint4 *__restrict__ k, uint4 *__restrict__ v,
                                               int32_t *__restrict__ pos, const int32_t *__restrict__ kept, int N,
                                               int nk)
{
    constexpr int PER = T * RV / NT;                  // 16-byte words per thread per tensor
    static_assert(PER * NT == T * RV && T <= NT, "tile shape");
    uint4 *kb = k + (size_t)sid * N * RV;
    uint4 *vb = v + (size_t)sid * N * RV;
    int32_t *pb = pos ? pos + (size_t)sid * N : nullptr;
    const int32_t *kp = kept + (size_t)sid * nk;
    // source rows of the words this thread moves in the tile at i0 (a row past nk names itself)
    int src[PER];
    int psrc = 0;
    auto fetch_sources = [&](int i0) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int r = i0 + (threadIdx.x + m * NT) / RV;
            src[m] = r < nk ? kp[r] : r;
        }
        if (pb && threadIdx.x < T) {
            const int r = i0 + threadIdx.x;
            psrc = r < nk ? kp[r] : r;
        }
    };
    fetch_sources(0);
    for (int i0 = 0; i0 < nk; i0 += T) {
        uint4 bk[PER], bv[PER];
        bool mv[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = threadIdx.x + m * NT;
            const int r = i0 + idx / RV, c = idx % RV;
            const int s = src[m];
            mv[m] = r < nk && s > r && s < N;         // valid kept[] has r <= s < N; s == r stays
            if (mv[m]) {
                const u32x4 a = __builtin_nontemporal_load((const u32x4 *)&kb[(size_t)s * RV + c]);
                const u32x4 b = __builtin_nontemporal_load((const u32x4 *)&vb[(size_t)s * RV + c]);
                bk[m] = make_uint4(a[0], a[1], a[2], a[3]);
                bv[m] = make_uint4(b[0], b[1], b[2], b[3]);
            }
        }
        int32_t pv = 0;
        bool pmv = false;
        if (pb && threadIdx.x < T) {
            const int r = i0 + threadIdx.x;
            if (r < nk && psrc > r && psrc < N) {
                pmv = true;
                pv = pb[psrc];
            }
        }
        if (i0 + T < nk) fetch_sources(i0 + T);
        // every source value of this tile must be in registers before anyone writes
#pragma unroll
        for (int m = 0; m < PER; ++m)
            if (mv[m]) {
                hold(bk[m]);
                hold(bv[m]);
            }
        if (pmv) hold((uint32_t)pv);
        __syncthreads();
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
}

}  // namespace tria
