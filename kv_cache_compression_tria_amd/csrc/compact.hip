// compact.hip -- in-place, order-preserving compaction of K, V and positions (gfx950).
//
// After selection, row i of each kept tensor takes row kept[i] (i < B) (chenxutan.com/d/2624
// section 4.2: the cache is indexed by the sorted kept indices).  kept is strictly ascending,
// so kept[i] >= i: every source lies at or after its destination.  One workgroup per stream
// walks destination tiles in order; within a tile every thread first loads all of its source
// rows into registers, the workgroup synchronises, and only then are the rows written.  A
// tile's destinations [i0, i0+T) lie below every later tile's sources (>= i0+T), and earlier
// tiles are complete, so no row is overwritten before it has been read.  Rows already in place
// (kept[i] == i) are not touched.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

template <int RV>   // 16-byte words per row: 16 for bf16, 32 for fp32 (head_dim 128)
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                  int32_t *__restrict__ pos,
                                                                  const int32_t *__restrict__ kept, int N, int nk)
{
    constexpr int T = kCompactRows;
    constexpr int PER = T * RV / kCompactThreads;     // 16-byte words per thread per tensor
    const int sid = blockIdx.x;
    uint4 *kb = k + (size_t)sid * N * RV;
    uint4 *vb = v + (size_t)sid * N * RV;
    int32_t *pb = pos ? pos + (size_t)sid * N : nullptr;
    const int32_t *kp = kept + (size_t)sid * nk;

    for (int i0 = 0; i0 < nk; i0 += T) {
        uint4 bk[PER], bv[PER];
        bool mv[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = threadIdx.x + m * kCompactThreads;
            const int r = i0 + idx / RV, c = idx % RV;
            mv[m] = false;
            if (r < nk) {
                const int s = kp[r];
                if (s != r && s > r && s < N) {       // valid kept[] has r <= s < N
                    mv[m] = true;
                    bk[m] = kb[(size_t)s * RV + c];
                    bv[m] = vb[(size_t)s * RV + c];
                }
            }
        }
        int32_t pv = 0;
        bool pmv = false;
        if (pb && threadIdx.x < T && i0 + (int)threadIdx.x < nk) {
            const int r = i0 + threadIdx.x;
            const int s = kp[r];
            if (s != r && s > r && s < N) {
                pmv = true;
                pv = pb[s];
            }
        }
        // every source value of this tile must be in registers before anyone writes
#pragma unroll
        for (int m = 0; m < PER; ++m)
            if (mv[m]) { hold(bk[m]); hold(bv[m]); }
        if (pmv) hold((uint32_t)pv);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            if (mv[m]) {
                const int idx = threadIdx.x + m * kCompactThreads;
                const int r = i0 + idx / RV, c = idx % RV;
                kb[(size_t)r * RV + c] = bk[m];
                vb[(size_t)r * RV + c] = bv[m];
            }
        }
        if (pmv) pb[i0 + threadIdx.x] = pv;
    }
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

}  // namespace tria
