// compact.hip -- in-place, order-preserving compaction of K, V and positions (gfx950): one block
// per stream (the method and its ordering argument are in compact_stream.cuh).
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

}  // namespace tria
