// copy.hip -- a plain streaming device copy (gfx950; instrumentation).  It computes nothing of the
// method: it is the read + write rate the benchmark reports beside the prune step's, the ceiling of
// what the in-place compaction (which reads and writes every moved row) can reach.
//
// Grid-stride over 16-byte words; each lane issues eight non-temporal loads before its eight
// stores, and the grid is capped at 16384 blocks of 256 threads (measured on MI355X: 5.3-5.4 TB/s
// read + write for 8 GiB from 8192 blocks up; fewer blocks or four loads in flight are slower).
#include <algorithm>

#include "tria_internal.h"

namespace tria {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyDepth = 8;          // loads in flight per lane
constexpr int kCopyMaxBlocks = 16384;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4 *__restrict__ s, u32x4 *__restrict__ d,
                                                            size_t n16)
{
    const size_t stride = (size_t)gridDim.x * kCopyThreads * kCopyDepth;
    for (size_t base = (size_t)blockIdx.x * kCopyThreads * kCopyDepth + threadIdx.x; base < n16; base += stride) {
        u32x4 r[kCopyDepth];
#pragma unroll
        for (int u = 0; u < kCopyDepth; ++u) {
            const size_t i = base + (size_t)u * kCopyThreads;
            if (i < n16) r[u] = __builtin_nontemporal_load(&s[i]);
        }
#pragma unroll
        for (int u = 0; u < kCopyDepth; ++u) {
            const size_t i = base + (size_t)u * kCopyThreads;
            if (i < n16) __builtin_nontemporal_store(r[u], &d[i]);
        }
    }
}

hipError_t launch_copy(const void *src, void *dst, size_t n16, hipStream_t st)
{
    const size_t per_block = (size_t)kCopyThreads * kCopyDepth;
    const size_t blocks = std::min<size_t>((n16 + per_block - 1) / per_block, kCopyMaxBlocks);
    copy_kernel<<<(unsigned)blocks, kCopyThreads, 0, st>>>((const u32x4 *)src, (u32x4 *)dst, n16);
    return hipGetLastError();
}

}  // namespace tria
