// decode.hip -- appending newly generated K/V rows to a fixed-capacity cache (gfx950).
//
// The decode loop around the prune step (TriAttention pages: the 10100.com article, section
// "TriAttention方法", and watermelonwater.tech "TriAttention 方案设计" item 4: prune once every 128
// generated tokens; chenxutan.com/d/2624 section 4, the attention layer that appends each new
// token's K/V to the cache and prunes it back to the budget).  Each stream's cache holds up to
// `cap` rows; the rows of the newest tokens go in at row `len` of every stream.  A plain
// coalesced copy: one 16-byte word per thread and tensor.
#include "common.cuh"
#include "tria_internal.h"

namespace tria {

constexpr int kAppendThreads = 256;

template <int RV>   // 16-byte words per row: 16 for bf16, 32 for fp32 (head_dim 128)
__global__ __launch_bounds__(kAppendThreads) void append_kernel(uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                int32_t *__restrict__ pos, const uint4 *__restrict__ kn,
                                                                const uint4 *__restrict__ vn,
                                                                const int32_t *__restrict__ pn, int cap, int len,
                                                                int n_new, long long total)
{
    const long long i = (long long)blockIdx.x * kAppendThreads + threadIdx.x;   // word of the new rows
    if (i >= total) return;
    const long long row = i / RV;              // row of the new-rows tensor [streams][n_new]
    const int c = (int)(i - row * RV);
    const long long s = row / n_new;
    const int r = (int)(row - s * n_new);
    const size_t dst = ((size_t)s * cap + len + r) * RV + c;
    k[dst] = kn[i];
    v[dst] = vn[i];
    if (pos && c == 0) pos[(size_t)s * cap + len + r] = pn[row];
}

hipError_t launch_append(tria_dtype dt, void *k, void *v, int32_t *pos, int n_streams, int cap, int len,
                         const void *kn, const void *vn, const int32_t *pn, int n_new, hipStream_t st)
{
    const int RV = dt == TRIA_BF16 ? 16 : 32;
    const long long total = (long long)n_streams * n_new * RV;
    const long long blocks = (total + kAppendThreads - 1) / kAppendThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (dt == TRIA_BF16)
        append_kernel<16><<<(unsigned)blocks, kAppendThreads, 0, st>>>((uint4 *)k, (uint4 *)v, pos, (const uint4 *)kn,
                                                                       (const uint4 *)vn, pn, cap, len, n_new, total);
    else
        append_kernel<32><<<(unsigned)blocks, kAppendThreads, 0, st>>>((uint4 *)k, (uint4 *)v, pos, (const uint4 *)kn,
                                                                       (const uint4 *)vn, pn, cap, len, n_new, total);
    return hipGetLastError();
}

}  // namespace tria
