// noalloc.hip -- tria_prune_static: the prune step with its scratch in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array `scratch` lives in the library's code object: every device the library runs on holds
// its own copy (TRIA_STATIC_WORKSPACE_BYTES) from the library's load until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per device and kept.
//
// Layout of the array: [0, 256) the step's status word (the OR of the error words of every chunk),
// [256, end) the workspace of tria_prune for one chunk of sequences.  A call whose workspace does
// not fit is split into chunks of whole sequences, pruned one after the other on the caller's
// stream (the scratch is reused in stream order).  Every region a kernel reads is written earlier
// in the same call (the error and arrival words are cleared by the step's first kernel), so the
// contents left by the previous call do not matter; calls that overlap on one device (different
// streams, or threads) share the array and race.
#include <mutex>

#include "tria_internal.h"

static __device__ __align__(256) unsigned char scratch[TRIA_STATIC_WORKSPACE_BYTES];

namespace {

constexpr size_t kStaticBytes = TRIA_STATIC_WORKSPACE_BYTES;
constexpr size_t kStatusBytes = 256;
static_assert(kStaticBytes % 256 == 0 && kStaticBytes > kStatusBytes, "static workspace size");

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};   // device address of `scratch` per device, once looked up

// The device address of the static array on the current device (looked up on the first call on
// that device), or null on failure.
void *scratch_address(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

// status = err (first chunk) or status |= err (later chunks): the step's status word collects
// every chunk's error bits, since each chunk's score clears its own error word
__global__ void fold_status_kernel(int *__restrict__ status, const int *__restrict__ err, int first)
{
    if (threadIdx.x == 0) *status = first ? *err : (*status | *err);
}

}  // namespace

extern "C" tria_status tria_prune_static(const tria_calib *c, tria_dtype dt, void *k, void *v, int32_t *pos,
                                         const int32_t *t, int n_seq, int N, int B, float *F, int32_t *kept,
                                         unsigned flags, void **ws_used, void *stream)
{
    if (ws_used) *ws_used = nullptr;
    if (!c || !k || !v || !t || !F || !kept || n_seq <= 0 || N <= 0 || B <= 0) return TRIA_E_INVALID;
    if (dt != TRIA_BF16 && dt != TRIA_F32) return TRIA_E_INVALID;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return TRIA_E_INVALID;
    // the largest chunk of whole sequences whose workspace fits the array
    const size_t room = kStaticBytes - kStatusBytes;
    if (tria_prune_workspace_bytes(c, dt, 1, N, B, flags) == 0) return TRIA_E_INVALID;
    if (tria_prune_workspace_bytes(c, dt, 1, N, B, flags) > room) return TRIA_E_WORKSPACE;
    int lo = 1, hi = n_seq;
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        const size_t need = tria_prune_workspace_bytes(c, dt, mid, N, B, flags);
        if (need != 0 && need <= room) lo = mid;
        else hi = mid - 1;
    }
    const int chunk = lo;
    void *base = scratch_address(dev);
    if (!base) return TRIA_E_DEVICE;
    int *status = (int *)base;
    void *ws = (char *)base + kStatusBytes;
    hipStream_t st = (hipStream_t)stream;
    const size_t per_seq = (size_t)c->L * c->Hkv;                   // streams per sequence
    const size_t row = (size_t)TRIA_D * (dt == TRIA_BF16 ? 2 : 4);  // bytes per K / V row
    const size_t nk = (size_t)(B < N ? B : N);
    for (int s0 = 0; s0 < n_seq; s0 += chunk) {
        const int ns = n_seq - s0 < chunk ? n_seq - s0 : chunk;
        const size_t st0 = (size_t)s0 * per_seq;                     // first stream of the chunk
        tria_status r = tria_prune(c, dt, (char *)k + st0 * N * row, (char *)v + st0 * N * row,
                                   pos ? pos + st0 * N : nullptr, t + s0, ns, N, B, F + st0 * N, kept + st0 * nk,
                                   flags, ws, room, stream);
        if (r != TRIA_OK) return r;
        // every score workspace starts with its error word
        fold_status_kernel<<<1, 64, 0, st>>>(status, (const int *)ws, s0 == 0);
        if (hipGetLastError() != hipSuccess) return TRIA_E_DEVICE;
    }
    if (ws_used) *ws_used = base;
    return TRIA_OK;
}
