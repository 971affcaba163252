// abi.cpp -- the extern "C" entry points: argument validation, calibration-table build,
// workspace layout and launch sequencing.  All device work is in the *.hip kernel files.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <set>
#include <utility>
#include <vector>

#include "tria_internal.h"

namespace {

constexpr unsigned kScoreFlags =
    TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE | TRIA_TRIG_WEIGHT_R | TRIA_OFFSET_MAX | TRIA_SCORE_TILED;

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// w_f / (2 pi) as an unsigned 64-bit fraction of a turn, i.e. round(w_f / (2 pi) * 2^64).
// Computed in x87 extended precision (64-bit significand): the value is below 2^62, so the
// product is accurate to well under one unit; the phase of an integer position n is then
// n * nu mod 2^64, exact in integer arithmetic.
uint64_t turn_fraction(double w)
{
    const long double two_pi = 6.283185307179586476925286766559005768L;
    long double x = (long double)w / two_pi;           // < 1/(2 pi) for w <= 1
    long double scaled = ldexpl(x, 64);
    return (uint64_t)llroundl(scaled);
}

}  // namespace

namespace tria {

hipError_t allow_dynamic_lds(const void *kernel, int bytes)
{
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;   // (kernel, device)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kernel, dev})) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.insert({kernel, dev});
    return e;
}
}

extern "C" {

const char *tria_status_string(tria_status s)
{
    switch (s) {
    case TRIA_OK: return "ok";
    case TRIA_E_INVALID: return "invalid argument";
    case TRIA_E_UNSUPPORTED: return "unsupported shape or option";
    case TRIA_E_NOMEM: return "device allocation failed";
    case TRIA_E_DEVICE: return "HIP runtime or launch error";
    case TRIA_E_NONFINITE: return "non-finite key value or score";
    case TRIA_E_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

tria_status tria_band_tables(double theta, int d, const int32_t *offsets, int n_off, double *w, double *C, double *S,
                             uint64_t *nu)
{
    if (!w || !C || !S || !nu || !(theta > 1.0) || !isfinite(theta)) return TRIA_E_INVALID;
    if (n_off < 0 || (n_off > 0 && !offsets) || (n_off == 0 && offsets)) return TRIA_E_INVALID;
    if (d != TRIA_D) return TRIA_E_UNSUPPORTED;
    std::vector<int64_t> off;
    if (n_off == 0) {
        for (int i = 0; i <= 16; ++i) off.push_back(int64_t(1) << i);
    } else {
        for (int i = 0; i < n_off; ++i) {
            if (offsets[i] < 0 || offsets[i] >= (1 << 24)) return TRIA_E_INVALID;
            off.push_back(offsets[i]);
        }
    }
    for (int f = 0; f < TRIA_HALF; ++f) {
        w[f] = (double)(float)pow(theta, -2.0 * (double)f / (double)TRIA_D);
        double c = 0.0, s = 0.0;
        for (int64_t dd : off) {            // w_f * dd is exact in fp64 (24 + 24 bits)
            c += cos(w[f] * (double)dd);
            s += sin(w[f] * (double)dd);
        }
        C[f] = c / (double)off.size();
        S[f] = s / (double)off.size();
        nu[f] = turn_fraction(w[f]);
    }
    return TRIA_OK;
}

tria_status tria_load_calib(tria_calib **out, int L, int Hq, int Hkv, int d, const float *qc,
                            const float *qn, const float *rb, double theta, const int32_t *offsets,
                            int n_off, void *stream)
{
    if (!out) return TRIA_E_INVALID;
    *out = nullptr;
    if (L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || !qc || !qn || !rb) return TRIA_E_INVALID;
    if (!(theta > 1.0) || !isfinite(theta)) return TRIA_E_INVALID;
    if (n_off < 0 || (n_off > 0 && !offsets) || (n_off == 0 && offsets)) return TRIA_E_INVALID;
    if (d != TRIA_D) return TRIA_E_UNSUPPORTED;
    if (Hq % Hkv != 0) return TRIA_E_UNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > TRIA_MAX_G) return TRIA_E_UNSUPPORTED;

    std::vector<int64_t> off;
    if (n_off == 0) {
        for (int i = 0; i <= 16; ++i) off.push_back(int64_t(1) << i);
    } else {
        for (int i = 0; i < n_off; ++i) {
            if (offsets[i] < 0 || offsets[i] >= (1 << 24)) return TRIA_E_INVALID;
            off.push_back(offsets[i]);
        }
    }
    // Per-band constants in fp64: w_f, the offset mean of exp(i w_f d), the turn fraction.
    double w[TRIA_HALF], C[TRIA_HALF], S[TRIA_HALF];
    std::vector<uint64_t> nu(TRIA_HALF);
    {
        const tria_status st = tria_band_tables(theta, d, offsets, n_off, w, C, S, nu.data());
        if (st != TRIA_OK) return st;
    }
    const size_t nh = (size_t)L * Hq;
    for (size_t i = 0; i < nh * TRIA_D; ++i)
        if (!isfinite(qc[i])) return TRIA_E_INVALID;
    for (size_t i = 0; i < nh * TRIA_HALF; ++i) {
        if (!isfinite(qn[i]) || qn[i] < 0.f) return TRIA_E_INVALID;
        if (!(rb[i] >= 0.f && rb[i] <= 1.f)) return TRIA_E_INVALID;
    }

    std::vector<double2> P(nh * TRIA_HALF);
    std::vector<float2> P32(nh * TRIA_HALF);
    std::vector<float> W(nh * TRIA_HALF);
    std::vector<float> PW(nh * TRIA_HALF * 3);   // [L][Hkv][64][3][G]: Re P, Im P, W of the group
    std::vector<double2> Qc(nh * TRIA_HALF);     // qbar_f as complex numbers
    for (size_t hh = 0; hh < nh; ++hh) {
        for (int f = 0; f < TRIA_HALF; ++f) {
            const double qr = qc[hh * TRIA_D + f], qi = qc[hh * TRIA_D + TRIA_HALF + f];
            const double pr = qr * C[f] - qi * S[f];
            const double pi = qr * S[f] + qi * C[f];
            P[hh * TRIA_HALF + f] = make_double2(pr, pi);
            Qc[hh * TRIA_HALF + f] = make_double2(qr, qi);
            P32[hh * TRIA_HALF + f] = make_float2((float)pr, (float)pi);
            W[hh * TRIA_HALF + f] = (float)((1.0 - (double)rb[hh * TRIA_HALF + f]) * (double)qn[hh * TRIA_HALF + f]);
            const size_t grp = hh / G, h = hh % G;
            float *pw = &PW[((grp * TRIA_HALF + f) * 3) * G + h];
            pw[0] = P32[hh * TRIA_HALF + f].x;
            pw[G] = P32[hh * TRIA_HALF + f].y;
            pw[2 * G] = W[hh * TRIA_HALF + f];
        }
    }

    tria_calib *c = new (std::nothrow) tria_calib();
    if (!c) return TRIA_E_NOMEM;
    c->L = L; c->Hq = Hq; c->Hkv = Hkv; c->d = d; c->G = G; c->theta = theta;
    c->n_off = (int)off.size();
    if (hipGetDevice(&c->device) != hipSuccess) { delete c; return TRIA_E_DEVICE; }
    const size_t bP = tria::align256(sizeof(double2) * P.size());
    const size_t bP32 = tria::align256(sizeof(float2) * P32.size());
    const size_t bW = tria::align256(sizeof(float) * W.size());
    const size_t bnu = tria::align256(sizeof(uint64_t) * TRIA_HALF);
    const size_t bPW = tria::align256(sizeof(float) * PW.size());
    const size_t bR = tria::align256(sizeof(float) * nh * TRIA_HALF);
    const size_t bQc = tria::align256(sizeof(double2) * nh * TRIA_HALF);
    const size_t bOff = tria::align256(sizeof(int64_t) * off.size());
    c->block_bytes = bP + bP32 + bW + bnu + bPW + bR + bQc + bOff;
    if (hipMalloc(&c->block, c->block_bytes) != hipSuccess) { delete c; return TRIA_E_NOMEM; }
    char *b = (char *)c->block;
    c->P = (double2 *)b;
    c->P32 = (float2 *)(b + bP);
    c->W = (float *)(b + bP + bP32);
    c->nu = (uint64_t *)(b + bP + bP32 + bW);
    c->PW = (float *)(b + bP + bP32 + bW + bnu);
    c->R = (float *)(b + bP + bP32 + bW + bnu + bPW);
    c->Qc = (double2 *)(b + bP + bP32 + bW + bnu + bPW + bR);
    c->off = (int64_t *)(b + bP + bP32 + bW + bnu + bPW + bR + bQc);
    hipStream_t st = (hipStream_t)stream;
    bool ok = hipStreamSynchronize(st) == hipSuccess;
    ok = ok && hipMemcpy(c->P, P.data(), sizeof(double2) * P.size(), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->P32, P32.data(), sizeof(float2) * P32.size(), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->W, W.data(), sizeof(float) * W.size(), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->nu, nu.data(), sizeof(uint64_t) * TRIA_HALF, hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->PW, PW.data(), sizeof(float) * PW.size(), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->R, rb, sizeof(float) * nh * TRIA_HALF, hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->Qc, Qc.data(), sizeof(double2) * Qc.size(), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipMemcpy(c->off, off.data(), sizeof(int64_t) * off.size(), hipMemcpyHostToDevice) == hipSuccess;
    if (!ok) {
        (void)hipFree(c->block);
        delete c;
        return TRIA_E_DEVICE;
    }
    *out = c;
    return TRIA_OK;
}

void tria_free_calib(tria_calib *c)
{
    if (!c) return;
    if (c->block) (void)hipFree(c->block);
    delete c;
}

int tria_calib_dim(const tria_calib *c, int which)
{
    if (!c) return -1;
    switch (which) {
    case 0: return c->L;
    case 1: return c->Hq;
    case 2: return c->Hkv;
    case 3: return c->d;
    case 4: return c->G;
    }
    return -1;
}

size_t tria_score_workspace_bytes(const tria_calib *c, tria_dtype dt, int n_seq, int n_keys, unsigned flags)
{
    if (!c || n_seq <= 0 || n_keys <= 0 || (dt != TRIA_BF16 && dt != TRIA_F32)) return 0;
    if ((flags & ~kScoreFlags) != 0) return 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return 0;   // the path depends on the device
    return tria::score_ws_layout(c, dt, n_seq, n_keys, flags).total;
}

tria_status tria_score(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                       const int32_t *t, int n_seq, int N, float *F, float *raw, float *stats,
                       unsigned flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!c || !k || !t || !F) return TRIA_E_INVALID;
    if (dt != TRIA_BF16 && dt != TRIA_F32) return TRIA_E_INVALID;
    if (n_seq <= 0 || N <= 0 || N > (1 << 24)) return TRIA_E_INVALID;
    if ((flags & ~kScoreFlags) != 0) return TRIA_E_INVALID;
    if ((flags & (TRIA_TRIG_WEIGHT_R | TRIA_OFFSET_MAX)) && (flags & (TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE)))
        return TRIA_E_UNSUPPORTED;
    if ((flags & TRIA_OFFSET_MAX) && (dt != TRIA_BF16 || c->n_off > tria::kMaxdOffsetsLimit)) return TRIA_E_UNSUPPORTED;
    if ((flags & (TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE)) && !pos) return TRIA_E_INVALID;
    if ((size_t)n_seq * c->L * c->Hkv > (size_t)0x7fffffff) return TRIA_E_INVALID;
    if (!aligned(k, 16) || !aligned(F, 4) || (raw && !aligned(raw, 4)) || (stats && !aligned(stats, 4)) ||
        (pos && !aligned(pos, 4)))
        return TRIA_E_INVALID;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return TRIA_E_INVALID;
    tria_score_ws lay = tria::score_ws_layout(c, dt, n_seq, N, flags);
    if (!ws || ws_bytes < lay.total || !aligned(ws, 256)) return TRIA_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    char *w = (char *)ws;
    // bf16 keys on the matrix cores rotate the queries in their own prologue kernel; the other paths
    // get them from the rotation kernel.  Both clear the error word first (no memset node: safe
    // under graph capture).
    // (pre-RoPE bf16 keys on the staged clusters, lay.rot, take the prologue too)
    const bool mfma = dt == TRIA_BF16 && (lay.rot || !(flags & (TRIA_PER_KEY_PHASE | TRIA_KEYS_PRE_ROPE)));
    float *qrot = mfma ? nullptr : (float *)(w + lay.qrot_off);
    if (!mfma && tria::launch_rotate(c, t, n_seq, qrot, (int *)(w + lay.err_off), (flags & TRIA_TRIG_WEIGHT_R) != 0,
                                     st) != hipSuccess)
        return TRIA_E_DEVICE;
    if (tria::launch_score(c, dt, k, pos, t, n_seq, N, qrot, F, raw, stats, flags, lay, w, st) != hipSuccess)
        return TRIA_E_DEVICE;
    return TRIA_OK;
}

tria_status tria_score_check(const void *ws, size_t ws_bytes, void *stream)
{
    (void)ws_bytes;
    if (!ws) return TRIA_E_INVALID;
    // Every score workspace layout starts with the non-finite flag (one int at offset 0).
    int flag = 0;
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(&flag, ws, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return TRIA_E_DEVICE;
    if (hipStreamSynchronize(st) != hipSuccess) return TRIA_E_DEVICE;
    if (flag & ~1) return TRIA_E_DEVICE;   // a timed-out wait (2: stream cluster, 4: tile compaction)
    return flag ? TRIA_E_NONFINITE : TRIA_OK;
}

tria_status tria_calib_stats(tria_dtype dt, const void *q, int L, int Hq, int n_cal, int d, float *qc, float *qn,
                             float *rb, void *stream)
{
    if (!q || !qc || !qn || !rb) return TRIA_E_INVALID;
    if (dt != TRIA_BF16 && dt != TRIA_F32) return TRIA_E_INVALID;
    if (L <= 0 || Hq <= 0 || n_cal <= 0) return TRIA_E_INVALID;
    if ((long long)L * Hq > 0x7fffffffLL) return TRIA_E_INVALID;
    if (d != TRIA_D) return TRIA_E_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(qc, 4) || !aligned(qn, 4) || !aligned(rb, 4)) return TRIA_E_INVALID;
    if (tria::launch_calib_stats(dt, q, L * Hq, n_cal, qc, qn, rb, (hipStream_t)stream) != hipSuccess)
        return TRIA_E_DEVICE;
    return TRIA_OK;
}

size_t tria_select_workspace_bytes(int n_streams, int n_keys, int budget)
{
    if (n_streams <= 0 || n_keys <= 0 || budget <= 0) return 0;
    return 256;  // selection runs entirely in LDS; nothing is staged in the workspace
}

tria_status tria_select_topB(const float *F, int n_streams, int N, int B, int32_t *kept, void *ws,
                             size_t ws_bytes, void *stream)
{
    if (!F || !kept || n_streams <= 0 || N <= 0 || B <= 0 || N > (1 << 24)) return TRIA_E_INVALID;
    if (!aligned(F, 4) || !aligned(kept, 4)) return TRIA_E_INVALID;
    if (ws_bytes < tria_select_workspace_bytes(n_streams, N, B) || !ws) return TRIA_E_WORKSPACE;
    if (tria::launch_select(F, n_streams, N, B, kept, nullptr, nullptr, (hipStream_t)stream) != hipSuccess)
        return TRIA_E_DEVICE;
    return TRIA_OK;
}

tria_status tria_compact(tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *kept,
                         int n_streams, int N, int B, int d, void *stream)
{
    if (!k || !v || !kept || n_streams <= 0 || N <= 0 || B <= 0 || N > (1 << 24)) return TRIA_E_INVALID;
    if (dt != TRIA_BF16 && dt != TRIA_F32) return TRIA_E_INVALID;
    if (d != TRIA_D) return TRIA_E_UNSUPPORTED;
    if (!aligned(k, 16) || !aligned(v, 16) || (pos && !aligned(pos, 4)) || !aligned(kept, 4))
        return TRIA_E_INVALID;
    if (B >= N) return TRIA_OK;  // identity: every row stays where it is
    if (tria::launch_compact(dt, k, v, pos, kept, n_streams, N, B, (hipStream_t)stream) != hipSuccess)
        return TRIA_E_DEVICE;
    return TRIA_OK;
}

tria_status tria_copy(const void *src, void *dst, size_t n_bytes, void *stream)
{
    if (!src || !dst || n_bytes == 0 || n_bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16)) return TRIA_E_INVALID;
    const char *s = (const char *)src, *d = (const char *)dst;
    if (s < d + n_bytes && d < s + n_bytes) return TRIA_E_INVALID;     // the buffers overlap
    if (tria::launch_copy(src, dst, n_bytes / 16, (hipStream_t)stream) != hipSuccess) return TRIA_E_DEVICE;
    return TRIA_OK;
}

size_t tria_prune_workspace_bytes(const tria_calib *c, tria_dtype dt, int n_seq, int n_keys, int budget,
                                  unsigned flags)
{
    if (!c || n_seq <= 0 || n_keys <= 0 || budget <= 0) return 0;
    const size_t score = tria_score_workspace_bytes(c, dt, n_seq, n_keys, flags);
    if (score == 0) return 0;
    // the tile-parallel compaction's counter and flags after the score's workspace
    const long long n_streams = (long long)n_seq * c->L * c->Hkv;
    if (n_streams <= 0x7fffffffLL && tria::compact_tiles_applies((int)n_streams, n_keys, budget))
        return tria::align256(score) + tria::align256(tria::compact_tiles_sync_words((int)n_streams, budget) * 4);
    return score;
}

tria_status tria_prune(const tria_calib *c, tria_dtype dt, void *k, void *v, int32_t *pos,
                       const int32_t *t, int n_seq, int N, int B, float *F, int32_t *kept,
                       unsigned flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!c || !kept || !v || B <= 0) return TRIA_E_INVALID;
    // the compaction's checks, before anything is launched
    if (!aligned(v, 16) || (pos && !aligned(pos, 4)) || !aligned(kept, 4)) return TRIA_E_INVALID;
    tria_status s = tria_score(c, dt, k, pos, t, n_seq, N, F, nullptr, nullptr, flags, ws, ws_bytes, stream);
    if (s != TRIA_OK) return s;
    const int n_streams = n_seq * c->L * c->Hkv;
    // the selection reads the score's error word: after a failed score it keeps every row in place,
    // so that the compaction moves nothing
    const tria_score_ws lay = tria::score_ws_layout(c, dt, n_seq, N, flags);
    const int *guard = (const int *)((const char *)ws + lay.err_off);
    // the stream-cluster scorers leave a side copy of every 16th score, which the selection samples
    const float *samp = lay.cluster ? (const float *)((const char *)ws + lay.samp_off) : nullptr;
    if (tria::compact_tiles_applies(n_streams, N, B)) {
        // the selection, then the tile-parallel compaction, when the workspace has room for its
        // synchronisation words (tria_prune_workspace_bytes reserves them); else the fused
        // per-stream selection and compaction below
        const size_t sync_off = tria::align256(lay.total);
        const size_t words = tria::compact_tiles_sync_words(n_streams, B);
        if (ws_bytes >= sync_off + words * 4) {
            int *sync = (int *)((char *)ws + sync_off);
            if (tria::launch_select(F, n_streams, N, B, kept, guard, samp, (hipStream_t)stream, sync,
                                    tria::compact_tiles_per_stream(B)) != hipSuccess)
                return TRIA_E_DEVICE;
            if (tria::launch_compact_tiles(dt, k, v, pos, kept, n_streams, N, B, sync, (int *)guard,
                                           (hipStream_t)stream) != hipSuccess)
                return TRIA_E_DEVICE;
            return TRIA_OK;
        }
    }
    if (tria::select_compact_fused(N, B)) {
        // selection and compaction in one kernel (same results as the two calls)
        if (tria::launch_select_compact(dt, F, n_streams, N, B, kept, guard, samp, k, v, pos,
                                        (hipStream_t)stream) != hipSuccess)
            return TRIA_E_DEVICE;
        return TRIA_OK;
    }
    if (tria::launch_select(F, n_streams, N, B, kept, guard, samp, (hipStream_t)stream) != hipSuccess)
        return TRIA_E_DEVICE;
    return tria_compact(dt, k, v, pos, kept, n_streams, N, B, TRIA_D, stream);
}

tria_status tria_append(tria_dtype dt, void *k, void *v, int32_t *pos, int n_streams, int cap, int len,
                        const void *kn, const void *vn, const int32_t *pn, int n_new, int d, void *stream)
{
    if (!k || !v || !kn || !vn || (pos == nullptr) != (pn == nullptr)) return TRIA_E_INVALID;
    if (dt != TRIA_BF16 && dt != TRIA_F32) return TRIA_E_INVALID;
    if (n_streams <= 0 || cap <= 0 || len < 0 || n_new < 1 || (long long)len + n_new > cap) return TRIA_E_INVALID;
    if (d != TRIA_D) return TRIA_E_UNSUPPORTED;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kn, 16) || !aligned(vn, 16) || (pos && !aligned(pos, 4)) ||
        (pn && !aligned(pn, 4)))
        return TRIA_E_INVALID;
    if (tria::launch_append(dt, k, v, pos, n_streams, cap, len, kn, vn, pn, n_new, (hipStream_t)stream) != hipSuccess)
        return TRIA_E_DEVICE;
    return TRIA_OK;
}

tria_status tria_decode_step(const tria_calib *c, tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *t,
                             int n_seq, int cap, int len, int B, const void *kn, const void *vn, const int32_t *pn,
                             int n_new, float *F, int32_t *kept, unsigned flags, void *ws, size_t ws_bytes,
                             int *new_len, void *stream)
{
    if (!c || !new_len || B <= 0 || n_seq <= 0) return TRIA_E_INVALID;
    if ((long long)n_seq * c->L * c->Hkv > 0x7fffffffLL) return TRIA_E_INVALID;
    const int n_streams = n_seq * c->L * c->Hkv;
    tria_status s = tria_append(dt, k, v, pos, n_streams, cap, len, kn, vn, pn, n_new, TRIA_D, stream);
    if (s != TRIA_OK) return s;
    if (len + n_new == cap && cap > B) {
        s = tria_prune(c, dt, k, v, pos, t, n_seq, cap, B, F, kept, flags, ws, ws_bytes, stream);
        if (s != TRIA_OK) return s;
        *new_len = B;
    } else {
        *new_len = len + n_new;
    }
    return TRIA_OK;
}

}  // extern "C"
