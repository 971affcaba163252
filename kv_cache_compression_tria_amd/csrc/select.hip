// select.hip -- top-B selection per stream (gfx950).
//
// Keep the B keys with the largest final score, ties to the lower index, written in ascending
// index order (chenxutan.com/d/2624 section 4.2: top-k of the scores, then sorted to keep the
// cache order).  One workgroup per stream.  Scores are mapped to order-preserving unsigned keys
// (-0 folded onto +0); the B-th largest key T and the number k of keys equal to T that are kept
// are found by radix digits over LDS histograms.  Final scores cluster in a few exponent values,
// so a digit can pile onto few bins: each wave first counts its heavy bins with one ballot per
// bin and a single atomic, and only the scattered rest use per-lane atomics.  Every key > T is
// kept and the first k keys == T (in index order), at slot
// #(key > T before j) + min(#(key == T before j), k).
//   select_stream_kernel (streams of 8193 to 32768 keys): brackets T from a sample, passes over F
//     once, resolves T among the bracketed keys and writes the output from two bitmaps;
//   select_lds_kernel (streams up to 8192 keys): the same steps over an LDS copy of the keys;
//   select_compact_kernel, select_lds_compact_kernel (tria_prune): the streamed or the LDS
//     selection of a stream followed by its compaction, in one block;
//   select_global_kernel (longer streams): three digits (11, 11, 10 bits) over all keys re-read
//     from F in every pass; wave w owns the contiguous key range [w*N/16, (w+1)*N/16), and the
//     candidate list and the output are written in index order from per-wave counts and a prefix
//     over the 16 wave totals.
#include "common.cuh"
#include "compact_stream.cuh"
#include "tria_internal.h"

namespace tria {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
constexpr int kCand = 4096;       // candidate list in LDS
constexpr int kSelectDigitBins = 256;    // the sample's histogram and the bracketed keys' 8-bit digits
constexpr int kSelectBitmapWords = 2 * ((kSelectStreamKeys + 31) / 32);
constexpr int kSelectShortKeys = 8192;   // streams up to this many keys: LDS copy, 256-thread blocks
constexpr int kSelectSamples = 2048;     // sampled scores behind the bracket (streamed selection)
static_assert(kCand >= kBins0, "the fallback's histogram lives in the candidate keys");
static_assert(kSelectBitmapWords >= kBins0, "the LDS selection's fallback histogram lives in the bitmap words");
static_assert(kSelectShortKeys * 4 + (kSelectBitmapWords + kCand + kSelectDigitBins) * 4 + 1024 <= 64 * 1024,
              "the LDS selection exceeds 64 KB without a dynamic-LDS attribute");
static_assert((kSelectBitmapWords + kCand + kSelectDigitBins) * 4 + kCand * 2 + 1024 <= 34 * 1024,
              "the streamed selection's LDS no longer lets four blocks share a CU");
static_assert(kSelectStreamKeys <= 65536, "candidate indices of the streamed selection are 16-bit");

// the score of an order key (inverse of order_key)
__device__ __forceinline__ float key_float(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Exclusive prefix over the lanes of a 64-bit ballot mask: the number of set lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Clears the synchronisation words of the tile-parallel compaction that follows the selection in
// tria_prune (sync: [0] the tile counter, then `words` flags per stream); block sid clears its
// stream's flags and block 0 the counter.  Plain stores: the compaction is a later launch.
__device__ __forceinline__ void clear_compact_sync(int *__restrict__ sync, int words, int NT)
{
    if (!sync) return;
    int *w = sync + 1 + (size_t)blockIdx.x * words;
    for (int i = threadIdx.x; i < words; i += NT) w[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) sync[0] = 0;
}

__global__ __launch_bounds__(kSelectThreads) void select_global_kernel(const float *__restrict__ F, int N, int B,
                                                                       int32_t *__restrict__ kept,
                                                                       const int *__restrict__ guard,
                                                                       int *__restrict__ sync, int sync_words)
{
    clear_compact_sync(sync, sync_words, kSelectThreads);
    constexpr int NT = kSelectThreads;
    constexpr int NW = NT / 64;
    __shared__ uint32_t hist[kBins0];
    __shared__ uint32_t cand[kCand];
    __shared__ uint32_t wa[NW], wb[NW];
    __shared__ uint32_t s_prefix, s_k;

    const int sid = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform loop bounds
    const float *f = F + (size_t)sid * N;
    int32_t *out = kept + (size_t)sid * B;            // B < N on this path
    if (guard && *guard != 0) {                       // the scores are not usable: keep every row in place
        for (int i = threadIdx.x; i < B; i += NT) out[i] = i;
        return;
    }
    auto key_at = [&](int j) -> uint32_t { return order_key(f[j]); };
    // wave w owns the contiguous key range [lo, hi); it walks it 256 keys per step, lane l taking
    // keys b + 64e + l (e < 4): four independent reads per step, visited in index order
    const int per = (N + NW - 1) / NW;
    const int lo = min(N, wid * per), hi = min(N, lo + per);
    auto load4 = [&](int b, uint32_t (&u)[4], bool (&in)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = b + 64 * e + lane;
            in[e] = j < hi;
            u[e] = in[e] ? key_at(j) : 0u;
        }
    };
    // exclusive prefix over the waves of per-wave totals (a, b), via LDS
    auto wave_prefix = [&](uint32_t a, uint32_t b, uint32_t &pa, uint32_t &pb) {
        if (lane == 0) {
            wa[wid] = a;
            wb[wid] = b;
        }
        __syncthreads();
        pa = 0u;
        pb = 0u;
        for (int w = 0; w < wid; ++w) {
            pa += wa[w];
            pb += wb[w];
        }
        __syncthreads();
    };

    // digit 0 = bits 31..21 over every key; the keys of the chosen digit-0 bin are then copied
    // to a candidate list (when they fit) and digits 1 (bits 20..10) and 2 (bits 9..0) are
    // resolved over the candidates alone
    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)B;
    auto find_bin = [&](int shift, int nbins) {
        __syncthreads();
        if (wid == 0) {
            // lane l owns bins nbins-1-l*per .. nbins-per-l*per (descending); find the bin where
            // the count of larger-or-equal keys first reaches k
            const int per_lane = nbins / 64;
            uint32_t local = 0u;
            for (int i = 0; i < per_lane; ++i) local += hist[nbins - 1 - lane * per_lane - i];
            const uint32_t incl = wave_incl_scan(local);
            uint32_t excl = incl - local;
            if (excl < k && k <= incl) {
                for (int i = 0; i < per_lane; ++i) {
                    const int bin = nbins - 1 - lane * per_lane - i;
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
    for (int b = lo; b < hi; b += 256) {
        uint32_t u[4];
        bool in[4];
        load4(b, u, in);
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_add(hist, u[e] >> 21, in[e]);
    }
    find_bin(21, kBins0);
    mask = 0xffe00000u;

    // candidates (keys whose digit 0 matches), written in index order without atomics: count per
    // wave, prefix over the waves, then write
    const bool listed = hist[prefix >> 21] <= (uint32_t)kCand;   // uniform; read before hist is reused
    int ncand = 0;
    if (listed) {
        uint32_t c = 0u;
        for (int b = lo; b < hi; b += 256) {
            uint32_t u[4];
            bool in[4];
            load4(b, u, in);
#pragma unroll
            for (int e = 0; e < 4; ++e) c += __builtin_popcountll(__ballot(in[e] && (u[e] & mask) == prefix));
        }
        uint32_t run, unused;
        wave_prefix(c, 0u, run, unused);
        for (int b = lo; b < hi; b += 256) {
            uint32_t u[4];
            bool in[4];
            load4(b, u, in);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool m = in[e] && (u[e] & mask) == prefix;
                const uint64_t bal = __ballot(m);
                if (m) cand[run + lanes_below(bal)] = u[e];
                run += __builtin_popcountll(bal);
            }
        }
        ncand = (int)hist[prefix >> 21];
        __syncthreads();
    }
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
            for (int b = lo; b < hi; b += 256) {
                uint32_t u[4];
                bool in[4];
                load4(b, u, in);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hist_add(hist, (u[e] >> shift) & (uint32_t)(nbins - 1), in[e] && (u[e] & mask) == prefix);
            }
        }
        find_bin(shift, nbins);
        mask |= (uint32_t)(nbins - 1) << shift;
    }
    const uint32_t T = prefix;   // the B-th largest key; k of the keys equal to T are kept

    // ordered write: count each wave's keys > T and == T, prefix over the waves, then write
    uint32_t ngt = 0u, neq = 0u;
    for (int b = lo; b < hi; b += 256) {
        uint32_t u[4];
        bool in[4];
        load4(b, u, in);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ngt += __builtin_popcountll(__ballot(in[e] && u[e] > T));
            neq += __builtin_popcountll(__ballot(in[e] && u[e] == T));
        }
    }
    uint32_t gt_run, eq_run;
    wave_prefix(ngt, neq, gt_run, eq_run);
    for (int b = lo; b < hi; b += 256) {
        uint32_t u[4];
        bool in[4];
        load4(b, u, in);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool gt = in[e] && u[e] > T, eq = in[e] && u[e] == T;
            const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
            const uint32_t gb = gt_run + lanes_below(mgt), eb = eq_run + lanes_below(meq);
            // every key > T is kept, and the first k keys == T; slot = keys kept before this one
            const uint32_t slot = gt ? gb + min(eb, k) : ((eq && eb < k) ? gb + eb : 0xffffffffu);
            if (slot < (uint32_t)B) out[slot] = b + 64 * e + lane;   // always true for a kept key
            gt_run += __builtin_popcountll(mgt);
            eq_run += __builtin_popcountll(meq);
        }
    }
}

// Short streams (up to 8192 keys) keep their keys in LDS: loaded once as order keys, then the same
// steps as the streamed selection below, reading LDS instead of F.
// A sample of NT keys (every (N / NT)-th) brackets the threshold: a 256-bin histogram of the
// sample, linear in the score between the sample's extremes, gives two bin edges lo <= hi whose
// ranks are the expected sample rank of the B-th largest key, minus and plus 4.5 standard
// deviations of that binomial count (plus 2).  One pass over all keys then counts the keys at or
// above hi (all kept), lists the indices of the keys in [lo, hi) as candidates and stores the
// "above" bitmap.  When the bracket holds the threshold (#above < B <= #above + #candidates) and
// the candidates fit, four 8-bit radix digits over the candidates alone give the B-th largest key
// T and the number k of keys equal to T that are kept, and the candidates' bits are set in the
// two bitmaps (> T, == T).  Otherwise (a sample that misses, heavy ties, non-finite scores) three
// radix digits (11, 11, 10 bits) run over all keys, followed by a bitmap pass.  Finally thread w
// takes bitmap word w: a block-wide prefix of the words' bit counts places every kept index at
// slot #(key > T before j) + min(#(key == T before j), k).
// The selection of stream sid by one block of NT threads (every thread must call it); keys: N
// words of the block's dynamic LDS.
template <int NT>
__device__ __forceinline__ void select_lds_block(int sid, const float *__restrict__ F, int N, int B,
                                                 int32_t *__restrict__ kept, const int *__restrict__ guard,
                                                 uint32_t *keys)
{
    constexpr int NW = NT / 64;
    __shared__ uint32_t bm[kSelectBitmapWords];       // the two bitmaps, or the fallback's histogram
    __shared__ uint32_t cand[kCand];                  // candidate indices
    __shared__ uint32_t dh[kSelectDigitBins];         // sample histogram, candidate digits
    __shared__ uint32_t scan[NW + 1];
    __shared__ float s_min[NW], s_max[NW];
    __shared__ uint32_t s_prefix, s_k, s_ncand, s_nabove, s_lo, s_hi;

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float *f = F + (size_t)sid * N;
    int32_t *out = kept + (size_t)sid * B;            // B < N on this path
    if (guard && *guard != 0) {                       // the scores are not usable: keep every row in place
        for (int i = threadIdx.x; i < B; i += NT) out[i] = i;
        return;
    }
    const int nwords = (N + 31) >> 5;
    uint32_t *gtb = bm, *eqb = bm + nwords;

    for (int i = threadIdx.x; i < kSelectDigitBins; i += NT) dh[i] = 0u;
    if (threadIdx.x == 0) {
        s_ncand = 0u;
        s_nabove = 0u;
    }

    // ---- pass 1: order keys into LDS
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

    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)B;
    // wave 0 finds the bin of h (nbins bins, counted from the top) where the running count first
    // reaches k; prefix gains the bin's digit at `shift`, and k becomes the rank within the bin
    auto find_bin = [&](const uint32_t *h, int shift, int nbins) {
        __syncthreads();
        if (wid == 0) {
            const int per_lane = nbins / 64;
            uint32_t local = 0u;
            for (int i = 0; i < per_lane; ++i) local += h[nbins - 1 - lane * per_lane - i];
            const uint32_t incl = wave_incl_scan(local);
            uint32_t excl = incl - local;
            if (excl < k && k <= incl) {
                for (int i = 0; i < per_lane; ++i) {
                    const int bin = nbins - 1 - lane * per_lane - i;
                    const uint32_t c = h[bin];
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

    // ---- the bracket from a sample: its extremes, 256 linear bins, the bins of two sample ranks
    const int S = min(N, NT);
    const int stride = N / S;
    const bool smp = (int)threadIdx.x < S;
    const float sv = smp ? key_float(keys[threadIdx.x * stride]) : 0.f;
    {
        float lo = smp ? sv : INFINITY, hi = smp ? sv : -INFINITY;
        if (smp && !isfinite(sv)) {
            lo = -INFINITY;                           // a non-finite sample: no usable bracket
            hi = INFINITY;
        }
        for (int o = 32; o >= 1; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, 64));
            hi = fmaxf(hi, __shfl_xor(hi, o, 64));
        }
        if (lane == 0) {
            s_min[wid] = lo;
            s_max[wid] = hi;
        }
    }
    __syncthreads();
    float smin = INFINITY, smax = -INFINITY;
    for (int w = 0; w < NW; ++w) {
        smin = fminf(smin, s_min[w]);
        smax = fmaxf(smax, s_max[w]);
    }
    const float span = smax - smin;
    bool ok = isfinite(span) && span > 0.f;           // uniform
    if (ok) {
        const float scale = (float)kSelectDigitBins / span;
        hist_add(dh, (uint32_t)min(kSelectDigitBins - 1, max(0, (int)((sv - smin) * scale))), smp);
        __syncthreads();
        if (wid == 0) {
            const float pf = (float)B / (float)N;
            const float e = pf * (float)S;
            const float d = 4.5f * sqrtf((float)S * pf * (1.f - pf)) + 2.f;
            const uint32_t r_hi = (uint32_t)fmaxf(1.f, floorf(e - d));
            const uint32_t r_lo = (uint32_t)fminf((float)S, ceilf(e + d));
            constexpr int PL = kSelectDigitBins / 64;   // lane l owns bins 255 - PL*l downwards
            uint32_t local = 0u;
            for (int i = 0; i < PL; ++i) local += dh[kSelectDigitBins - 1 - lane * PL - i];
            const uint32_t incl = wave_incl_scan(local);
            for (int t = 0; t < 2; ++t) {
                const uint32_t r = t == 0 ? r_hi : r_lo;
                uint32_t run = incl - local;
                if (run < r && r <= incl) {
                    for (int i = 0; i < PL; ++i) {
                        const int bin = kSelectDigitBins - 1 - lane * PL - i;
                        run += dh[bin];
                        if (run >= r) {
                            if (t == 0)
                                s_hi = bin == kSelectDigitBins - 1 ? 0xffffffffu
                                                                   : order_key(smin + (float)(bin + 1) / scale);
                            else
                                s_lo = order_key(smin + (float)bin / scale);
                            break;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- pass 2: keys at or above hi (counted, "above" bitmap), candidates in [lo, hi)
    if (ok) {
        const uint32_t lo = s_lo, hi = s_hi;
        uint32_t nabove = 0u;
        for (int j0 = wid * 256; j0 < N; j0 += NT * 4) {
            uint32_t wa = 0u, tot = 0u;
            uint64_t bc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 64 * e + lane;
                const uint32_t u = j < N ? keys[j] : 0u;
                const uint64_t ma = __ballot(j < N && u >= hi);
                bc[e] = __ballot(j < N && u >= lo && u < hi);
                nabove += (uint32_t)__builtin_popcountll(ma);
                tot += (uint32_t)__builtin_popcountll(bc[e]);
                if (lane == 2 * e) wa = (uint32_t)ma;
                if (lane == 2 * e + 1) wa = (uint32_t)(ma >> 32);
            }
            const int w = (j0 >> 5) + lane;
            if (lane < 8 && w < nwords) {
                gtb[w] = wa;
                eqb[w] = 0u;
            }
            if (tot) {
                uint32_t base = 0u;
                if (lane == 0) base = atomicAdd(&s_ncand, tot);
                base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if ((bc[e] >> lane) & 1u) {
                        const uint32_t slot = base + lanes_below(bc[e]);
                        if (slot < (uint32_t)kCand) cand[slot] = (uint32_t)(j0 + 64 * e + lane);
                    }
                    base += (uint32_t)__builtin_popcountll(bc[e]);
                }
            }
        }
        if (lane == 0 && nabove) atomicAdd(&s_nabove, nabove);
        __syncthreads();
        const uint32_t na = s_nabove, nc = s_ncand;
        ok = na < (uint32_t)B && (uint32_t)B <= na + nc && nc <= (uint32_t)kCand;   // uniform
    }

    if (ok) {
        // ---- the threshold among the candidates: 8-bit digits.  Every candidate lies in [lo, hi),
        // so the bits above the highest one in which lo and hi - 1 differ are common to all of them:
        // the digits inside that prefix are skipped.
        const int nc = (int)s_ncand;
        k = (uint32_t)B - s_nabove;
        const uint32_t span_bits = s_lo ^ (s_hi - 1u);
        const int first = span_bits ? 3 - ((31 - __builtin_clz(span_bits)) >> 3) : 3;
        mask = first > 0 ? ~((1u << (32 - 8 * first)) - 1u) : 0u;
        prefix = s_lo & mask;
        for (int dgt = first; dgt < 4; ++dgt) {
            const int shift = 24 - 8 * dgt;
            for (int i = threadIdx.x; i < kSelectDigitBins; i += NT) dh[i] = 0u;
            __syncthreads();
            for (int base = 0; base < nc; base += NT) {
                const int i = base + threadIdx.x;
                const uint32_t u = i < nc ? keys[cand[i]] : 0u;
                hist_add(dh, (u >> shift) & (uint32_t)(kSelectDigitBins - 1), i < nc && (u & mask) == prefix);
            }
            find_bin(dh, shift, kSelectDigitBins);
            mask |= (uint32_t)(kSelectDigitBins - 1) << shift;
        }
        const uint32_t T = prefix;
        for (int i = threadIdx.x; i < nc; i += NT) {
            const uint32_t j = cand[i], u = keys[j];
            if (u > T) atomicOr(&gtb[j >> 5], 1u << (j & 31));
            else if (u == T) atomicOr(&eqb[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
    } else {
        // ---- fallback: digit 0 (bits 31..21) over all keys, candidates, digits 1 and 2
        uint32_t *hist = bm;                          // kSelectBitmapWords >= kBins0
        for (int i = threadIdx.x; i < kBins0; i += NT) hist[i] = 0u;
        if (threadIdx.x == 0) s_ncand = 0u;
        __syncthreads();
        for (int j0 = wid * 64; j0 < N; j0 += NT) {
            const int j = j0 + lane;
            const uint32_t u = j < N ? keys[j] : 0u;
            hist_add(hist, u >> 21, j < N);
        }
        prefix = 0u;
        k = (uint32_t)B;
        find_bin(hist, 21, kBins0);
        mask = 0xffe00000u;
        const bool listed = hist[prefix >> 21] <= (uint32_t)kCand;   // uniform
        if (listed) {
            for (int j0 = wid * 256; j0 < N; j0 += NT * 4) {
                uint64_t bal[4];
                uint32_t tot = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + 64 * e + lane;
                    const uint32_t u = j < N ? keys[j] : 0u;
                    bal[e] = __ballot(j < N && (u & mask) == prefix);
                    tot += (uint32_t)__builtin_popcountll(bal[e]);
                }
                if (tot) {
                    uint32_t base = 0u;
                    if (lane == 0) base = atomicAdd(&s_ncand, tot);
                    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if ((bal[e] >> lane) & 1u) cand[base + lanes_below(bal[e])] = (uint32_t)(j0 + 64 * e + lane);
                        base += (uint32_t)__builtin_popcountll(bal[e]);
                    }
                }
            }
        }
        __syncthreads();                              // candidates complete; hist is cleared next
        const int nc = (int)s_ncand;
        for (int dgt = 1; dgt <= 2; ++dgt) {
            const int shift = dgt == 1 ? 10 : 0;
            const int nbins = dgt == 1 ? 2048 : 1024;
            for (int i = threadIdx.x; i < nbins; i += NT) hist[i] = 0u;
            __syncthreads();
            if (listed) {
                for (int base = 0; base < nc; base += NT) {
                    const int i = base + threadIdx.x;
                    const uint32_t u = i < nc ? keys[cand[i]] : 0u;
                    hist_add(hist, (u >> shift) & (uint32_t)(nbins - 1), i < nc && (u & mask) == prefix);
                }
            } else {
                for (int j0 = wid * 64; j0 < N; j0 += NT) {
                    const int j = j0 + lane;
                    const uint32_t u = j < N ? keys[j] : 0u;
                    hist_add(hist, (u >> shift) & (uint32_t)(nbins - 1), j < N && (u & mask) == prefix);
                }
            }
            find_bin(hist, shift, nbins);
            mask |= (uint32_t)(nbins - 1) << shift;
        }
        const uint32_t T = prefix;
        // bitmaps over all keys (the histogram is no longer read: find_bin ended with a barrier)
        for (int j0 = wid * 256; j0 < N; j0 += NT * 4) {
            uint32_t wg = 0u, we = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 64 * e + lane;
                const uint32_t u = j < N ? keys[j] : 0u;
                const uint64_t mg = __ballot(j < N && u > T), me = __ballot(j < N && u == T);
                if (lane == 2 * e) { wg = (uint32_t)mg; we = (uint32_t)me; }
                if (lane == 2 * e + 1) { wg = (uint32_t)(mg >> 32); we = (uint32_t)(me >> 32); }
            }
            const int w = (j0 >> 5) + lane;
            if (lane < 8 && w < nwords) {
                gtb[w] = wg;
                eqb[w] = we;
            }
        }
        __syncthreads();
    }

    // ---- output: slots from prefix counts over the words, then the kept indices
    uint32_t gcarry = 0u, ecarry = 0u;
    for (int w0 = 0; w0 < nwords; w0 += NT) {
        const int w = w0 + threadIdx.x;
        const uint32_t g = w < nwords ? gtb[w] : 0u, e = w < nwords ? eqb[w] : 0u;
        // prefix of (popcount g, popcount e) packed as two 16-bit fields (each total < 65536)
        const uint32_t x = (uint32_t)__builtin_popcount(g) | ((uint32_t)__builtin_popcount(e) << 16);
        uint32_t tot;
        const uint32_t ex = block_excl_scan<NT>(x, scan, &tot);
        const uint32_t gbase = gcarry + (ex & 0xffffu), ebase = ecarry + (ex >> 16);
        uint32_t bits = g | e;
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            const uint32_t below = (1u << b) - 1u;
            const uint32_t ng = gbase + (uint32_t)__builtin_popcount(g & below);
            const uint32_t ne = ebase + (uint32_t)__builtin_popcount(e & below);
            const uint32_t slot = ((g >> b) & 1u) ? ng + min(ne, k) : (ne < k ? ng + ne : 0xffffffffu);
            if (slot < (uint32_t)B) out[slot] = 32 * w + b;   // always true for a kept key
        }
        gcarry += tot & 0xffffu;
        ecarry += tot >> 16;
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void select_lds_kernel(const float *__restrict__ F, int N, int B,
                                                        int32_t *__restrict__ kept, const int *__restrict__ guard,
                                                        int *__restrict__ sync, int sync_words)
{
    extern __shared__ uint32_t keys[];                // [N]
    clear_compact_sync(sync, sync_words, NT);
    select_lds_block<NT>(blockIdx.x, F, N, B, kept, guard, keys);
}

// Streams up to 32768 keys are selected straight from F (no LDS copy of the keys, 42 KB of LDS, so
// several streams run per CU and hide each other's memory latency):
//   1. a sample of up to 2048 scores brackets the threshold (the scorer's side copy of every 16th
//      score when the caller passes one, read contiguously; else every (N / 2048)-th score of F,
//      which touches every line of F once more): a 256-bin histogram of the sample,
//      linear in the score between its extremes, gives the bins of the sample ranks e -/+ (4.5
//      sigma + 2) from the top, where e = S B / N is the expected rank of the B-th largest key and
//      sigma the spread of that binomial count; their edges are the bounds lo <= hi;
//   2. one pass over F (16-byte loads, four keys per lane) counts the keys at or above hi (all
//      kept) and writes their bitmap, and lists the keys in [lo, hi) with their indices;
//   3. when the bracket holds the threshold (#above < B <= #above + #listed) and the list fits,
//      four 8-bit radix digits over the listed keys give the B-th largest key T and the number k
//      of keys equal to T that are kept, and the listed keys' bits are set in the two bitmaps
//      (> T, == T); otherwise (a sample that misses, heavy ties, an outlier stretching the bins,
//      non-finite scores) three radix digits (11, 11, 10 bits) run over all keys, each pass
//      re-reading F, and a bitmap pass follows;
//   4. thread w takes bitmap word w: a block-wide prefix of the words' bit counts places every
//      kept index at #(key > T before j) + min(#(key == T before j), k).
// The selection of stream sid by one block of NT threads (every thread must call it).  SMAX:
// sampled scores behind the bracket; DEPTH: 16-byte loads of F in flight per lane in the pass.
// samp (may be null): per stream, ceil(N / kSampleStride) scores, samp[s][i] = F[s][kSampleStride i].
// The sample only places the bracket: the selection is exact whatever it holds.
template <int NT, int SMAX, int DEPTH>
__device__ __forceinline__ void select_stream_block(int sid, const float *__restrict__ F, int N, int B,
                                                    int32_t *__restrict__ kept, const int *__restrict__ guard,
                                                    const float *__restrict__ samp)
{
    constexpr int NW = NT / 64;
    constexpr int SPT = (SMAX + NT - 1) / NT;         // samples per thread
    __shared__ uint32_t bm[kSelectBitmapWords];       // the two bitmaps
    __shared__ uint32_t ckey[kCand];                  // candidates' keys; the fallback's histogram
    __shared__ uint16_t cidx[kCand];                  // candidates' indices (N <= 32768)
    __shared__ uint32_t dh[kSelectDigitBins];
    __shared__ uint32_t scan[NW + 1];
    __shared__ float s_min[NW], s_max[NW];
    __shared__ uint32_t s_prefix, s_k, s_ncand, s_nabove, s_lo, s_hi;

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float *f = F + (size_t)sid * N;
    int32_t *out = kept + (size_t)sid * B;            // B < N on this path
    if (guard && *guard != 0) {                       // the scores are not usable: keep every row in place
        for (int i = threadIdx.x; i < B; i += NT) out[i] = i;
        return;
    }
    const int nwords = (N + 31) >> 5;
    uint32_t *gtb = bm, *eqb = bm + nwords;

    for (int i = threadIdx.x; i < kSelectDigitBins; i += NT) dh[i] = 0u;
    if (threadIdx.x == 0) {
        s_ncand = 0u;
        s_nabove = 0u;
    }

    uint32_t prefix = 0u, mask = 0u, k = (uint32_t)B;
    auto find_bin = [&](const uint32_t *h, int shift, int nbins) {
        __syncthreads();
        if (wid == 0) {
            const int per_lane = nbins / 64;
            uint32_t local = 0u;
            for (int i = 0; i < per_lane; ++i) local += h[nbins - 1 - lane * per_lane - i];
            const uint32_t incl = wave_incl_scan(local);
            uint32_t excl = incl - local;
            if (excl < k && k <= incl) {
                for (int i = 0; i < per_lane; ++i) {
                    const int bin = nbins - 1 - lane * per_lane - i;
                    const uint32_t c = h[bin];
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

    // ---- the bracket from a sample of the scores: the side copy, else a strided read of F
    const int ns = (N + kSampleStride - 1) / kSampleStride;
    const float *sp = samp ? samp + (size_t)sid * ns : f;
    const int S = min(samp ? ns : N, SMAX);
    const int stride = samp ? 1 : N / S;
    float sv[SPT];
    bool smp[SPT];
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
        const int t = q * NT + threadIdx.x;
        smp[q] = t < S;
        sv[q] = smp[q] ? sp[(size_t)t * stride] : 0.f;
        if (smp[q]) {
            if (isfinite(sv[q])) {
                lo = fminf(lo, sv[q]);
                hi = fmaxf(hi, sv[q]);
            } else {
                lo = -INFINITY;                       // a non-finite sample: no usable bracket
                hi = INFINITY;
            }
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, o, 64));
        hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    if (lane == 0) {
        s_min[wid] = lo;
        s_max[wid] = hi;
    }
    __syncthreads();
    float smin = INFINITY, smax = -INFINITY;
    for (int w = 0; w < NW; ++w) {
        smin = fminf(smin, s_min[w]);
        smax = fmaxf(smax, s_max[w]);
    }
    const float span = smax - smin;
    bool ok = isfinite(span) && span > 0.f;           // uniform
    if (ok) {
        const float scale = (float)kSelectDigitBins / span;
#pragma unroll
        for (int q = 0; q < SPT; ++q)
            hist_add(dh, (uint32_t)min(kSelectDigitBins - 1, max(0, (int)((sv[q] - smin) * scale))), smp[q]);
        __syncthreads();
        if (wid == 0) {
            const float pf = (float)B / (float)N;
            const float e = pf * (float)S;
            const float d = 4.5f * sqrtf((float)S * pf * (1.f - pf)) + 2.f;
            const uint32_t r_hi = (uint32_t)fmaxf(1.f, floorf(e - d));
            const uint32_t r_lo = (uint32_t)fminf((float)S, ceilf(e + d));
            constexpr int PL = kSelectDigitBins / 64;
            uint32_t local = 0u;
            for (int i = 0; i < PL; ++i) local += dh[kSelectDigitBins - 1 - lane * PL - i];
            const uint32_t incl = wave_incl_scan(local);
            for (int t = 0; t < 2; ++t) {
                const uint32_t r = t == 0 ? r_hi : r_lo;
                uint32_t run = incl - local;
                if (run < r && r <= incl) {
                    for (int i = 0; i < PL; ++i) {
                        const int bin = kSelectDigitBins - 1 - lane * PL - i;
                        run += dh[bin];
                        if (run >= r) {
                            if (t == 0)
                                s_hi = bin == kSelectDigitBins - 1 ? 0xffffffffu
                                                                   : order_key(smin + (float)(bin + 1) / scale);
                            else
                                s_lo = order_key(smin + (float)bin / scale);
                            break;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- one pass over F: keys at or above hi (counted, bitmap), candidates in [lo, hi)
    const bool vec = (N & 3) == 0 && ((uintptr_t)F & 15) == 0;   // uniform
    if (ok) {
        const uint32_t blo = s_lo, bhi = s_hi;
        uint32_t nabove = 0u;
        // one wave step of 256 keys (lane l holds keys c0 + 4l .. c0 + 4l + 3)
        auto step = [&](int c0, const uint32_t (&u)[4]) {
            uint32_t nib = 0u;
            uint64_t bc[4];
            uint32_t tot = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = c0 + 4 * lane + e;
                const bool in = j < N;
                const bool ab = in && u[e] >= bhi;
                nib |= (uint32_t)ab << e;
                bc[e] = __ballot(in && u[e] >= blo && u[e] < bhi);
                tot += (uint32_t)__builtin_popcountll(bc[e]);
                nabove += (uint32_t)__builtin_popcountll(__ballot(ab));
            }
            // eight lanes make one bitmap word (32 keys); lane 8m writes word c0/32 + m
            uint32_t word = nib << (4 * (lane & 7));
            word |= __shfl_xor(word, 1, 64);
            word |= __shfl_xor(word, 2, 64);
            word |= __shfl_xor(word, 4, 64);
            const int w = (c0 >> 5) + (lane >> 3);
            if ((lane & 7) == 0 && w < nwords) {
                gtb[w] = word;
                eqb[w] = 0u;
            }
            if (tot) {
                uint32_t base = 0u;
                if (lane == 0) base = atomicAdd(&s_ncand, tot);
                base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if ((bc[e] >> lane) & 1u) {
                        const uint32_t slot = base + lanes_below(bc[e]);
                        if (slot < (uint32_t)kCand) {
                            ckey[slot] = u[e];
                            cidx[slot] = (uint16_t)(c0 + 4 * lane + e);
                        }
                    }
                    base += (uint32_t)__builtin_popcountll(bc[e]);
                }
            }
        };
        if (vec) {
            // DEPTH steps' loads are issued before the first of them is used; buffer loads over the
            // stream's N scores (the whole offset in the range-checked vector offset) return zero
            // past the end, so the loads need no branches
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)f, 0, N * 4, 0x00020000);
            for (int c0 = wid * 256; c0 < N; c0 += DEPTH * NT * 4) {
                u32x4 x[DEPTH];
#pragma unroll
                for (int q = 0; q < DEPTH; ++q)
                    x[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (c0 + q * NT * 4 + 4 * lane), 0, 0);
#pragma unroll
                for (int q = 0; q < DEPTH; ++q) {
                    const int c = c0 + q * NT * 4;
                    if (c < N) {                              // uniform
                        const uint32_t u[4] = {order_key(__uint_as_float(x[q][0])), order_key(__uint_as_float(x[q][1])),
                                               order_key(__uint_as_float(x[q][2])), order_key(__uint_as_float(x[q][3]))};
                        step(c, u);
                    }
                }
            }
        } else {
            for (int c0 = wid * 256; c0 < N; c0 += NT * 4) {
                uint32_t u[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = c0 + 4 * lane + e;
                    u[e] = j < N ? order_key(f[j]) : 0u;
                }
                step(c0, u);
            }
        }
        if (lane == 0 && nabove) atomicAdd(&s_nabove, nabove);
        __syncthreads();
        const uint32_t na = s_nabove, nc = s_ncand;
        ok = na < (uint32_t)B && (uint32_t)B <= na + nc && nc <= (uint32_t)kCand;   // uniform
    }

    if (ok) {
        // ---- the threshold among the candidates: 8-bit digits.  Every candidate lies in [lo, hi),
        // so the bits above the highest one in which lo and hi - 1 differ are common to all of them:
        // the digits inside that prefix are skipped.
        const int nc = (int)s_ncand;
        k = (uint32_t)B - s_nabove;
        const uint32_t span_bits = s_lo ^ (s_hi - 1u);
        const int first = span_bits ? 3 - ((31 - __builtin_clz(span_bits)) >> 3) : 3;
        mask = first > 0 ? ~((1u << (32 - 8 * first)) - 1u) : 0u;
        prefix = s_lo & mask;
        for (int dgt = first; dgt < 4; ++dgt) {
            const int shift = 24 - 8 * dgt;
            for (int i = threadIdx.x; i < kSelectDigitBins; i += NT) dh[i] = 0u;
            __syncthreads();
            for (int base = 0; base < nc; base += NT) {
                const int i = base + threadIdx.x;
                const uint32_t u = i < nc ? ckey[i] : 0u;
                hist_add(dh, (u >> shift) & (uint32_t)(kSelectDigitBins - 1), i < nc && (u & mask) == prefix);
            }
            find_bin(dh, shift, kSelectDigitBins);
            mask |= (uint32_t)(kSelectDigitBins - 1) << shift;
        }
        const uint32_t T = prefix;
        for (int i = threadIdx.x; i < nc; i += NT) {
            const uint32_t j = cidx[i], u = ckey[i];
            if (u > T) atomicOr(&gtb[j >> 5], 1u << (j & 31));
            else if (u == T) atomicOr(&eqb[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
    } else {
        // ---- fallback: three radix digits (11, 11, 10 bits) over all keys, re-read from F
        uint32_t *hist = ckey;                        // kCand >= kBins0
        prefix = 0u;
        mask = 0u;
        k = (uint32_t)B;
        for (int dgt = 0; dgt < 3; ++dgt) {
            const int shift = dgt == 0 ? 21 : dgt == 1 ? 10 : 0;
            const int nbins = dgt == 2 ? 1024 : 2048;
            for (int i = threadIdx.x; i < nbins; i += NT) hist[i] = 0u;
            __syncthreads();
            for (int j0 = wid * 64; j0 < N; j0 += NT) {
                const int j = j0 + lane;
                const uint32_t u = j < N ? order_key(f[j]) : 0u;
                hist_add(hist, (u >> shift) & (uint32_t)(nbins - 1), j < N && (u & mask) == prefix);
            }
            find_bin(hist, shift, nbins);
            mask |= (uint32_t)(nbins - 1) << shift;
        }
        const uint32_t T = prefix;
        for (int j0 = wid * 256; j0 < N; j0 += NT * 4) {
            uint32_t wg = 0u, we = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 64 * e + lane;
                const uint32_t u = j < N ? order_key(f[j]) : 0u;
                const uint64_t mg = __ballot(j < N && u > T), me = __ballot(j < N && u == T);
                if (lane == 2 * e) { wg = (uint32_t)mg; we = (uint32_t)me; }
                if (lane == 2 * e + 1) { wg = (uint32_t)(mg >> 32); we = (uint32_t)(me >> 32); }
            }
            const int w = (j0 >> 5) + lane;
            if (lane < 8 && w < nwords) {
                gtb[w] = wg;
                eqb[w] = we;
            }
        }
        __syncthreads();
    }

    // ---- output: slots from prefix counts over the words, then the kept indices
    uint32_t gcarry = 0u, ecarry = 0u;
    for (int w0 = 0; w0 < nwords; w0 += NT) {
        const int w = w0 + threadIdx.x;
        const uint32_t g = w < nwords ? gtb[w] : 0u, e = w < nwords ? eqb[w] : 0u;
        const uint32_t x = (uint32_t)__builtin_popcount(g) | ((uint32_t)__builtin_popcount(e) << 16);
        uint32_t tot;
        const uint32_t ex = block_excl_scan<NT>(x, scan, &tot);
        const uint32_t gbase = gcarry + (ex & 0xffffu), ebase = ecarry + (ex >> 16);
        uint32_t bits = g | e;
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            const uint32_t below = (1u << b) - 1u;
            const uint32_t ng = gbase + (uint32_t)__builtin_popcount(g & below);
            const uint32_t ne = ebase + (uint32_t)__builtin_popcount(e & below);
            const uint32_t slot = ((g >> b) & 1u) ? ng + min(ne, k) : (ne < k ? ng + ne : 0xffffffffu);
            if (slot < (uint32_t)B) out[slot] = 32 * w + b;   // always true for a kept key
        }
        gcarry += tot & 0xffffu;
        ecarry += tot >> 16;
    }
}

template <int NT, int SMAX, int DEPTH>
__global__ __launch_bounds__(NT) void select_stream_kernel(const float *__restrict__ F, int N, int B,
                                                           int32_t *__restrict__ kept, const int *__restrict__ guard,
                                                           const float *__restrict__ samp, int *__restrict__ sync,
                                                           int sync_words)
{
    clear_compact_sync(sync, sync_words, NT);
    select_stream_block<NT, SMAX, DEPTH>(blockIdx.x, F, N, B, kept, guard, samp);
}

// The prune step's selection and compaction in one kernel, one block per stream: the block
// selects its stream's kept keys (written to kept), then compacts the stream's K, V and positions
// by them.  While some blocks of a CU select (bound by instruction issue and memory latency)
// others move rows (bound by HBM bandwidth), and the kept indices are read back while they are
// still in the caches.
constexpr int kSelectCompactThreads = 1024;

template <int RV>
__global__ __launch_bounds__(kSelectCompactThreads) void select_compact_kernel(const float *__restrict__ F, int N, int B,
                                                                            int32_t *__restrict__ kept,
                                                                            const int *__restrict__ guard,
                                                                            const float *__restrict__ samp,
                                                                            uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                            int32_t *__restrict__ pos)
{
    constexpr int NT = kSelectCompactThreads;
    select_stream_block<NT, kSelectSamples, 4>(blockIdx.x, F, N, B, kept, guard, samp);
    __syncthreads();   // the kept indices written by every thread are visible to the whole block
    compact_stream<RV, NT, kSelectCompactRows>(blockIdx.x, k, v, pos, kept, N, B);
}

// The same for streams that fit the LDS selection (up to kSelectShortKeys keys): the block copies
// its stream's scores into LDS, selects, and compacts.
template <int RV>
__global__ __launch_bounds__(kSelectCompactThreads) void select_lds_compact_kernel(const float *__restrict__ F, int N,
                                                                                int B, int32_t *__restrict__ kept,
                                                                                const int *__restrict__ guard,
                                                                                uint4 *__restrict__ k, uint4 *__restrict__ v,
                                                                                int32_t *__restrict__ pos)
{
    extern __shared__ uint32_t keys[];                // [N]
    select_lds_block<kSelectCompactThreads>(blockIdx.x, F, N, B, kept, guard, keys);
    __syncthreads();   // the kept indices written by every thread are visible to the whole block
    compact_stream<RV, kSelectCompactThreads, kSelectCompactRows>(blockIdx.x, k, v, pos, kept, N, B);
}

__global__ void identity_kernel(int32_t *__restrict__ kept, int n_streams, int N)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (size_t)n_streams * N) kept[i] = (int32_t)(i % N);
}

bool select_compact_fused(int N, int B) { return B < N && N <= kSelectStreamKeys; }

hipError_t launch_select_compact(tria_dtype dt, const float *F, int n_streams, int N, int B, int32_t *kept,
                                 const int *guard, const float *samp, void *k, void *v, int32_t *pos, hipStream_t st)
{
    if (!select_compact_fused(N, B)) return hipErrorInvalidValue;
    KernelTimer timer(TRIA_TIMER_SELECT_COMPACT, st);
    if (N <= kSelectShortKeys) {
        const size_t lds = (size_t)N * 4;
        if (dt == TRIA_BF16)
            select_lds_compact_kernel<16><<<n_streams, kSelectCompactThreads, lds, st>>>(F, N, B, kept, guard,
                                                                                       (uint4 *)k, (uint4 *)v, pos);
        else
            select_lds_compact_kernel<32><<<n_streams, kSelectCompactThreads, lds, st>>>(F, N, B, kept, guard,
                                                                                       (uint4 *)k, (uint4 *)v, pos);
    } else if (dt == TRIA_BF16) {
        select_compact_kernel<16><<<n_streams, kSelectCompactThreads, 0, st>>>(F, N, B, kept, guard, samp,
                                                                             (uint4 *)k, (uint4 *)v, pos);
    } else {
        select_compact_kernel<32><<<n_streams, kSelectCompactThreads, 0, st>>>(F, N, B, kept, guard, samp,
                                                                             (uint4 *)k, (uint4 *)v, pos);
    }
    return hipGetLastError();
}

hipError_t launch_select(const float *F, int n_streams, int N, int B, int32_t *kept, const int *guard,
                         const float *samp, hipStream_t st, int *sync, int sync_words)
{
    KernelTimer timer(TRIA_TIMER_SELECT, st);
    if (B >= N) {
        const size_t n = (size_t)n_streams * N;
        identity_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(kept, n_streams, N);
        return hipGetLastError();
    }
    if (N <= kSelectShortKeys) {
        select_lds_kernel<256><<<n_streams, 256, (size_t)N * 4, st>>>(F, N, B, kept, guard, sync, sync_words);
    } else if (N <= kSelectStreamKeys) {
        select_stream_kernel<512, kSelectSamples, 4><<<n_streams, 512, 0, st>>>(F, N, B, kept, guard, samp, sync,
                                                                                 sync_words);
    } else {
        select_global_kernel<<<n_streams, kSelectThreads, 0, st>>>(F, N, B, kept, guard, sync, sync_words);
    }
    return hipGetLastError();
}

}  // namespace tria
