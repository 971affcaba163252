// tria_internal.h -- private declarations shared by the host ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tria.h"

#define TRIA_D 128      // head_dim
#define TRIA_HALF 64    // RoPE bands per head
#define TRIA_MAX_G 8    // largest GQA group handled

struct tria_calib {
    int L, Hq, Hkv, d, G;
    double theta;
    int n_off;
    int device;
    // device table (one allocation, `block`)
    void *block;
    size_t block_bytes;
    double2 *P;      // [L][Hq][64] qbar_f * mean_{d in D} exp(i w_f d)   (fp64)
    float2 *P32;     // [L][Hq][64] the same rounded to fp32
    float *W;        // [L][Hq][64] norm weights (1 - R_f) E|q_f|
    uint64_t *nu;    // [64] w_f / (2 pi) as a 64-bit fraction of a turn
    float *PW;       // [L][Hkv][64][3][G] Re P32, Im P32 and W of each KV group, band-major
    float *R;        // [L][Hq][64] R_f (the weight of the trigonometric term under TRIA_TRIG_WEIGHT_R)
    double2 *Qc;     // [L][Hq][64] qbar_f itself (fp64 complex), for the per-offset series
    int64_t *off;    // [n_off] the future offsets D
};

// Workspace layout of tria_score (every region 256-byte aligned).
struct tria_score_ws {
    size_t qrot_off, raw_off, part_off, zst_off, err_off, ops_off, pivot_off, xpart_off, arrive_off, samp_off, total;
    int tiled;       // 1: the stream does not fit one block's LDS
    int tiles;       // key tiles (blocks) per stream on the tiled path
    int cluster;     // 1: long bf16 streams are scored by stream clusters (xpart, arrive, samp reserved)
    int has_raw;     // 1: raw scores, tile partials and per-head mean / 1/std are reserved
    int rot;         // 1: pre-RoPE bf16 keys, turned to their positions inside the staged cluster kernel
};

namespace tria {

constexpr int kTileKeys = 1024;       // keys per block on the tiled scoring path
constexpr int kScoreThreads = 256;
constexpr int kFusedLdsMax = 80 * 1024;   // raw scores of a stream kept on chip up to this size
constexpr int kClusterLds = 128 * 1024;   // raw scores one block of a stream cluster keeps on chip
constexpr int kClusterMaxBlocks = 1024;   // largest cluster grid the workspace has room for
constexpr int kStageShortStreams = 256;   // streams that fit one block use the staged clusters from this many
constexpr int kSelectThreads = 1024;
constexpr int kSelectStreamKeys = 32768;  // streams up to this many keys: the streamed selection (bitmaps of
                                          // 2 x N/32 words in LDS)
constexpr int kSampleStride = 16;     // the cluster scorers copy every 16th key's F to a side sample
constexpr int kCompactThreads = 1024;   // the compaction kernel: one block of 16 waves per stream,
constexpr int kCompactRows = 256;       // 256 rows per tile (few streams move faster with wide blocks)
constexpr int kSelectCompactRows = 128; // rows per tile of the fused selection + compaction (1024 threads)
constexpr int kTileCompactRows = 256;   // rows per block of the tile-parallel compaction (1024 threads)
constexpr int kTileCompactShortKeys = 8192;  // with many streams, the tile compaction for streams up to this long

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }


// Brackets the kernel launches of its scope with a HIP event pair on `st` when timing is enabled
// (tria_timing_enable); does nothing otherwise.
class KernelTimer {
  public:
    KernelTimer(int which, hipStream_t st);
    ~KernelTimer();
    KernelTimer(const KernelTimer &) = delete;
    KernelTimer &operator=(const KernelTimer &) = delete;

  private:
    int which_;
    hipStream_t st_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// Workspace layout of tria_score for these shapes and flags on the current device (the path choice
// included); tria_score and the workspace sizers use the same function.
tria_score_ws score_ws_layout(const tria_calib *c, tria_dtype dt, int n_seq, int n_keys, unsigned flags);
// True when bf16 streams of n_keys keys at group size G can be scored by stream clusters on the
// current device (cooperative launch, clusters of at most 32 blocks).
bool cluster_path_applies(int G, int n_keys);
bool stage_path_applies(int G, int n_keys);   // the staged cluster kernel (one of the two above)

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once per (kernel, device);
// thread-safe.
hipError_t allow_dynamic_lds(const void *kernel, int bytes);

// kernel launchers (return hipSuccess or the launch error)
hipError_t launch_rotate(const tria_calib *c, const int32_t *t, int n_seq, float *qrot, int *err, bool weight_r,
                         hipStream_t st);
hipError_t launch_score(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                        const int32_t *t, int n_seq, int N, const float *qrot, float *F, float *raw,
                        float *stats, unsigned flags, const tria_score_ws &lay, char *ws, hipStream_t st);
int mfma_ops_per_stream(int G);   // 16-byte operand words per lane and stream (prologue output)
// bf16 keys on the matrix cores: a prologue kernel rotates the queries (t, R-weighted with weight_r),
// builds the operands and pivots and clears the error word, then the scoring kernels run
// pos: key positions, read when lay.rot (pre-RoPE keys turned to their positions on the staged path)
hipError_t launch_score_mfma(const tria_calib *c, const void *k, const int32_t *pos, const int32_t *t, int n_seq,
                             int N, bool weight_r, float *F, float *raw, float *stats, const tria_score_ws &lay,
                             char *ws, hipStream_t st);
// per-head statistics and z-max of the tiled paths over raw [streams][G][N] and the tile partials
// part [streams][tiles][G][4] (sums around pivot[stream][h], or around 0 when pivot is null)
hipError_t launch_tile_finish(int G, int streams, int N, int tiles, const float *raw, const double *part,
                              const float *pivot, float *F, float *stats, const tria_score_ws &lay, char *ws,
                              hipStream_t st);
// TRIA_OFFSET_MAX scoring (matrix cores, bf16 keys): the largest per-offset trigonometric series
hipError_t launch_score_maxd(const tria_calib *c, const void *k, const int32_t *t, int n_seq, int N, bool weight_r,
                             float *F, float *raw, float *stats, const tria_score_ws &lay, char *ws, hipStream_t st);
constexpr int kMaxdOffsetsLimit = 32;   // TRIA_OFFSET_MAX: most future offsets supported
// TRIA_PER_KEY_PHASE / TRIA_KEYS_PRE_ROPE scoring (vector ALU, any dtype)
hipError_t launch_score_perkey(const tria_calib *c, tria_dtype dt, const void *k, const int32_t *pos,
                               const int32_t *t, int n_seq, int N, unsigned flags, float *F, float *raw_out,
                               float *stats, const tria_score_ws &lay, char *ws, hipStream_t st);
hipError_t launch_calib_stats(tria_dtype dt, const void *q, int n_heads, int n_cal, float *qc, float *qn, float *rb,
                              hipStream_t st);
hipError_t launch_append(tria_dtype dt, void *k, void *v, int32_t *pos, int n_streams, int cap, int len,
                         const void *kn, const void *vn, const int32_t *pn, int n_new, hipStream_t st);
hipError_t launch_zmax(int G, const float *raw, const double *part, int streams, int N, int tiles, float *F,
                       float *stats, hipStream_t st);
// guard (device, may be null): when *guard != 0 at run time the kernels write kept = 0..B-1 (rows stay in
// place) instead of selecting.  samp (device, may be null): the cluster scorers' side copy of every
// kSampleStride-th score ([streams][ceil(N / kSampleStride)]), which the streamed selection samples
// instead of F; it only places the bracket, so the kept sets do not depend on it.
// sync (device, may be null): the tile-parallel compaction's counter and flags (sync_words flags per
// stream), which the selection clears for the compaction launched after it
hipError_t launch_select(const float *F, int n_streams, int N, int B, int32_t *kept, const int *guard,
                         const float *samp, hipStream_t st, int *sync = nullptr, int sync_words = 0);
// the streaming copy of tria_copy: n16 16-byte words (copy.hip)
hipError_t launch_copy(const void *src, void *dst, size_t n16, hipStream_t st);
hipError_t launch_compact(tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *kept,
                          int n_streams, int N, int B, hipStream_t st);
// The tile-parallel compaction (tria_prune): one block per tile of kTileCompactRows destination
// rows.  compact_tiles_applies: whether tria_prune takes it for n_streams streams of N keys on the
// current device (fewer streams than two per CU, or streams of up to kTileCompactShortKeys keys); compact_tiles_sync_words: its counter and flags (ints,
// to be cleared by the selection launched before it, see launch_select); err: the step's error
// word (bit 4 set if a tile's wait for its predecessors timed out).
bool compact_tiles_applies(int n_streams, int N, int B);
size_t compact_tiles_sync_words(int n_streams, int B);
int compact_tiles_per_stream(int B);
hipError_t launch_compact_tiles(tria_dtype dt, void *k, void *v, int32_t *pos, const int32_t *kept, int n_streams,
                                int N, int B, int *sync, int *err, hipStream_t st);
// selection and compaction in one kernel (tria_prune) for the shapes where select_compact_fused holds
bool select_compact_fused(int N, int B);
hipError_t launch_select_compact(tria_dtype dt, const float *F, int n_streams, int N, int B, int32_t *kept,
                                 const int *guard, const float *samp, void *k, void *v, int32_t *pos,
                                 hipStream_t st);

}  // namespace tria
