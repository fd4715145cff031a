// Internal launch interface between the C ABI (api.cpp) and the gfx950 kernels (kernels.hip).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>
#include "tri.h"

namespace tri {

constexpr int kCompactChunk = 256;      // destination rows per compaction workgroup
// Launch shape of the scoring kernel (the measured best on MI355X).
constexpr int kScoreTile = 1024;        // key rows per scoring workgroup
constexpr int kScoreWaves = 8;          // waves per scoring workgroup
constexpr int kRangeParts = 2;          // score-range slots per (unit, score tile)
constexpr int kRangeWaves = 4;          // waves whose rows one range slot covers
constexpr int kFusedMax = TRI_FUSED_MAX_LEN;       // longest cache the fused single-kernel pass takes (slots)
constexpr int kFusedThreads = 512;      // threads of a fused workgroup (one per unit)
constexpr int kFusedBlocks = TRI_FUSED_MAX_BLOCKS; // paged: block-table entries a fused workgroup stages in LDS

// Everything a kernel needs about the cache, flattened.
struct CacheView {
  const void *k, *v;                    // k/v read-only for scoring, written by compaction
  int32_t *pos;
  int64_t layer_stride, stride_b, stride_h, stride_s;
  int64_t pos_layer_stride, pos_stride_b, pos_stride_h;
  const int32_t *block_table;
  int32_t block_size, max_blocks;
  int32_t block_shift;                  // log2(block_size) when it is a power of two, else -1
  int32_t layers, batch, heads, head_dim;
  int32_t dtype, rope, paged;
  int32_t capacity;                     // slots per unit
};

struct PassView {
  const float *u, *c_hat;
  const int32_t *lengths, *t;
  double theta;
  int32_t budget, recent;
  // aggregation variants (agg 0: the collapsed score)
  const float *centres;                 // [layers][heads][columns][head_dim]
  int32_t agg, group, n_offsets;
  int32_t columns, dpad;                // columns per (layer, head): 64 or 128; column of (head g, offset k) g*dpad + k
  const uint32_t *check;                // non-null: the precondition word; kernels return at entry when it is nonzero
};

// The precondition check of a call (tri_params.check): zeroes *check and, for paged caches when claims is given,
// the claims bitmap (one bit per pool block, ceil(num_blocks / 32) words), then sets the TRI_CHECK_* bits of every
// violated precondition (tri_checks.h).  claims null: no duplicate-block check.
hipError_t launch_check(const CacheView &cv, const PassView &pv, int32_t capacity, int32_t max_length,
                        int32_t num_blocks, uint32_t *check, uint32_t *claims, hipStream_t s);

// Columns of one offset block per query head in a variant's centres: 16 offsets, or 32 beyond 16.
inline int variant_dpad(int n_offsets) { return n_offsets <= 16 ? 16 : 32; }

hipError_t launch_prepare(const float *qbar, const float *c, int layers, int h_q, int h_kv, int d,
                          double theta, int rope, const int32_t *offsets_host, int n_offsets,
                          float *u, float *c_hat, hipStream_t s);
hipError_t launch_prepare_variant(const float *qbar, int layers, int h_q, int h_kv, int d, double theta, int rope,
                                  const int32_t *offsets_host, int n_offsets, float *centres, hipStream_t s);

// range (nullable): per (unit, score tile, part) the min and max order key of the scores of that part of the tile
// (the rows of kRangeWaves waves), [units][tiles][kRangeParts][2] words; written by the scoring kernel, read by
// the selection.
hipError_t launch_score(const CacheView &cv, const PassView &pv, float *scores, int64_t score_stride,
                        uint32_t *range, hipStream_t s);

// flags (units x chunks) and counter (one per unit) may be null (then the selection does not reset them); range null: the selection finds the
// score range itself.
hipError_t launch_select(const CacheView &cv, const PassView &pv, const float *scores, int64_t score_stride,
                         int32_t *keep, int32_t *new_lengths, uint32_t *flags, uint32_t *counter,
                         uint32_t *range, hipStream_t s);

// Whether the selection kernel can also compact (the keep list, and for a paged cache the block-table row up to
// the capacity, fit in its LDS), and that launch: selection
// and in-place moves of every unit by one workgroup, plus the paged tables (block_table_out, freed, n_freed
// null for contiguous caches).
bool select_moves_fit(const CacheView &cv, const PassView &pv);
constexpr int kSelectMoveMinUnits = 1024;   // fewest units for which tri_evict_step selects and compacts in one kernel
hipError_t launch_select_move(const CacheView &cv, const PassView &pv, const float *scores, int64_t score_stride,
                              int32_t *keep, int32_t *new_lengths, uint32_t *range, int32_t *block_table_out,
                              int32_t *freed, int32_t *n_freed, hipStream_t s);

constexpr int kFusedMinUnits = TRI_FUSED_MIN_UNITS;  // fewest units for which the fused pass is the default

// Whether the fused pass can take this cache (capacity, or the host bound on lengths, <= kFusedMax, and
// paged tables short enough to stage in LDS).
bool fused_fits(const CacheView &cv);

// Score, select and compact in one kernel, one workgroup per unit (caches of at most kFusedMax slots).
// scores and keep may be null.
hipError_t launch_fused(const CacheView &cv, const PassView &pv, float *scores, int64_t score_stride, int32_t *keep,
                        int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                        hipStream_t s);

// Calibration statistics: float64 partial sums per (layer, head, token chunk), then one reduction in chunk order.
constexpr int kCalibChunk = 4096;   // calibration tokens per partial-sum workgroup
struct QueryView {
  const void *q;
  int64_t stride_l, stride_n, stride_h;
  int64_t n;
  int32_t layers, heads, head_dim, dtype, rope;
};
hipError_t launch_calibrate(const QueryView &qv, double *partial, float *qbar, float *c, hipStream_t s);

// Decode attention over a (compacted) cache: split-K partial softmax sums, then one combine per query head.
constexpr int kDecodeSplitMax = 2048;    // most keys per partial-sum workgroup
// Keys per partial-sum workgroup: long streams per workgroup run fastest, so the longest split that still
// leaves enough workgroups (units x splits >= 4096) to fill the GPU, between 512 and kDecodeSplitMax.
int decode_split(int64_t units, int max_length);
struct DecodeView {
  const void *q;                         // [layers][batch][h_q][d], the cache's dtype
  float scale;
  int32_t h_q, group, max_length, split, splits;
};
hipError_t launch_decode(const CacheView &cv, const PassView &pv, const DecodeView &dv, float *partial, float *out,
                         hipStream_t s);

// The pass behind tri_evict_step (api.cpp).  control_only: ws holds only the first control_bytes() bytes of the
// workspace layout (tickets, score ranges, flags), and scores and keep must be given.
tri_status evict_step(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                      int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed, void *ws,
                      size_t ws_bytes, hipStream_t stream, const hipEvent_t *events, bool control_only);
// Bytes of the workspace's control words for these shapes (0 on bad input).
size_t control_bytes(const tri_cache *cache, const tri_params *params);
// Sets the thread's last-error message and returns st.
tri_status fail_status(tri_status st, const char *msg);

hipError_t launch_reset(uint32_t *flags, int64_t n_flags, uint32_t *counter, int64_t units, hipStream_t s);

hipError_t launch_compact(const CacheView &cv, const PassView &pv, const int32_t *keep,
                          int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                          uint32_t *flags, uint32_t *counter, hipStream_t s);

}  // namespace tri
