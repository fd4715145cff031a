// C ABI of the eviction pass: host-side validation, workspace carving and the launch sequence.
// Nothing here touches device memory or the HIP runtime before validation has passed.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tri_internal.h"

namespace {

thread_local char g_err[512] = "";

tri_status fail(tri_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

tri_status ok() {
  g_err[0] = '\0';
  return TRI_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_size(int32_t dtype) { return dtype == TRI_BF16 ? 2 : 4; }

int64_t capacity(const tri_cache *c) {
  return c->layout == TRI_PAGED ? (int64_t)c->max_blocks_per_seq * c->block_size : (int64_t)c->max_len;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layout: [per-unit tickets | score ranges | flags | block claims | keep | scores], each part 256-byte
// aligned.  Block claims (one bit per pool block) exist for checked calls on paged caches only.
struct WsLayout {
  size_t counter, range, flags, claims, keep, scores, total;
  int64_t n_flags, n_units;
};

WsLayout ws_layout(const tri_cache *c, const tri_params *p) {
  WsLayout w{};
  const int64_t units = (int64_t)c->num_layers * c->batch * c->num_kv_heads;
  const int64_t cpu = (p->budget + tri::kCompactChunk - 1) / tri::kCompactChunk;
  const int64_t stride = tri_score_stride(c);
  w.n_flags = units * cpu;
  w.counter = 0;
  w.n_units = units;
  const int64_t tiles = (tri_score_stride(c) + tri::kScoreTile - 1) / tri::kScoreTile;
  w.range = round_up((size_t)units * 4);
  w.flags = w.range + round_up((size_t)(units * tiles * tri::kRangeParts) * 8);
  w.claims = w.flags + round_up((size_t)w.n_flags * 4);
  const bool claims = p->check != nullptr && c->layout == TRI_PAGED;
  w.keep = w.claims + (claims ? round_up((size_t)((c->num_blocks + 31) / 32) * 4) : 0);
  w.scores = w.keep + round_up((size_t)(units * p->budget) * 4);
  w.total = w.scores + round_up((size_t)(units * stride) * 4);
  return w;
}

tri_status check_cache(const tri_cache *c) {
  if (!c) return fail(TRI_ERR_INVALID_ARG, "cache is NULL");
  if (c->layout != TRI_CONTIGUOUS && c->layout != TRI_PAGED) return fail(TRI_ERR_INVALID_ARG, "bad layout %d", c->layout);
  if (c->dtype != TRI_BF16 && c->dtype != TRI_F32) return fail(TRI_ERR_INVALID_ARG, "bad dtype %d", c->dtype);
  if (c->rope != TRI_ROPE_HALF && c->rope != TRI_ROPE_INTERLEAVED) return fail(TRI_ERR_INVALID_ARG, "bad rope %d", c->rope);
  if (c->num_layers < 1 || c->batch < 1 || c->num_kv_heads < 1)
    return fail(TRI_ERR_INVALID_ARG, "num_layers, batch and num_kv_heads must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(TRI_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", c->head_dim);
  if (!c->k || !c->v || !c->pos) return fail(TRI_ERR_INVALID_ARG, "k, v and pos must be non-NULL");
  if (!aligned(c->k, 16) || !aligned(c->v, 16)) return fail(TRI_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (!aligned(c->pos, 4)) return fail(TRI_ERR_INVALID_ARG, "pos must be 4-byte aligned");
  const int e = elem_size(c->dtype);
  if (c->layer_stride < 0 || (c->layer_stride * e) % 16) return fail(TRI_ERR_INVALID_ARG, "layer_stride must be >= 0 and 16-byte aligned");
  if (c->pos_layer_stride < 0) return fail(TRI_ERR_INVALID_ARG, "pos_layer_stride must be >= 0");
  const int64_t units = (int64_t)c->num_layers * c->batch * c->num_kv_heads;
  if (units > (int64_t)1 << 30) return fail(TRI_ERR_UNSUPPORTED, "too many units (%lld)", (long long)units);
  if (c->layout == TRI_CONTIGUOUS) {
    if (c->max_len < 1) return fail(TRI_ERR_INVALID_ARG, "max_len must be >= 1");
    if (c->stride_b < 0 || c->stride_h < 0 || c->stride_s < 0) return fail(TRI_ERR_INVALID_ARG, "strides must be >= 0");
    if ((c->stride_b * e) % 16 || (c->stride_h * e) % 16 || (c->stride_s * e) % 16)
      return fail(TRI_ERR_INVALID_ARG, "row strides must be multiples of 16 bytes");
    if (c->stride_s < c->head_dim) return fail(TRI_ERR_INVALID_ARG, "stride_s smaller than head_dim");
    if (c->pos_stride_b < 0 || c->pos_stride_h < 0) return fail(TRI_ERR_INVALID_ARG, "pos strides must be >= 0");
    if ((int64_t)c->max_len * c->stride_s * e >= ((int64_t)1 << 31))
      return fail(TRI_ERR_UNSUPPORTED, "one unit's rows span %lld bytes (must be < 2^31)",
                  (long long)((int64_t)c->max_len * c->stride_s * e));
  } else {
    if (c->block_size < 1 || c->num_blocks < 1 || c->max_blocks_per_seq < 1)
      return fail(TRI_ERR_INVALID_ARG, "block_size, num_blocks and max_blocks_per_seq must be >= 1");
    if (!c->block_table) return fail(TRI_ERR_INVALID_ARG, "paged cache needs block_table");
    if (!aligned(c->block_table, 4)) return fail(TRI_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  }
  if (capacity(c) > TRI_MAX_LEN) return fail(TRI_ERR_UNSUPPORTED, "slot capacity %lld exceeds %d", (long long)capacity(c), TRI_MAX_LEN);
  // one scoring workgroup per (unit, half of a 1024-slot tile): the grid must fit a signed 32-bit index
  if (units * ((capacity(c) + tri::kScoreTile - 1) / tri::kScoreTile) * tri::kRangeParts >= ((int64_t)1 << 31))
    return fail(TRI_ERR_UNSUPPORTED, "%lld units of %lld slots need more than 2^31 scoring workgroups", (long long)units,
                (long long)capacity(c));
  return TRI_OK;
}

tri_status check_params(const tri_cache *c, const tri_params *p) {
  if (!p) return fail(TRI_ERR_INVALID_ARG, "params is NULL");
  if (!p->u || !p->c_hat || !p->lengths || !p->t) return fail(TRI_ERR_INVALID_ARG, "u, c_hat, lengths and t must be non-NULL");
  if (!aligned(p->u, 4) || !aligned(p->c_hat, 4) || !aligned(p->lengths, 4) || !aligned(p->t, 4))
    return fail(TRI_ERR_INVALID_ARG, "u, c_hat, lengths and t must be 4-byte aligned");
  if (!(p->rope_theta > 0.0) || !std::isfinite(p->rope_theta)) return fail(TRI_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (p->budget < 1) return fail(TRI_ERR_INVALID_ARG, "budget must be >= 1");
  if (p->recent < 0 || p->recent > p->budget) return fail(TRI_ERR_INVALID_ARG, "need 0 <= recent <= budget");
  if (p->max_length < 0 || p->max_length > capacity(c))
    return fail(TRI_ERR_INVALID_ARG, "max_length %d outside 0 .. slot capacity %lld", p->max_length, (long long)capacity(c));
  if (p->check && !aligned(p->check, 4)) return fail(TRI_ERR_INVALID_ARG, "check must be 4-byte aligned");
  if ((p->flags & ~(TRI_PASS_UNFUSED | TRI_PASS_FUSED)) || p->flags == (TRI_PASS_UNFUSED | TRI_PASS_FUSED))
    return fail(TRI_ERR_INVALID_ARG, "bad flags 0x%x", (unsigned)p->flags);
  if (const tri_variant *v = p->variant) {
    if (v->aggregation != TRI_AGG_MAX && v->aggregation != TRI_AGG_HEAD_MAX)
      return fail(TRI_ERR_INVALID_ARG, "bad aggregation %d", v->aggregation);
    if (v->group < 1 || v->n_offsets < 1 || tri_variant_columns(v->group, v->n_offsets) == 0)
      return fail(TRI_ERR_UNSUPPORTED, "variant group %d with %d offsets (group x offsets rounded up to 16 or 32 "
                  "must be at most 128 columns)", v->group, v->n_offsets);
    if (!v->centres || !aligned(v->centres, 16)) return fail(TRI_ERR_INVALID_ARG, "variant centres must be non-NULL and 16-byte aligned");
    if (v->reserved != 0) return fail(TRI_ERR_INVALID_ARG, "variant reserved must be 0");
    if (c->dtype != TRI_BF16) return fail(TRI_ERR_UNSUPPORTED, "aggregation variants need a bf16 cache");
  }
  return TRI_OK;
}

// Kernel view of a cache; launches are sized by `capacity`, the host bound on lengths when the caller gives one.
tri::CacheView view(const tri_cache *c, const tri_params *p) {
  tri::CacheView v{};
  v.k = c->k;
  v.v = c->v;
  v.pos = c->pos;
  v.layer_stride = c->layer_stride;
  v.stride_b = c->stride_b;
  v.stride_h = c->stride_h;
  v.stride_s = c->stride_s;
  v.pos_layer_stride = c->pos_layer_stride;
  v.pos_stride_b = c->pos_stride_b;
  v.pos_stride_h = c->pos_stride_h;
  v.block_table = c->block_table;
  v.block_size = c->block_size;
  v.max_blocks = c->max_blocks_per_seq;
  v.block_shift = -1;
  if (c->layout == TRI_PAGED && c->block_size > 0 && (c->block_size & (c->block_size - 1)) == 0)
    for (int sh = 0; sh < 31; ++sh)
      if ((1 << sh) == c->block_size) v.block_shift = sh;
  v.layers = c->num_layers;
  v.batch = c->batch;
  v.heads = c->num_kv_heads;
  v.head_dim = c->head_dim;
  v.dtype = c->dtype;
  v.rope = c->rope;
  v.paged = c->layout == TRI_PAGED;
  v.capacity = (int32_t)(p->max_length > 0 ? std::min<int64_t>(p->max_length, capacity(c)) : capacity(c));
  return v;
}

tri::PassView pview(const tri_params *p) {
  tri::PassView v{};
  v.u = p->u;
  v.c_hat = p->c_hat;
  v.lengths = p->lengths;
  v.t = p->t;
  v.theta = p->rope_theta;
  v.budget = p->budget;
  v.recent = p->recent;
  v.check = p->check;
  if (p->variant) {
    v.centres = p->variant->centres;
    v.agg = p->variant->aggregation;
    v.group = p->variant->group;
    v.n_offsets = p->variant->n_offsets;
    v.columns = tri_variant_columns(v.group, v.n_offsets);
    v.dpad = tri::variant_dpad(v.n_offsets);
  }
  return v;
}

tri_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(TRI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// The precondition check a call runs first when tri_params.check is given (claims: the workspace's block
// claims for calls that compact, else null).
hipError_t launch_checks(const tri_cache *c, const tri_params *p, uint32_t *claims, hipStream_t stream) {
  if (!p->check) return hipSuccess;
  return tri::launch_check(view(c, p), pview(p), (int32_t)capacity(c), p->max_length, c->num_blocks, p->check,
                           c->layout == TRI_PAGED ? claims : nullptr, stream);
}

tri_status check_compact_outputs(const tri_cache *c, const tri_params *p, const int32_t *table_out,
                                 const int32_t *freed, const int32_t *n_freed) {
  if (c->layout == TRI_PAGED) {
    if (!table_out || !freed || !n_freed) return fail(TRI_ERR_INVALID_ARG, "paged cache needs block_table_out, freed and n_freed");
    if (table_out == c->block_table) return fail(TRI_ERR_INVALID_ARG, "block_table_out must not alias block_table");
  } else if (table_out || freed || n_freed) {
    return fail(TRI_ERR_INVALID_ARG, "block_table_out, freed and n_freed must be NULL for a contiguous cache");
  }
  (void)p;
  return TRI_OK;
}

}  // namespace

namespace tri {
// Sets the thread's last-error message (the probes, in their own translation unit, report through it).
__attribute__((visibility("hidden"))) void set_error(const char *msg) { snprintf(g_err, sizeof g_err, "%s", msg); }
}  // namespace tri

extern "C" {

int32_t tri_variant_columns(int32_t group, int32_t n_offsets) {
  if (group < 1 || n_offsets < 1 || n_offsets > 32) return 0;
  const int64_t c = (int64_t)group * tri::variant_dpad(n_offsets);
  return c <= 64 ? 64 : (c <= 128 ? 128 : 0);
}

const char *tri_status_string(tri_status s) {
  switch (s) {
    case TRI_OK: return "TRI_OK";
    case TRI_ERR_INVALID_ARG: return "TRI_ERR_INVALID_ARG";
    case TRI_ERR_UNSUPPORTED: return "TRI_ERR_UNSUPPORTED";
    case TRI_ERR_WORKSPACE: return "TRI_ERR_WORKSPACE";
    case TRI_ERR_HIP: return "TRI_ERR_HIP";
  }
  return "TRI_ERR_UNKNOWN";
}

const char *tri_last_error(void) { return g_err; }

int64_t tri_score_stride(const tri_cache *cache) {
  if (!cache) return 0;
  const int64_t cap = capacity(cache);
  return cap <= 0 ? 0 : (cap + 63) / 64 * 64;
}

size_t tri_workspace_bytes(const tri_cache *cache, const tri_params *params) {
  if (check_cache(cache) != TRI_OK || check_params(cache, params) != TRI_OK) return 0;
  return ws_layout(cache, params).total;
}

tri_status tri_prepare_centres(const float *qbar, const float *c, int32_t num_layers, int32_t h_q, int32_t h_kv,
                               int32_t head_dim, double rope_theta, int32_t rope, const int32_t *offsets,
                               int32_t n_offsets, float *u, float *c_hat, hipStream_t stream) {
  if (!qbar || !c || !u || !c_hat || !offsets) return fail(TRI_ERR_INVALID_ARG, "NULL pointer argument");
  if (num_layers < 1 || h_kv < 1 || h_q < h_kv || h_q % h_kv)
    return fail(TRI_ERR_INVALID_ARG, "need num_layers >= 1 and h_q a positive multiple of h_kv");
  if (head_dim != 64 && head_dim != 128) return fail(TRI_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", head_dim);
  if (rope != TRI_ROPE_HALF && rope != TRI_ROPE_INTERLEAVED) return fail(TRI_ERR_INVALID_ARG, "bad rope %d", rope);
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return fail(TRI_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (n_offsets < 1 || n_offsets > TRI_MAX_OFFSETS) return fail(TRI_ERR_INVALID_ARG, "need 1 <= n_offsets <= %d", TRI_MAX_OFFSETS);
  if ((int64_t)num_layers * h_kv > (int64_t)1 << 30) return fail(TRI_ERR_UNSUPPORTED, "too many heads");
  return hip_status(tri::launch_prepare(qbar, c, num_layers, h_q, h_kv, head_dim, rope_theta, rope, offsets,
                                        n_offsets, u, c_hat, stream),
                    "tri_prepare_centres launch");
}

tri_status tri_prepare_variant_centres(const float *qbar, int32_t num_layers, int32_t h_q, int32_t h_kv,
                                       int32_t head_dim, double rope_theta, int32_t rope, const int32_t *offsets,
                                       int32_t n_offsets, float *centres, hipStream_t stream) {
  if (!qbar || !centres || !offsets) return fail(TRI_ERR_INVALID_ARG, "NULL pointer argument");
  if (num_layers < 1 || h_kv < 1 || h_q < h_kv || h_q % h_kv)
    return fail(TRI_ERR_INVALID_ARG, "need num_layers >= 1 and h_q a positive multiple of h_kv");
  if (n_offsets < 1 || tri_variant_columns(h_q / h_kv, n_offsets) == 0)
    return fail(TRI_ERR_UNSUPPORTED, "variant group %d with %d offsets (group x offsets rounded up to 16 or 32 must "
                "be at most 128 columns)", h_q / h_kv, n_offsets);
  if (head_dim != 64 && head_dim != 128) return fail(TRI_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", head_dim);
  if (rope != TRI_ROPE_HALF && rope != TRI_ROPE_INTERLEAVED) return fail(TRI_ERR_INVALID_ARG, "bad rope %d", rope);
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return fail(TRI_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if ((int64_t)num_layers * h_kv > (int64_t)1 << 30) return fail(TRI_ERR_UNSUPPORTED, "too many heads");
  return hip_status(tri::launch_prepare_variant(qbar, num_layers, h_q, h_kv, head_dim, rope_theta, rope, offsets,
                                                n_offsets, centres, stream),
                    "tri_prepare_variant_centres launch");
}

tri_status tri_score(const tri_cache *cache, const tri_params *params, float *scores, hipStream_t stream) {
  tri_status st;
  if ((st = check_cache(cache)) != TRI_OK || (st = check_params(cache, params)) != TRI_OK) return st;
  if (!scores || !aligned(scores, 16)) return fail(TRI_ERR_INVALID_ARG, "scores must be non-NULL and 16-byte aligned");
  hipError_t e = launch_checks(cache, params, nullptr, stream);
  if (e != hipSuccess) return hip_status(e, "check launch");
  return hip_status(tri::launch_score(view(cache, params), pview(params), scores, tri_score_stride(cache), nullptr, stream),
                    "tri_score launch");
}

tri_status tri_topk(const tri_cache *cache, const tri_params *params, const float *scores, int32_t *keep,
                    int32_t *new_lengths, hipStream_t stream) {
  tri_status st;
  if ((st = check_cache(cache)) != TRI_OK || (st = check_params(cache, params)) != TRI_OK) return st;
  if (!scores || !aligned(scores, 16)) return fail(TRI_ERR_INVALID_ARG, "scores must be non-NULL and 16-byte aligned");
  if (!keep || !new_lengths || !aligned(keep, 4) || !aligned(new_lengths, 4))
    return fail(TRI_ERR_INVALID_ARG, "keep and new_lengths must be non-NULL and 4-byte aligned");
  if (new_lengths == params->lengths) return fail(TRI_ERR_INVALID_ARG, "new_lengths must not alias lengths");
  hipError_t e = launch_checks(cache, params, nullptr, stream);
  if (e != hipSuccess) return hip_status(e, "check launch");
  return hip_status(tri::launch_select(view(cache, params), pview(params), scores, tri_score_stride(cache), keep, new_lengths,
                                       nullptr, nullptr, nullptr, stream),
                    "tri_topk launch");
}

tri_status tri_compact(const tri_cache *cache, const tri_params *params, const int32_t *keep, int32_t *block_table_out,
                       int32_t *freed, int32_t *n_freed, void *ws, size_t ws_bytes, hipStream_t stream) {
  tri_status st;
  if ((st = check_cache(cache)) != TRI_OK || (st = check_params(cache, params)) != TRI_OK) return st;
  if (!keep || !aligned(keep, 4)) return fail(TRI_ERR_INVALID_ARG, "keep must be non-NULL and 4-byte aligned");
  if ((st = check_compact_outputs(cache, params, block_table_out, freed, n_freed)) != TRI_OK) return st;
  const WsLayout w = ws_layout(cache, params);
  if (!ws || !aligned(ws, kAlign)) return fail(TRI_ERR_INVALID_ARG, "ws must be non-NULL and 256-byte aligned");
  if (ws_bytes < w.total) return fail(TRI_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  char *base = static_cast<char *>(ws);
  uint32_t *counter = reinterpret_cast<uint32_t *>(base + w.counter);
  uint32_t *flags = reinterpret_cast<uint32_t *>(base + w.flags);
  hipError_t e = launch_checks(cache, params, reinterpret_cast<uint32_t *>(base + w.claims), stream);
  if (e != hipSuccess) return hip_status(e, "check launch");
  e = tri::launch_reset(flags, w.n_flags, counter, w.n_units, stream);
  if (e != hipSuccess) return hip_status(e, "tri_compact reset launch");
  return hip_status(tri::launch_compact(view(cache, params), pview(params), keep, block_table_out, freed, n_freed, flags,
                                        counter, stream),
                    "tri_compact launch");
}

}  // extern "C"

namespace tri {

size_t control_bytes(const tri_cache *cache, const tri_params *params) {
  if (check_cache(cache) != TRI_OK || check_params(cache, params) != TRI_OK) return 0;
  return ws_layout(cache, params).keep;
}

// The pass; with control_only the workspace holds only the control words (tickets, score ranges, flags: the first
// control_bytes() bytes of the layout) and scores and keep must be given.
tri_status evict_step(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                      int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed, void *ws,
                      size_t ws_bytes, hipStream_t stream, const hipEvent_t *events, bool control_only) {
  tri_status st;
  if ((st = check_cache(cache)) != TRI_OK || (st = check_params(cache, params)) != TRI_OK) return st;
  if (!new_lengths || !aligned(new_lengths, 4)) return fail(TRI_ERR_INVALID_ARG, "new_lengths must be non-NULL and 4-byte aligned");
  if (new_lengths == params->lengths) return fail(TRI_ERR_INVALID_ARG, "new_lengths must not alias lengths");
  if (scores && !aligned(scores, 16)) return fail(TRI_ERR_INVALID_ARG, "scores must be 16-byte aligned");
  if (keep && !aligned(keep, 4)) return fail(TRI_ERR_INVALID_ARG, "keep must be 4-byte aligned");
  if (control_only && (!scores || !keep)) return fail(TRI_ERR_INVALID_ARG, "scores and keep must be non-NULL");
  if ((st = check_compact_outputs(cache, params, block_table_out, freed, n_freed)) != TRI_OK) return st;
  const WsLayout w = ws_layout(cache, params);
  const size_t need = control_only ? w.keep : w.total;
  if (!ws || !aligned(ws, kAlign)) return fail(TRI_ERR_INVALID_ARG, "ws must be non-NULL and 256-byte aligned");
  if (ws_bytes < need) return fail(TRI_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (events && (!events[0] || !events[1] || !events[2] || !events[3]))
    return fail(TRI_ERR_INVALID_ARG, "events must hold four created hipEvent_t");
  const tri::CacheView cv = view(cache, params);
  const tri::PassView pv = pview(params);
  hipError_t e = launch_checks(cache, params, reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + w.claims), stream);
  if (e != hipSuccess) return hip_status(e, "check launch");
  const int64_t units = (int64_t)cv.layers * cv.batch * cv.heads;
  const bool fused = !params->variant && !(params->flags & TRI_PASS_UNFUSED) && tri::fused_fits(cv) &&
                     ((params->flags & TRI_PASS_FUSED) || units >= tri::kFusedMinUnits);
  if (fused) {
    // Short caches: one kernel scores, selects and compacts each unit; scores and keep only when asked for.
    // With `events`, the first is recorded before it and the other three after it.
    if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return hip_status(e, "event record");
    e = tri::launch_fused(cv, pv, scores, tri_score_stride(cache), keep, new_lengths, block_table_out, freed, n_freed,
                          stream);
    if (e != hipSuccess) return hip_status(e, "fused launch");
    for (int i = 1; events && i < 4; ++i)
      if ((e = hipEventRecord(events[i], stream)) != hipSuccess) return hip_status(e, "event record");
    return ok();
  }
  char *base = static_cast<char *>(ws);
  uint32_t *counter = reinterpret_cast<uint32_t *>(base + w.counter);
  uint32_t *flags = reinterpret_cast<uint32_t *>(base + w.flags);
  uint32_t *range = reinterpret_cast<uint32_t *>(base + w.range);
  if (!keep) keep = reinterpret_cast<int32_t *>(base + w.keep);
  if (!scores) scores = reinterpret_cast<float *>(base + w.scores);
  const int64_t stride = tri_score_stride(cache);

  // One launch sequence; with `events`, an event is recorded before, between and after the kernels.
  if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return hip_status(e, "event record");
  if ((e = tri::launch_score(cv, pv, scores, stride, range, stream)) != hipSuccess) return hip_status(e, "score launch");
  if (events && (e = hipEventRecord(events[1], stream)) != hipSuccess) return hip_status(e, "event record");
  if (tri::select_moves_fit(cv, pv) && units >= tri::kSelectMoveMinUnits) {
    // One kernel selects and compacts each unit: a unit's selection latency overlaps other units' moves.  With few
    // units one workgroup per unit moves too little at once, and the moves are spread over several per unit.
    // With `events`, the third is recorded right after the second.
    if (events && (e = hipEventRecord(events[2], stream)) != hipSuccess) return hip_status(e, "event record");
    e = tri::launch_select_move(cv, pv, scores, stride, keep, new_lengths, range, block_table_out, freed, n_freed,
                                stream);
    if (e != hipSuccess) return hip_status(e, "select launch");
  } else {
    e = tri::launch_select(cv, pv, scores, stride, keep, new_lengths, flags, counter, range, stream);
    if (e != hipSuccess) return hip_status(e, "select launch");
    if (events && (e = hipEventRecord(events[2], stream)) != hipSuccess) return hip_status(e, "event record");
    e = tri::launch_compact(cv, pv, keep, block_table_out, freed, n_freed, flags, counter, stream);
    if (e != hipSuccess) return hip_status(e, "compact launch");
  }
  if (events && (e = hipEventRecord(events[3], stream)) != hipSuccess) return hip_status(e, "event record");
  return ok();
}

tri_status fail_status(tri_status st, const char *msg) { return fail(st, "%s", msg); }

}  // namespace tri

extern "C" {

static tri_status check_decode(const tri_cache *cache, const int32_t *lengths, int32_t max_length, const void *q,
                               int32_t h_q) {
  tri_status st;
  if ((st = check_cache(cache)) != TRI_OK) return st;
  if (!lengths || !aligned(lengths, 4)) return fail(TRI_ERR_INVALID_ARG, "lengths must be non-NULL and 4-byte aligned");
  if (max_length < 1 || max_length > capacity(cache))
    return fail(TRI_ERR_INVALID_ARG, "max_length %d outside 1 .. slot capacity %lld", max_length, (long long)capacity(cache));
  if (!q || !aligned(q, 16)) return fail(TRI_ERR_INVALID_ARG, "q must be non-NULL and 16-byte aligned");
  if (h_q < cache->num_kv_heads || h_q % cache->num_kv_heads) return fail(TRI_ERR_INVALID_ARG, "h_q must be a multiple of num_kv_heads");
  const int g = h_q / cache->num_kv_heads;
  if (g != 1 && g != 2 && g % 4) return fail(TRI_ERR_UNSUPPORTED, "query heads per KV head %d (1, 2 or a multiple of 4)", g);
  const int64_t units = (int64_t)cache->num_layers * cache->batch * cache->num_kv_heads;
  const int split = tri::decode_split(units, max_length);
  const int64_t splits = (max_length + split - 1) / split;
  if (units * splits * (g > 2 ? g / 4 : 1) >= ((int64_t)1 << 31) || units * g >= ((int64_t)1 << 31))
    return fail(TRI_ERR_UNSUPPORTED, "too many decode workgroups");
  return TRI_OK;
}

static size_t decode_ws(const tri_cache *cache, int32_t h_q, int32_t max_length) {
  const int64_t units = (int64_t)cache->num_layers * cache->batch * cache->num_kv_heads;
  const int split = tri::decode_split(units, max_length);
  const int64_t splits = (max_length + split - 1) / split;
  return round_up((size_t)units * (h_q / cache->num_kv_heads) * splits * (cache->head_dim + 2) * sizeof(float));
}

size_t tri_decode_workspace_bytes(const tri_cache *cache, int32_t h_q, int32_t max_length) {
  if (!cache || check_cache(cache) != TRI_OK) return 0;
  if (max_length < 1 || max_length > capacity(cache) || h_q < cache->num_kv_heads || h_q % cache->num_kv_heads) return 0;
  return decode_ws(cache, h_q, max_length);
}

tri_status tri_decode_attention(const tri_cache *cache, const int32_t *lengths, int32_t max_length, const void *q,
                                int32_t h_q, float scale, float *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  tri_status st;
  if ((st = check_decode(cache, lengths, max_length, q, h_q)) != TRI_OK) return st;
  if (!std::isfinite(scale)) return fail(TRI_ERR_INVALID_ARG, "scale must be finite");
  if (!out || !aligned(out, 4)) return fail(TRI_ERR_INVALID_ARG, "out must be non-NULL and 4-byte aligned");
  if (!ws || !aligned(ws, kAlign)) return fail(TRI_ERR_INVALID_ARG, "ws must be non-NULL and 256-byte aligned");
  const size_t need = decode_ws(cache, h_q, max_length);
  if (ws_bytes < need) return fail(TRI_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  tri_params p{};
  p.lengths = lengths;
  p.max_length = max_length;
  tri::DecodeView dv{};
  dv.q = q;
  dv.scale = scale;
  dv.h_q = h_q;
  dv.group = h_q / cache->num_kv_heads;
  dv.max_length = max_length;
  dv.split = tri::decode_split((int64_t)cache->num_layers * cache->batch * cache->num_kv_heads, max_length);
  dv.splits = (max_length + dv.split - 1) / dv.split;
  return hip_status(tri::launch_decode(view(cache, &p), pview(&p), dv, static_cast<float *>(ws), out, stream),
                    "tri_decode_attention launch");
}

static tri_status check_queries(const tri_queries *q) {
  if (!q) return fail(TRI_ERR_INVALID_ARG, "queries is NULL");
  if (q->dtype != TRI_BF16 && q->dtype != TRI_F32) return fail(TRI_ERR_INVALID_ARG, "bad dtype %d", q->dtype);
  if (q->rope != TRI_ROPE_HALF && q->rope != TRI_ROPE_INTERLEAVED) return fail(TRI_ERR_INVALID_ARG, "bad rope %d", q->rope);
  if (q->num_layers < 1 || q->num_heads < 1 || q->n < 1) return fail(TRI_ERR_INVALID_ARG, "need num_layers, num_heads, n >= 1");
  if (q->head_dim != 64 && q->head_dim != 128) return fail(TRI_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", q->head_dim);
  if (q->reserved != 0) return fail(TRI_ERR_INVALID_ARG, "reserved must be 0");
  if (!q->q || !aligned(q->q, 16)) return fail(TRI_ERR_INVALID_ARG, "queries must be non-NULL and 16-byte aligned");
  const int64_t e = elem_size(q->dtype);
  if (q->stride_l < 0 || q->stride_n < 0 || q->stride_h < 0 || (q->stride_l * e) % 16 || (q->stride_n * e) % 16 ||
      (q->stride_h * e) % 16)
    return fail(TRI_ERR_INVALID_ARG, "query strides must be non-negative and 16-byte multiples");
  const int64_t chunks = (q->n + tri::kCalibChunk - 1) / tri::kCalibChunk;
  if ((int64_t)q->num_layers * q->num_heads * chunks >= ((int64_t)1 << 31))
    return fail(TRI_ERR_UNSUPPORTED, "too many calibration chunks");
  return TRI_OK;
}

static size_t calib_ws(const tri_queries *q) {
  const int64_t chunks = (q->n + tri::kCalibChunk - 1) / tri::kCalibChunk;
  return round_up((size_t)q->num_layers * q->num_heads * chunks * (3 * q->head_dim / 2) * sizeof(double));
}

size_t tri_calibrate_workspace_bytes(const tri_queries *queries) {
  if (check_queries(queries) != TRI_OK) return 0;
  return calib_ws(queries);
}

tri_status tri_calibrate(const tri_queries *queries, float *qbar, float *c, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  tri_status st;
  if ((st = check_queries(queries)) != TRI_OK) return st;
  if (!qbar || !c || !aligned(qbar, 4) || !aligned(c, 4)) return fail(TRI_ERR_INVALID_ARG, "qbar and c must be non-NULL and 4-byte aligned");
  if (!ws || !aligned(ws, kAlign)) return fail(TRI_ERR_INVALID_ARG, "ws must be non-NULL and 256-byte aligned");
  if (ws_bytes < calib_ws(queries)) return fail(TRI_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, calib_ws(queries));
  tri::QueryView v{};
  v.q = queries->q;
  v.stride_l = queries->stride_l;
  v.stride_n = queries->stride_n;
  v.stride_h = queries->stride_h;
  v.n = queries->n;
  v.layers = queries->num_layers;
  v.heads = queries->num_heads;
  v.head_dim = queries->head_dim;
  v.dtype = queries->dtype;
  v.rope = queries->rope;
  return hip_status(tri::launch_calibrate(v, static_cast<double *>(ws), qbar, c, stream), "tri_calibrate launch");
}

tri_status tri_evict_step(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                          int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  return tri::evict_step(cache, params, scores, keep, new_lengths, block_table_out, freed, n_freed, ws, ws_bytes,
                         stream, nullptr, false);
}

tri_status tri_evict_step_profiled(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                                   int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                                   void *ws, size_t ws_bytes, hipStream_t stream, const hipEvent_t *events) {
  if (!events) return fail(TRI_ERR_INVALID_ARG, "events is NULL");
  return tri::evict_step(cache, params, scores, keep, new_lengths, block_table_out, freed, n_freed, ws, ws_bytes,
                         stream, events, false);
}

}  // extern "C"
