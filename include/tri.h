/*
 * tri.h - C ABI of the TriAttention KV-cache eviction pass on MI355X (gfx950).
 *
 * The pass ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-5;
 * "WeianMao/triattention", How it works) scores every cached key from
 * pre-rotation query centres and norm statistics, keeps the best keys up to a
 * budget per (layer, sequence, KV head) -- the "unit" -- and compacts the kept
 * K/V rows and their position ids to the front of the unit's cache.
 *
 * Score of slot p of a unit (stored, already rotated key K[p]; G query heads per
 * KV head; offsets D; decode position t of the sequence):
 *   s(p) = (1/G) sum_g [ (1/|D|) sum_{Delta} RoPE(qbar_g, t+Delta) . K[p] + sum_i c_{g,i} |z_i(K[p])| ]
 * which the library evaluates in the equivalent collapsed form
 *   s(p) = w . K[p] + sum_i chat_i |z_i(K[p])|,  w = RoPE(u, t),
 *   u = mean_{g,Delta} RoPE(qbar_g, Delta),  chat = mean_g c_g,
 * where z_i is the i-th rotary pair and RoPE multiplies z_i by exp(j n theta^(-2i/d)).
 *
 * Conventions for every call:
 *  - All pointers are DEVICE pointers unless the argument says "host".
 *  - The caller owns and allocates every buffer (including the workspace); the
 *    library never allocates, frees, synchronises or copies device->host.
 *  - Work is enqueued asynchronously on `stream`; a call returns as soon as its
 *    kernels are enqueued.
 *  - Arguments are validated on the host before anything is enqueued: on any
 *    non-OK status nothing was enqueued and tri_last_error() describes why.
 *  - Launch failures return TRI_ERR_HIP.  Device-side data preconditions
 *    (listed per call) are checked only when tri_params.check is given;
 *    otherwise violating them gives unspecified results.
 *  - The only global state is a thread-local error string (and the device array of
 *    tri_evict_step_noalloc).  Calls on distinct streams with distinct buffers may
 *    run concurrently.
 */
#ifndef TRI_H
#define TRI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRI_OK = 0,
  TRI_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad budget/recent, misalignment */
  TRI_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, dtype, length beyond limits */
  TRI_ERR_WORKSPACE = 3,     /* ws_bytes smaller than tri_workspace_bytes() */
  TRI_ERR_HIP = 4            /* a HIP launch failed; tri_last_error() has hipGetErrorString */
} tri_status;

typedef enum { TRI_BF16 = 0, TRI_F32 = 1 } tri_dtype;
typedef enum { TRI_CONTIGUOUS = 0, TRI_PAGED = 1 } tri_layout;
/* Rotary pairing: HALF pairs dims (i, i + d/2) (rotate-half, Qwen family); INTERLEAVED pairs (2i, 2i+1). */
typedef enum { TRI_ROPE_HALF = 0, TRI_ROPE_INTERLEAVED = 1 } tri_rope;

/* Largest cached length per unit the selection kernel accepts. */
#define TRI_MAX_LEN 65536
/* Largest number of offsets Delta accepted by tri_prepare_centres. */
#define TRI_MAX_OFFSETS 64
#define TRI_FUSED_MAX_LEN 8192      /* longest cache the fused pass takes */
#define TRI_FUSED_MAX_BLOCKS 1024   /* paged: most block-table entries per sequence the fused pass takes */
#define TRI_FUSED_MIN_UNITS 2048    /* fewest units for which the fused pass is the default */
#define TRI_PASS_UNFUSED 1          /* tri_params.flags: always run score, select and compact as three kernels */
#define TRI_PASS_FUSED 2            /* tri_params.flags: fused pass whenever the caches fit it */

/*
 * The cache of `num_layers` layers.  K and V share one layout and one set of strides.
 *
 * TRI_CONTIGUOUS: element e of the row of (layer l, sequence b, KV head h, slot s) is at
 *     k[l*layer_stride + b*stride_b + h*stride_h + s*stride_s + e]   (same for v),
 *   and its position id at pos[l*pos_layer_stride + b*pos_stride_b + h*pos_stride_h + s].
 *   Slots 0 .. max_len-1 exist per unit.  Any stride order works (head-major or token-major);
 *   rows must be 16-byte aligned (every stride times the element size a multiple of 16), and one
 *   unit's rows must span less than 2^31 bytes (max_len * stride_s * element size), else
 *   TRI_ERR_UNSUPPORTED.
 *
 * TRI_PAGED: per layer a pool of num_blocks blocks of block_size slots:
 *     k[l*layer_stride + ((blk*block_size + o)*num_kv_heads + h)*head_dim + e]
 *     pos[l*pos_layer_stride + (blk*block_size + o)*num_kv_heads + h]
 *   Logical slot s of sequence b is block block_table[b*max_blocks_per_seq + s/block_size],
 *   offset o = s % block_size.  One block table serves every layer.  max_len is ignored;
 *   the per-unit slot capacity is max_blocks_per_seq*block_size.  stride_* are ignored.
 *
 * Position ids must increase along the slots of every unit (true of a fresh cache and kept
 * by compaction): ties in score are broken by lower slot, which is then lower position.
 */
typedef struct tri_cache {
  int32_t layout;            /* tri_layout */
  int32_t dtype;             /* tri_dtype, storage type of k and v */
  int32_t rope;              /* tri_rope */
  int32_t num_layers;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;          /* 64 or 128 */
  int32_t max_len;           /* contiguous only */
  void *k;
  void *v;
  int32_t *pos;
  int64_t layer_stride, stride_b, stride_h, stride_s;          /* elements of k/v */
  int64_t pos_layer_stride, pos_stride_b, pos_stride_h;        /* elements of pos */
  int32_t block_size;        /* paged only */
  int32_t num_blocks;        /* paged only */
  int32_t max_blocks_per_seq;/* paged only */
  int32_t reserved;
  const int32_t *block_table;/* paged only: [batch][max_blocks_per_seq] */
} tri_cache;

/*
 * Per-pass parameters.
 *   u       float [num_layers][num_kv_heads][head_dim]  from tri_prepare_centres
 *   c_hat   float [num_layers][num_kv_heads][head_dim/2] from tri_prepare_centres
 *   lengths int32 [batch]: cached slots per sequence (same for every layer and head).
 *           Precondition: 0 <= lengths[b] <= slot capacity and <= TRI_MAX_LEN.
 *   t       int32 [batch]: current decode position of each sequence (>= the largest cached
 *           position; equal to lengths[b] for a cache that was never compacted).
 *   budget  slots kept per unit, >= 1;  recent: the last `recent` slots are always kept,
 *           0 <= recent <= budget.
 *   max_length  0, or a host-side bound on every lengths[b] (1 <= max_length <= slot capacity).
 *           lengths live on the device, so launches are otherwise sized by the slot capacity; a
 *           bound sizes them by it instead, which pays when caches are far shorter than their
 *           capacity (the recurring pass at budget plus a few decode steps).  Precondition when
 *           nonzero: lengths[b] <= max_length (slots past it are neither scored nor kept).
 *   flags   0, TRI_PASS_UNFUSED or TRI_PASS_FUSED.  tri_evict_step can run the pass as one kernel
 *           with one workgroup per unit (scores and keep list held in LDS) when every cache is at most
 *           TRI_FUSED_MAX_LEN slots -- the slot capacity, or max_length when given -- and paged block
 *           tables need at most TRI_FUSED_MAX_BLOCKS entries per sequence.  With flags 0 it does so
 *           when there are also at least TRI_FUSED_MIN_UNITS units (fewer leave most of the GPU idle);
 *           TRI_PASS_FUSED drops that condition; TRI_PASS_UNFUSED always runs the three-kernel sequence
 *           (score, select, compact).  Every path gives bitwise identical results.
 *   check   NULL, or a device word.  When given, tri_score, tri_topk, tri_compact and tri_evict_step* first check
 *           the device-side data preconditions: every lengths[b] within 0 .. slot capacity (and <= max_length
 *           when given), every t[b] >= lengths[b], for a paged cache every used block-table entry (the first
 *           ceil(lengths[b] / block_size) of each row) within 0 .. num_blocks-1, and in the calls that compact no
 *           block id used by two entries.  They write the TRI_CHECK_* bits of those violated into *check (0 when
 *           all hold); if any is, every kernel of the call returns without reading or writing the cache.  The
 *           caller reads the word once the call's work is done.  Without it these preconditions are not checked
 *           and violating them gives unspecified results, out-of-bounds accesses included.
 */
typedef struct tri_variant tri_variant;

/* Bits of tri_params.check: the device-side data preconditions a checked call found violated. */
#define TRI_CHECK_LENGTH 1u        /* some lengths[b] < 0, > slot capacity, or > max_length when given */
#define TRI_CHECK_DECODE_POS 2u    /* some t[b] < lengths[b] */
#define TRI_CHECK_BLOCK_RANGE 4u   /* paged: a used block-table entry outside 0 .. num_blocks-1 */
#define TRI_CHECK_BLOCK_DUP 8u     /* paged, calls that compact: one block id used by two table entries */

typedef struct tri_params {
  const float *u;
  const float *c_hat;
  double rope_theta;
  const int32_t *lengths;
  const int32_t *t;
  int32_t budget;
  int32_t recent;
  int32_t max_length;
  int32_t flags;
  const tri_variant *variant;   /* HOST pointer; NULL for the collapsed score (see tri_variant) */
  uint32_t *check;              /* DEVICE word or NULL: check the device-side preconditions first (below) */
} tri_params;

/*
 * Aggregation variants of the score ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 step 2 and
 * 复现注意事项: the pages leave the aggregation of the distance series open).  The collapsed score averages
 * the rotary logits RoPE(qbar_g, t + Delta) . K[p] over the query heads g of the KV head's group and the
 * offsets Delta, which collapses to one dot product.  A variant aggregates them otherwise:
 *   TRI_AGG_MAX       max over heads and offsets
 *   TRI_AGG_HEAD_MAX  mean over heads of the max over offsets
 * plus the same norm term (c_hat . |z(K[p])|).  Such scores need every logit: a [keys x d] . [d x G|D|] product
 * per unit, which runs on the matrix cores (bf16 caches only; w split into a bf16 high part and residual).
 *   centres     float [num_layers][num_kv_heads][tri_variant_columns(group, n_offsets)][head_dim] from
 *               tri_prepare_variant_centres (device)
 *   group       query heads per KV head;  n_offsets  1..32 (as given to tri_prepare_variant_centres); supported
 *               when tri_variant_columns(group, n_offsets) is nonzero (e.g. 8 heads with up to 16 offsets, 4 heads
 *               with up to 32)
 * With a variant, tri_evict_step always runs the separate scoring kernel; u is unused (c_hat still is).
 */
#define TRI_AGG_MAX 1
#define TRI_AGG_HEAD_MAX 2
struct tri_variant {
  const float *centres;
  int32_t aggregation;
  int32_t group;
  int32_t n_offsets;
  int32_t reserved;      /* must be 0 */
};

/*
 * Columns per (layer, KV head) of a variant's rotated centres: each query head of the group takes a block of
 * dpad = 16 columns (n_offsets <= 16) or 32 (n_offsets <= 32), and the blocks are padded to 64 or 128 columns.
 * 0 when the group's blocks exceed 128 columns or the arguments are out of range (the variant is not supported).
 */
int32_t tri_variant_columns(int32_t group, int32_t n_offsets);

/*
 * Rotated centres for the aggregation variants: centres[l][h][g*dpad + k] = RoPE(qbar[l][h*G + g], offsets[k])
 * (float64, rounded once) for g < G = h_q / h_kv and k < n_offsets, zero elsewhere, with
 * tri_variant_columns(G, n_offsets) columns per (l, h) and dpad as described there.  qbar as for
 * tri_prepare_centres (device), offsets a HOST array.  Run once per change of centres.
 */
tri_status tri_prepare_variant_centres(const float *qbar, int32_t num_layers, int32_t h_q, int32_t h_kv,
                                       int32_t head_dim, double rope_theta, int32_t rope, const int32_t *offsets,
                                       int32_t n_offsets, float *centres, hipStream_t stream);

/*
 * Centre vectors of the collapsed score ("TriAttention：基于三角函数 KV 压缩的高效长推理",
 * 流程详解 steps 1-3: centres from calibration, distance series, norm weighting).
 *   qbar  float [num_layers][h_q][head_dim]  pre-rotation query centres (device)
 *   c     float [num_layers][h_q][head_dim/2] norm coefficients per rotary pair (device)
 *   offsets int32 [n_offsets] HOST array of future offsets Delta, 1 <= n_offsets <= TRI_MAX_OFFSETS
 *   u     float [num_layers][h_kv][head_dim] out: mean over the group's query heads g
 *         (query head hq belongs to KV head hq / (h_q/h_kv)) and over Delta of RoPE(qbar_g, Delta),
 *         computed in float64, rounded once
 *   c_hat float [num_layers][h_kv][head_dim/2] out: group mean of c
 * h_q must be a positive multiple of h_kv.  Run once per change of centres.
 */
tri_status tri_prepare_centres(const float *qbar, const float *c, int32_t num_layers, int32_t h_q,
                               int32_t h_kv, int32_t head_dim, double rope_theta, int32_t rope,
                               const int32_t *offsets, int32_t n_offsets, float *u, float *c_hat,
                               hipStream_t stream);

/* Slots per unit in the scores buffer: the slot capacity rounded up to a multiple of 64. */
int64_t tri_score_stride(const tri_cache *cache);

/*
 * Bytes of workspace tri_evict_step / tri_compact need (depends on shapes only).  0 on bad input.
 * The workspace needs no initialization: every word a pass reads was written earlier in the same pass.
 * A workspace must not be shared by passes that run concurrently.
 */
size_t tri_workspace_bytes(const tri_cache *cache, const tri_params *params);

/*
 * Score every cached key ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-3).
 *   scores float [num_layers][batch][num_kv_heads][tri_score_stride(cache)] out; entry s of a unit
 *   is written for s < lengths[b] only.  Float32 accumulation; w = RoPE(u, t_b) is formed with
 *   float64 angles.
 */
tri_status tri_score(const tri_cache *cache, const tri_params *params, float *scores, hipStream_t stream);

/*
 * Select the kept slots of every unit (流程详解 step 4).  If L = lengths[b] <= budget every slot is
 * kept.  Otherwise the last `recent` slots are kept, plus the best budget-recent of slots
 * 0 .. L-recent-1 ordered by score (higher first; NaN lowest, -0 equal to +0) then by slot (lower
 * first).  keep int32 [units][budget] out: the kept slots of the unit in ascending order (entries
 * past min(L, budget) are not written).  new_lengths int32 [batch] out: min(L, budget).
 */
tri_status tri_topk(const tri_cache *cache, const tri_params *params, const float *scores,
                    int32_t *keep, int32_t *new_lengths, hipStream_t stream);

/*
 * Compact every unit in place (流程详解 step 5): for j < min(L, budget), row j of K and V and pos[j]
 * become row keep[j] / pos[keep[j]] of the unit, bit for bit.  Units with L <= budget are untouched.
 * Slots past min(L, budget) are left unspecified.  Paged caches additionally get
 *   block_table_out int32 [batch][ceil(budget/block_size)]: the first ceil(min(L,budget)/block_size)
 *     entries of each sequence's table (the rest of the row is not written);
 *   freed int32 [sum_b ceil(L_b/block_size)] out: for each sequence in order, its blocks past those,
 *     in logical order;  n_freed int32 [1] out: their number.
 * For contiguous caches block_table_out, freed and n_freed must be NULL.
 * ws / ws_bytes: workspace of at least tri_workspace_bytes(cache, params) bytes.
 */
tri_status tri_compact(const tri_cache *cache, const tri_params *params, const int32_t *keep,
                       int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The whole eviction pass ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-5; "WeianMao/triattention",
 * How it works): score every cached key of every unit, keep the recent window and the best candidates up to the
 * budget, and compact the kept rows in place -- tri_score, tri_topk and tri_compact in one launch sequence over all
 * layers, with results bit for bit those of the three calls.  Depending on the shapes it runs as three kernels, as
 * two (scoring, then one workgroup per unit that selects and compacts, for many units), or as one fused kernel for
 * short caches (tri_params.flags).  scores and keep may be NULL, in which case they live in the workspace; when
 * given they receive the same contents as from the separate calls.  new_lengths int32 [batch] out (must not alias
 * lengths); block_table_out, freed, n_freed as for tri_compact.  All buffers are the caller's; nothing is allocated
 * and nothing waits on the host.  A non-OK status means nothing was enqueued (tri_last_error says why).
 */
tri_status tri_evict_step(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                          int32_t *new_lengths, int32_t *block_table_out, int32_t *freed,
                          int32_t *n_freed, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * tri_evict_step that also records events[0..3] (HOST array of caller-created hipEvent_t) on `stream`:
 * before the scoring launch, between scoring and selection, between selection and compaction, and
 * after compaction, so a caller can time each kernel of the pass on the stream it runs on.
 */
tri_status tri_evict_step_profiled(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                                   int32_t *new_lengths, int32_t *block_table_out, int32_t *freed,
                                   int32_t *n_freed, void *ws, size_t ws_bytes, hipStream_t stream,
                                   const hipEvent_t *events);

/*
 * tri_evict_step for callers that cannot allocate device memory when they call it (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the workspace's control words (per-unit tickets, score
 * ranges, chunk flags) live in an array the library owns, TRI_NOALLOC_SCRATCH_BYTES bytes per device, held from the
 * first call on a device until the process ends.  Nothing is allocated and nothing needs clearing: every word a
 * call reads was written earlier in the same call.  scores and keep are outputs the caller passes (non-NULL); the
 * other arguments, results and errors are as for tri_evict_step, which this call matches bit for bit.  Shapes
 * whose control words exceed the array (tri_workspace_bytes less the keep and score parts) give
 * TRI_ERR_UNSUPPORTED.  All calls on one device share its array: calls that overlap on one device (concurrent
 * streams, other threads) race and must not be issued.  The current device must be the one the buffers and
 * `stream` belong to.
 */
#define TRI_NOALLOC_SCRATCH_BYTES (16u << 20)
tri_status tri_evict_step_noalloc(const tri_cache *cache, const tri_params *params, float *scores, int32_t *keep,
                                  int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                                  hipStream_t stream);

/*
 * Decode attention over the kept cache ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 step 5:
 * inference attends over the compressed cache).  For every layer l, sequence b and query head hq (of KV head
 * hq / (h_q / num_kv_heads)):
 *     out[l][b][hq] = sum over slots p < lengths[b] of softmax_p(scale * q[l][b][hq] . K[p]) * V[p]
 * (0 when lengths[b] is 0), split over chunks of slots and combined exactly (running max and sum).  It reads
 * the cache the way the pass leaves it: pass tri_evict_step's new_lengths and, for a paged cache, a cache
 * whose block_table is its block_table_out (max_blocks_per_seq = ceil(budget / block_size)).
 *   cache       as for the pass; K and V are only read
 *   lengths     int32 [batch] device;  max_length  host bound on lengths, 1 .. slot capacity (sizes the splits)
 *   q           [num_layers][batch][h_q][head_dim] in the cache's dtype, device, 16-byte aligned
 *   h_q         a multiple of num_kv_heads with h_q / num_kv_heads = 1, 2 or a multiple of 4
 *   scale       logit scale (1/sqrt(head_dim) for standard attention)
 *   out         float [num_layers][batch][h_q][head_dim]
 *   ws          tri_decode_workspace_bytes(cache, h_q, max_length) bytes, 256-byte aligned, no initialization
 *               needed; not to be shared by concurrent calls
 * Precondition: lengths[b] <= max_length (slots past it are ignored).
 */
size_t tri_decode_workspace_bytes(const tri_cache *cache, int32_t h_q, int32_t max_length);
tri_status tri_decode_attention(const tri_cache *cache, const int32_t *lengths, int32_t max_length, const void *q,
                                int32_t h_q, float scale, float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Calibration statistics ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 step 1: query centres
 * measured on a calibration set; step 3: norm weighting).  From n pre-rotation queries per (layer, query
 * head): qbar = their mean, and c_i = mean over the queries of |z_i(q)| minus |z_i(qbar)| (z_i the i-th
 * rotary pair, paired as `rope` says), the norm mass the centre does not carry.  These are the qbar and c
 * that tri_prepare_centres takes.
 *   queries  element e of the query of (layer l, calibration token j, query head h) at
 *            q[l*stride_l + j*stride_n + h*stride_h + e] (dtype TRI_BF16 or TRI_F32; e contiguous; base and
 *            every stride times the element size 16-byte aligned)
 *   qbar     float [num_layers][num_heads][head_dim] out;  c  float [num_layers][num_heads][head_dim/2] out
 *   ws       caller-owned workspace of tri_calibrate_workspace_bytes(queries) bytes, 256-byte aligned; it needs
 *            no initialization and must not be shared by calls that run concurrently
 * Sums run in float64 in a fixed order (pair norms in float32 from the stored values), so results are
 * deterministic.  Errors as for the other calls: everything is checked before anything is enqueued.
 */
typedef struct tri_queries {
  int32_t dtype;             /* tri_dtype */
  int32_t rope;              /* tri_rope */
  int32_t num_layers;
  int32_t num_heads;         /* query heads */
  int32_t head_dim;          /* 64 or 128 */
  int32_t reserved;          /* must be 0 */
  int64_t n;                 /* calibration queries per (layer, head), >= 1 */
  const void *q;
  int64_t stride_l, stride_n, stride_h;   /* elements */
} tri_queries;

size_t tri_calibrate_workspace_bytes(const tri_queries *queries);
tri_status tri_calibrate(const tri_queries *queries, float *qbar, float *c, void *ws, size_t ws_bytes,
                         hipStream_t stream);

const char *tri_status_string(tri_status status);
/* Message for the last non-OK status returned on this thread ("" if none). */
const char *tri_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TRI_H */
