// gfx950 kernels of the TriAttention KV-cache eviction pass.
//
// Method ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-5; "WeianMao/triattention",
// How it works): every cached key gets a score from pre-rotation query centres (a series of
// sinusoids of the query-key distance) plus a norm weighting; the best keys up to a budget are
// kept per (layer, sequence, KV head) and compacted to the front of the cache.
//
// The distance series is linear in the stored key, so for one unit it collapses to a single dot
// product with w = RoPE(u, t) plus sum_i chat_i |z_i(K)|.  That is ~2.5 flop per byte of K: the
// pass is HBM-bound and the kernels below are built around streaming, not matrix cores.
//
//   k_prepare  u, chat from the query centres and norm statistics (float64, once per centre set)
//   k_score    streams K with 128-bit loads, one 4-wave workgroup per half of a 1024-row tile; lane s of a
//              row's lane group loads chunk s of each rotary half, so half-split pairs meet inside the lane;
//              bf16 math runs on v_dot2_f32_bf16 with no conversions; the row sum is a DPP butterfly.
//   k_select   one workgroup per unit; per-slot bins stay in registers; a value-space histogram between the
//              candidates' min and max picks the bin of the threshold, an exact radix select over that
//              bin's members gives it; ties go to the lower slot; two block scans emit the ascending keep
//              list.  With MOVE the same workgroup then compacts its unit (move_unit), for passes with many
//              units, so one unit's selection latency overlaps other units' moves.
//   k_compact  workgroups take per-unit ordered tickets for destination chunks; each loads the rows it
//              moves, publishes "sources loaded", waits only for earlier chunks of its unit whose
//              sources reach into its destination range, then stores.  Destination j <= source
//              keep[j] makes that the only hazard of the in-place move.
//   k_fused    the whole pass for caches of at most 8192 slots, one workgroup per unit: scores as order
//              keys in LDS, an exact radix select there, then the in-place moves in ascending chunks.
//
// Around the pass (the steps before and after it, and variants of its score):
//   k_calib_partial / k_calib_finish   query centres and missed pair-norm mass from calibration queries
//                                      (float64 sums per token chunk, combined in a fixed order)
//   k_decode_partial / k_decode_combine  decode attention over the kept cache (split-K online softmax)
//   k_prepare_variant / k_score_var    scores that aggregate the rotary logits with a max, so they do not
//                                      collapse: every logit from a bf16 matrix-core chain
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tri_checks.h"
#include "tri_internal.h"

namespace tri {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of LPR lanes (LPR in {4, 8, 16, 32}); every lane gets the sum.
// After the two quad steps the four lanes of a quad agree, so the mirrors act as xor 4 / xor 8.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_f32<kDppMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// A checked call whose preconditions failed: every kernel of the pass returns at entry (nothing is read or written).
__device__ __forceinline__ bool checks_failed(const PassView &pv) { return pv.check != nullptr && *pv.check != 0u; }

// Workgroups are dealt to the chip's XCDs (each with its own L2) round-robin.  For kernels that move rows of a
// paged pool, workgroup i takes unit xcd_grouped_unit(i): the workgroups of XCD x take the (layer, sequence)
// pairs lb = x, x + kXcds, ..., all heads of each in a row.  A paged slot keeps the position ids of all its heads in
// one 32-byte segment; with the heads' moves in one L2 their 4-byte reads and writes of that segment meet there
// instead of each costing a partial-line transfer to HBM.  -1: a padding workgroup (grid xcd_grouped_grid).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_grouped_unit(int i, int heads, int pairs) {
  const int x = i % kXcds, q = i / kXcds;
  const int lb = (q / heads) * kXcds + x;
  return lb < pairs ? lb * heads + q % heads : -1;
}
inline int64_t xcd_grouped_grid(int heads, int pairs) { return (int64_t)(pairs + kXcds - 1) / kXcds * kXcds * heads; }

// ------------------------------------------------------------------------------------ prepare

struct Offsets { int32_t v[TRI_MAX_OFFSETS]; };

// One workgroup per (layer, KV head); thread i owns rotary pair i.
//   u_i    = mean_g z_i(qbar_g) * mean_Delta exp(j Delta omega_i)   (= mean_{g,Delta} RoPE(qbar_g, Delta))
//   chat_i = mean_g c_{g,i}
__global__ void k_prepare(const float *__restrict__ qbar, const float *__restrict__ c, int h_q, int h_kv,
                          int d, double theta, int rope, Offsets offs, int n_off, float *__restrict__ u,
                          float *__restrict__ c_hat) {
  const int lh = blockIdx.x;
  const int l = lh / h_kv, h = lh % h_kv;
  const int G = h_q / h_kv;
  const int i = threadIdx.x;
  if (i >= d / 2) return;
  const double om = pow(theta, -2.0 * i / d);
  double es = 0.0, ec = 0.0;
  for (int k = 0; k < n_off; ++k) {
    double s, co;
    sincos((double)offs.v[k] * om, &s, &co);
    ec += co;
    es += s;
  }
  const int pa = rope == TRI_ROPE_HALF ? i : 2 * i;
  const int pb = rope == TRI_ROPE_HALF ? i + d / 2 : 2 * i + 1;
  double qa = 0.0, qb = 0.0, cs = 0.0;
  for (int g = 0; g < G; ++g) {
    const int64_t row = (int64_t)l * h_q + (int64_t)h * G + g;
    qa += qbar[row * d + pa];
    qb += qbar[row * d + pb];
    cs += c[row * (d / 2) + i];
  }
  const double inv = 1.0 / ((double)G * n_off);
  u[(int64_t)lh * d + pa] = (float)((qa * ec - qb * es) * inv);
  u[(int64_t)lh * d + pb] = (float)((qa * es + qb * ec) * inv);
  c_hat[(int64_t)lh * (d / 2) + i] = (float)(cs / G);
}

// Rotated centres of the aggregation variants: one workgroup per (layer, KV head); of the `ncol` columns, column
// g*dpad + k holds RoPE(qbar_g, offsets[k]) in float64, rounded once; columns past the group or the offsets hold
// zeros.
__global__ void k_prepare_variant(const float *__restrict__ qbar, int h_q, int h_kv, int d, double theta, int rope,
                                  Offsets offs, int n_off, int ncol, int dpad, float *__restrict__ centres) {
  const int lh = blockIdx.x;
  const int l = lh / h_kv, h = lh % h_kv;
  const int G = h_q / h_kv;
  for (int idx = threadIdx.x; idx < ncol * (d / 2); idx += blockDim.x) {
    const int col = idx / (d / 2), i = idx % (d / 2);
    const int g = col / dpad, k = col % dpad;
    const int pa = rope == TRI_ROPE_HALF ? i : 2 * i;
    const int pb = rope == TRI_ROPE_HALF ? i + d / 2 : 2 * i + 1;
    float *out = centres + ((int64_t)lh * ncol + col) * d;
    if (g >= G || k >= n_off) {
      out[pa] = 0.f;
      out[pb] = 0.f;
      continue;
    }
    const int64_t row = (int64_t)l * h_q + (int64_t)h * G + g;
    const double qa = qbar[row * d + pa], qb = qbar[row * d + pb];
    double sn, cs;
    sincos((double)offs.v[k] * pow(theta, -2.0 * i / d), &sn, &cs);
    out[pa] = (float)(qa * cs - qb * sn);
    out[pb] = (float)(qa * sn + qb * cs);
  }
}

// ------------------------------------------------------------------------------------ score

// Order-preserving map of a float score to uint32: larger score -> larger key.  NaN ranks as -inf
// and -0 as +0, so equal keys mean equal rank values.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) x = 0xff800000u;
  if (x == 0x80000000u) x = 0u;
  return (x & 0x80000000u) ? ~x : (x | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {  // inverse of order_key (canonical NaN -> -inf)
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}


// Rows in flight per lane of the scoring kernel (the measured best on MI355X).
constexpr int64_t kTemporalKeyBytes = 192ll << 20;   // scored keys up to this size are loaded through the caches
constexpr int kScoreUnroll = 8;
constexpr int kScoreUnrollPaged = 2;   // paged rows are 2 KB apart: fewer rows in flight, more waves resident

// Key loads of the scoring kernels are non-temporal: each key row is read once per pass (but see kTemporalKeyBytes).
template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
  return __builtin_nontemporal_load(p);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
// a.lo*b.lo + a.hi*b.hi + c with float32 accumulation (v_dot2_f32_bf16); bf16 products are exact in float32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}
// Two bf16 into one dword: lo from the low half of x, hi from the low half of y (or the high halves).
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }
__device__ __forceinline__ uint32_t bf16_bits(float f) {  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One cached row as a lane holds it: 16 bytes of each rotary half (chunk `seg` of the half).
struct KRow { u32x4 a, b; };

// Score math of one row, shared by the scoring and fused kernels.  A row of d elements is split into its two
// rotary halves; lane s of a row's LPR-lane group holds 16 bytes at chunk s of each half, so with the
// half-split pairing element k of the first chunk and element k of the second chunk form a rotary pair inside
// the lane.  bf16 rows use v_dot2_f32_bf16 directly on the stored pairs: for |z|^2 on (a, b) packed together,
// and for w . K with w split exactly into a bf16 high part and a bf16 residual (error <= 2^-18 |w| per element).
template <int DT, int D, int ROPE>
struct RowScorer {
  static constexpr int E = DT == TRI_BF16 ? 2 : 4;
  static constexpr int HB = D * E / 2;   // bytes per rotary half of a row
  static constexpr int LPR = HB / 16;    // lanes per row
  static constexpr int VPC = 16 / E;     // elements per 16-byte chunk
  static constexpr bool HALF = ROPE == TRI_ROPE_HALF;

  float cr[VPC];
  uint32_t wa_hi[4], wa_lo[4], wb_hi[4], wb_lo[4];
  float wfa[4], wfb[4];

  // w = RoPE(u, t) (angles and products in float64, rounded once) and chat of unit (layer, KV head) `ukv`
  // into LDS; threads 0 .. D/2-1 take one rotary pair each.
  static __device__ void centre(const PassView &pv, int64_t ukv, int t, float *s_w, float *s_c, int tid) {
    if (tid < D / 2) centre_pair(pv, ukv, t, tid, s_w, s_c);
  }
  // rotary pair i of w and chat_i
  static __device__ void centre_pair(const PassView &pv, int64_t ukv, int t, int i, float *s_w, float *s_c) {
    const double om = pow(pv.theta, -2.0 * i / D);
    double sn, cs;
    sincos((double)t * om, &sn, &cs);
    const int pa = HALF ? i : 2 * i;
    const int pb = HALF ? i + D / 2 : 2 * i + 1;
    const double ua = pv.u[ukv * D + pa], ub = pv.u[ukv * D + pb];
    s_w[pa] = (float)(ua * cs - ub * sn);
    s_w[pb] = (float)(ua * sn + ub * cs);
    s_c[i] = pv.c_hat[ukv * (D / 2) + i];
  }

  // Per-lane constants: w for the lane's 2*VPC dims and chat for its VPC pairs.
  __device__ void init(const float *s_w, const float *s_c, int seg) {
    const int da = seg * VPC, db = D / 2 + seg * VPC;   // first dim of chunk a / chunk b
    if constexpr (HALF) {
#pragma unroll
      for (int k = 0; k < VPC; ++k) cr[k] = s_c[da + k];
    } else {
#pragma unroll
      for (int k = 0; k < VPC / 2; ++k) {
        cr[k] = s_c[da / 2 + k];
        cr[VPC / 2 + k] = s_c[db / 2 + k];
      }
    }
    // bf16: w as packed (hi, residual) bf16 pairs matching the data dwords; f32: plain floats.
    if constexpr (DT == TRI_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = s_w[da + 2 * i], x1 = s_w[da + 2 * i + 1];
        uint32_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
        uint32_t l0 = bf16_bits(x0 - __uint_as_float(h0 << 16)), l1 = bf16_bits(x1 - __uint_as_float(h1 << 16));
        wa_hi[i] = h0 | (h1 << 16);
        wa_lo[i] = l0 | (l1 << 16);
        x0 = s_w[db + 2 * i];
        x1 = s_w[db + 2 * i + 1];
        h0 = bf16_bits(x0);
        h1 = bf16_bits(x1);
        l0 = bf16_bits(x0 - __uint_as_float(h0 << 16));
        l1 = bf16_bits(x1 - __uint_as_float(h1 << 16));
        wb_hi[i] = h0 | (h1 << 16);
        wb_lo[i] = l0 | (l1 << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wfa[i] = s_w[da + i];
        wfb[i] = s_w[db + i];
      }
    }
  }

  // The row's score, complete in every lane of its group (DPP butterfly over the LPR lanes).
  __device__ float operator()(const KRow &x) const {
    float dot = 0.f, nrm = 0.f;
    if constexpr (DT == TRI_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dot = dot2(wa_hi[i], x.a[i], dot);
        dot = dot2(wa_lo[i], x.a[i], dot);
        dot = dot2(wb_hi[i], x.b[i], dot);
        dot = dot2(wb_lo[i], x.b[i], dot);
      }
      if constexpr (HALF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t p0 = pack_lo(x.a[i], x.b[i]), p1 = pack_hi(x.a[i], x.b[i]);
          nrm = fmaf(cr[2 * i], __builtin_amdgcn_sqrtf(dot2(p0, p0, 0.f)), nrm);
          nrm = fmaf(cr[2 * i + 1], __builtin_amdgcn_sqrtf(dot2(p1, p1, 0.f)), nrm);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          nrm = fmaf(cr[i], __builtin_amdgcn_sqrtf(dot2(x.a[i], x.a[i], 0.f)), nrm);
          nrm = fmaf(cr[4 + i], __builtin_amdgcn_sqrtf(dot2(x.b[i], x.b[i], 0.f)), nrm);
        }
      }
    } else {
      float fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = __uint_as_float(x.a[i]);
        fb[i] = __uint_as_float(x.b[i]);
        dot = fmaf(wfa[i], fa[i], dot);
        dot = fmaf(wfb[i], fb[i], dot);
      }
      if constexpr (HALF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) nrm = fmaf(cr[i], __builtin_amdgcn_sqrtf(fmaf(fa[i], fa[i], fb[i] * fb[i])), nrm);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          nrm = fmaf(cr[i], __builtin_amdgcn_sqrtf(fmaf(fa[2 * i], fa[2 * i], fa[2 * i + 1] * fa[2 * i + 1])), nrm);
          nrm = fmaf(cr[2 + i], __builtin_amdgcn_sqrtf(fmaf(fb[2 * i], fb[2 * i], fb[2 * i + 1] * fb[2 * i + 1])), nrm);
        }
      }
    }
    return group_sum<LPR>(dot + nrm);
  }
};

// Grid: (((layer*batch + seq)*tiles + tile)*kRangeParts + part)*heads + head.  A workgroup of kRangeWaves waves
// scores one range part of a kScoreTile-row tile of one unit (512 rows) and fills that part's range slot; each wave
// owns 128 contiguous rows, lane groups of LPR lanes per row (see RowScorer).  (Whole-tile workgroups of 8 waves
// fit once per compute unit at this kernel's register count, leaving a third of the wave slots empty; half-tile
// ones fit three times.)
// TEMP: key loads through the caches instead of non-temporal ones, for passes whose scored keys fit in the last-level
// cache: the compaction that follows then finds the kept K rows there.
template <int DT, int D, int ROPE, int PAGED, int TEMP>
__global__ __launch_bounds__(64 * kRangeWaves) void k_score(CacheView cv, PassView pv, float *__restrict__ scores,
                                                int64_t score_stride, int tiles, uint32_t *__restrict__ range) {
  // Contiguous caches address a unit's rows as a uniform base plus a 32-bit per-lane byte offset (the host
  // only launches this form when capacity * row stride fits in 31 bits); paged rows use 64-bit addresses.
  constexpr int E = DT == TRI_BF16 ? 2 : 4;
  constexpr int HB = D * E / 2;              // bytes per rotary half of a row
  constexpr int LPR = HB / 16;               // lanes per row
  constexpr int RPW = 64 / LPR;              // rows per wave per load
  constexpr int WAVES = kRangeWaves;
  constexpr int ROWS_PER_WAVE = kScoreTile / kScoreWaves;
  constexpr int SPAN = WAVES * ROWS_PER_WAVE;    // rows per workgroup
  constexpr int PARTS = kRangeParts;             // workgroups per tile
  static_assert(PARTS * WAVES == kScoreWaves, "a workgroup fills one range slot");
  constexpr int UNR_WANT = PAGED ? kScoreUnrollPaged : kScoreUnroll;
  constexpr int UNR = UNR_WANT * RPW <= ROWS_PER_WAVE ? UNR_WANT : ROWS_PER_WAVE / RPW;  // rows in flight
  constexpr int STEP = RPW * UNR;
  constexpr int ITERS = ROWS_PER_WAVE / STEP;
  static_assert(UNR >= 1 && ITERS >= 1 && ITERS * STEP == ROWS_PER_WAVE, "tile shape");
  static_assert(LPR >= 4 && LPR <= 16, "lanes per row");

  __shared__ float s_w[D];
  __shared__ float s_c[D / 2];
  __shared__ int64_t s_blk[PAGED ? SPAN : 1];  // paged: byte offset of this head's row 0 in every block the span touches
  __shared__ uint32_t s_rng[WAVES][2];          // per wave: min and max order key of its scores

  if (checks_failed(pv)) return;
  const int H = cv.heads;
  int bid = blockIdx.x;
  const int h = bid % H;
  bid /= H;
  const int part = bid % PARTS;
  bid /= PARTS;
  const int tile = bid % tiles;
  bid /= tiles;
  const int b = bid % cv.batch;
  const int l = bid / cv.batch;
  const int L = pv.lengths[b];
  const int tile0 = tile * kScoreTile + part * SPAN;   // first row of this workgroup
  if (tile0 >= L) {
    // A tile that holds keys has every range slot written (the selection reads them): rows past the length add
    // the neutral pair (key(+inf), key(-inf)).
    if (range != nullptr && tile * kScoreTile < L && threadIdx.x == 0) {
      const int64_t unit = (int64_t)(l * cv.batch + b) * H + h;
      *(uint2 *)(range + 2 * ((unit * tiles + tile) * kRangeParts + part)) = make_uint2(0xffffffffu, 0u);
    }
    return;
  }
  const bool full = tile0 + SPAN <= L;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane % LPR, rsub = lane / LPR;
  const int rbase = tile0 + wave * ROWS_PER_WAVE + rsub;

  const char *kbase = (const char *)cv.k + (int64_t)l * cv.layer_stride * E;
  const char *ubase = kbase + ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h) * E;  // contiguous only
  const uint32_t rstride = (uint32_t)(cv.stride_s * E);                                     // contiguous only
  const int blk0 = PAGED ? tile0 / cv.block_size : 0;
  if constexpr (PAGED) {
    const int nblk = (min(tile0 + SPAN, L) - 1) / cv.block_size - blk0 + 1;
    for (int i = tid; i < nblk; i += blockDim.x)
      s_blk[i] = ((int64_t)cv.block_table[(int64_t)b * cv.max_blocks + blk0 + i] * cv.block_size * H + h) * (int64_t)(D * E);
    __syncthreads();
  }
  using Row = KRow;
  auto load_at = [&](int row) -> Row {
    Row r;
    const char *p;
    if constexpr (PAGED) {
      // power-of-two blocks (the usual case) split the slot with a shift and a mask
      const int bsh = cv.block_shift;
      const int bi = bsh >= 0 ? row >> bsh : row / cv.block_size;
      const int o = row - bi * cv.block_size;
      p = kbase + s_blk[bi - blk0] + (uint32_t)(o * H * (D * E) + seg * 16);
    } else {
      p = ubase + ((uint32_t)row * rstride + (uint32_t)(seg * 16));
    }
    if constexpr (TEMP) {
      r.a = *(const u32x4 *)p;
      r.b = *(const u32x4 *)(p + HB);
    } else {
      r.a = stream_load((const u32x4 *)p);
      r.b = stream_load((const u32x4 *)(p + HB));
    }
    return r;
  };
  auto load_row = [&](int row) -> Row {
    if (!full && row >= L) {
      Row r;
      r.a = r.b = u32x4{0u, 0u, 0u, 0u};
      return r;
    }
    return load_at(row);
  };

  // First batch of loads goes out before the prologue so its latency hides the float64 math.
  Row cur[UNR];
#pragma unroll
  for (int k = 0; k < UNR; ++k) cur[k] = load_row(rbase + k * RPW);

  using RS = RowScorer<DT, D, ROPE>;
  RS::centre(pv, (int64_t)l * H + h, pv.t[b], s_w, s_c, tid);
  __syncthreads();
  RS rs;
  rs.init(s_w, s_c, seg);
  auto row_score = [&](const Row &x) -> float { return rs(x); };

  float *out = scores + ((int64_t)(l * cv.batch + b) * H + h) * score_stride;
  // Running range of this workgroup's scores (NaN scores are ignored: they rank lowest anyway).
  float smin = __builtin_huge_valf(), smax = -__builtin_huge_valf();
  auto emit = [&](const Row (&rows)[UNR], int r0) {
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const float sc = row_score(rows[k]);
      const int row = r0 + k * RPW;
      if (full || row < L) {
        smin = fminf(smin, sc);
        smax = fmaxf(smax, sc);
        if (seg == 0) out[row] = sc;
      }
    }
  };
  if (full) {
    Row nxt[UNR];
    int it = 0;
#pragma unroll 1
    for (; it + 1 < ITERS; it += 2) {
      const int r0 = rbase + it * STEP;
#pragma unroll
      for (int k = 0; k < UNR; ++k) nxt[k] = load_at(r0 + STEP + k * RPW);
      emit(cur, r0);
      if (it + 2 < ITERS) {
#pragma unroll
        for (int k = 0; k < UNR; ++k) cur[k] = load_at(r0 + 2 * STEP + k * RPW);
      }
      emit(nxt, r0 + STEP);
    }
    if (it < ITERS) emit(cur, rbase + it * STEP);
  } else {
#pragma unroll 1
    for (int it = 0; it < ITERS; ++it) {
      const int r0 = rbase + it * STEP;
      if (r0 - rsub >= L) break;   // wave-uniform: the rest of this wave's rows are past the end
      emit(cur, r0);
      if (it + 1 < ITERS) {
#pragma unroll
        for (int k = 0; k < UNR; ++k) cur[k] = load_row(r0 + STEP + k * RPW);
      }
    }
  }
  if (range != nullptr) {
    // Publish the score range of the workgroup's rows, as order keys, in its slot [unit][tile][part]: a plain
    // store, no atomics.  Rows past the length add the neutral pair (key(+inf), key(-inf)).
    const uint32_t kmax = wave_max(order_key(smax)), kmin = wave_min(order_key(smin));
    if (lane == 0) {
      s_rng[wave][0] = kmin;
      s_rng[wave][1] = kmax;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        lo = min(lo, s_rng[w][0]);
        hi = max(hi, s_rng[w][1]);
      }
      const int64_t unit = (int64_t)(l * cv.batch + b) * H + h;
      *(uint2 *)(range + 2 * ((unit * tiles + tile) * kRangeParts + part)) = make_uint2(lo, hi);
    }
  }
}

// ------------------------------------------------------------------------------------ aggregation variants


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Lane l and lane l ^ 16 (resp. l ^ 32) combined, without the LDS: v_permlane16_swap / v_permlane32_swap with the
// value as both operands leave the value of one lane of the pair in each result, the partner's in the other.
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Variant scores on the matrix cores.  Range slots as k_score (per 1024-row tile and range part).  Per step of
// 16 keys a chain of v_mfma_f32_16x16x32_bf16 computes the logits of the 16 keys against the 64 or 128 columns of
// the unit (tiles of 16; column g*dpad + k = query head g, offset k, dpad = 16 or 32):
//   A = the rotated centres W = RoPE(centre, t), split into a bf16 high part and residual that accumulate into the
//       same float32 tile -- the fragments of the first 64 columns held in registers, those of the next 64 (XT) in
//       LDS in fragment order, read back each step;
//   B = the keys (lane holds key lane%16, dims (lane/16)*8 .. +8 of each 32-dim step).  Contiguous caches, and
//       paged pools whose block size is a multiple of 16, load the step's 16 rows whole (four rows per load
//       instruction) and pass them through a per-wave LDS block into that layout; other paged pools load the
//       16-byte fragments directly.
// Lane l then holds columns (l/16)*4 + i (i < 4) of every tile for key l%16; padding columns start at -inf, so
// maxima run over whole tiles, in-lane and then across the four lanes of the key.  The norm term comes from the
// same key fragments: rotary pairs meet inside one lane for both pairings.
// A workgroup is one part (kVarWaves waves, range slot `part`) of every cols-th tile of a unit, tiles j, j + cols,
// ...: building the centre fragments (float64 rotation, LDS transpose) is paid once for all of them, and each
// wave's loads run one step ahead across tile boundaries.  Paged rows find their block through the table one step
// before their load is issued.
constexpr int kVarWaves = 4;        // waves per variant workgroup
constexpr int kVarParts = kScoreWaves / kVarWaves;   // workgroups per tile
constexpr int kVarTiles = 8;        // tiles per variant workgroup (the host spreads a unit over ceil(tiles / this))
constexpr int kVarDepth = 2;        // 16-key steps in flight per wave (the ring of key fragments)
constexpr bool kVarCoal = true;     // whole-row loads, transposed to the matrix-core layout through LDS

template <int D, int ROPE, int PAGED, int AGG, int XT>
__global__ __launch_bounds__(64 * kVarWaves, XT ? 1 : 2) void k_score_var(CacheView cv, PassView pv,
                                                              float *__restrict__ scores, int64_t score_stride,
                                                              int tiles, int cols, uint32_t *__restrict__ range) {
  constexpr int KS = D / 32;                       // 32-dim steps of one MFMA
  constexpr int NT = 4;                            // column tiles with their centre fragments in registers
  constexpr int NTT = NT + (XT ? 4 : 0);           // all column tiles (XT: four more, fragments in LDS)
  constexpr int ROWS_PER_WAVE = kScoreTile / kScoreWaves;
  constexpr int STEPS = ROWS_PER_WAVE / 16;        // steps per tile
  constexpr bool HALF = ROPE == TRI_ROPE_HALF;
  constexpr int E = 2;                             // bf16 only
  constexpr int WP = D + 8;                        // padded LDS row: the 16 columns of a fragment read hit distinct banks
  // PAGED: 0 contiguous, 1 paged, 2 paged with block sizes a multiple of 16 (a step's 16 rows share a block)
  constexpr bool COAL = kVarCoal && PAGED != 1;
  constexpr int RB = D * E, CPR = RB / 16;         // bytes and 16-byte chunks per row
  // the first 64 columns' centres staged for the transpose into register fragments; once those are loaded the same
  // bytes hold the fragments of the next 64 columns (XT), in the order lanes read them: [tile][step][hi, lo][lane]
  constexpr int STAGE_BYTES = 2 * NT * 16 * WP * 2, XFRAG_BYTES = XT ? 4 * KS * 2 * 64 * 16 : 0;
  __shared__ __align__(16) unsigned char s_wbuf[STAGE_BYTES > XFRAG_BYTES ? STAGE_BYTES : XFRAG_BYTES];
  uint16_t (*const s_wh)[WP] = reinterpret_cast<uint16_t (*)[WP]>(s_wbuf);
  uint16_t (*const s_wl)[WP] = reinterpret_cast<uint16_t (*)[WP]>(s_wbuf + NT * 16 * WP * 2);
  u32x4 *const s_xf = reinterpret_cast<u32x4 *>(s_wbuf);
  __shared__ u32x4 s_kb[COAL ? kVarWaves * 16 * CPR : 1];   // per wave: one step's 16 rows, chunks swizzled
  __shared__ double s_cs[D / 2], s_sn[D / 2];
  __shared__ float s_c[D / 2];
  __shared__ uint32_t s_rng[kVarTiles][kVarWaves][2];   // per tile walked and wave: min and max order key
  static_assert(kVarParts == kRangeParts && kVarWaves == kRangeWaves, "a variant workgroup fills one range slot");

  if (checks_failed(pv)) return;
  const int H = cv.heads;
  int bid = blockIdx.x;
  const int h = bid % H;
  bid /= H;
  const int part = bid % kVarParts;
  bid /= kVarParts;
  const int j = bid % cols;
  bid /= cols;
  const int b = bid % cv.batch;
  const int l = bid / cv.batch;
  const int L = pv.lengths[b];
  const int ntile = (L + kScoreTile - 1) / kScoreTile;      // tiles holding keys
  if (j >= ntile) return;
  const int nk = (ntile - 1 - j) / cols + 1;                 // tiles of this workgroup: j + k*cols, k < nk
  const int nsteps = nk * STEPS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = part * kVarWaves + (tid >> 6);            // the wave's place in a tile (which rows it takes)
  const int64_t unit = (int64_t)(l * cv.batch + b) * H + h;
  const int m = lane & 15, r = lane >> 4;          // key within a step; 8-dim group within a 32-dim step
  const char *kbase = (const char *)cv.k + (int64_t)l * cv.layer_stride * E;
  const char *ubase = kbase + ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h) * E;
  const int32_t *btab = cv.block_table + (int64_t)b * cv.max_blocks;
  const int bsh = cv.block_shift;
  // first row of the wave's 16 keys in flat step g (tile j + (g/STEPS)*cols)
  auto step_row = [&](int g) { return (j + (g / STEPS) * cols) * kScoreTile + wave * ROWS_PER_WAVE + (g % STEPS) * 16; };
  auto block_of = [&](int row) { return bsh >= 0 ? row >> bsh : row / cv.block_size; };
  // The key a lane loads in step g: lanes past the end re-read the last key (their results are never stored), so
  // every step loads and computes unconditionally; a branch around either would make the compiler drain the
  // ring's loads in flight before the next ones issue.
  auto lane_row = [&](int g) { return min(step_row(g) + m, L - 1); };
  // Whole-row loads: load s covers bytes s*1024 .. +1024 of the step's 16 rows (in row order), lane l the 16
  // bytes at l*16: row n of the step, chunk position c.  It fetches the row's chunk c ^ (n % CPR), so that the
  // layout it lands in LDS (as loaded, position n*CPR + c) reads back conflict-free in the matrix-core layout.
  auto coal_row = [&](int g, int s) { return min(step_row(g) + (s * 1024 + lane * 16) / RB, L - 1); };
  // Paged: the physical block of the rows a lane loads in step g.  With PAGED == 2 every row a step loads (its
  // 16-aligned rows, or the last key when clamped) lies in the block of min(first row, L - 1).
  auto table = [&](int g) -> int32_t {
    const int gg = min(g, nsteps - 1);
    return btab[block_of(PAGED == 2 ? min(step_row(gg), L - 1) : lane_row(gg))];
  };
  auto paged_row = [&](int32_t blk, int row) -> const char * {
    return kbase + (((int64_t)blk * cv.block_size + (row - block_of(row) * cv.block_size)) * H + h) * (D * E);
  };
  auto load_step = [&](int g, int32_t blk, u32x4 (&a)[KS]) {
    if constexpr (COAL) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int o = s * 1024 + lane * 16, n = o / RB, c = (o % RB) / 16;
        const int row = coal_row(g, s);
        const char *p = PAGED ? paged_row(blk, row) : ubase + (int64_t)row * cv.stride_s * E;
        a[s] = stream_load((const u32x4 *)(p + (c ^ (n & (CPR - 1))) * 16));
      }
    } else {
      const int row = lane_row(g);
      const char *p = (PAGED ? paged_row(blk, row) : ubase + (int64_t)row * cv.stride_s * E) + r * 16;
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = stream_load((const u32x4 *)(p + s * 64));
    }
  };
  // Keys run NB - 1 steps ahead of the matrix cores (a ring of NB 16-key steps); paged block numbers one further.
  constexpr int NB = kVarDepth;
  u32x4 ring[NB][KS];
  int32_t blk_next = 0;
#pragma unroll
  for (int q = 0; q < NB - 1; ++q) load_step(min(q, nsteps - 1), PAGED ? table(q) : 0, ring[q]);
  if constexpr (PAGED) blk_next = table(NB - 1);

  // W = RoPE(centre, t) for the 64 columns, float64 angles, split into bf16 high part + residual in LDS.
  const int64_t ukv = (int64_t)l * H + h;
  if (tid < D / 2) {
    double sn, cs;
    sincos((double)pv.t[b] * pow(pv.theta, -2.0 * tid / D), &sn, &cs);
    s_cs[tid] = cs;
    s_sn[tid] = sn;
    s_c[tid] = pv.c_hat[ukv * (D / 2) + tid];
  }
  __syncthreads();
  for (int idx = tid; idx < NT * 16 * (D / 2); idx += blockDim.x) {
    const int col = idx / (D / 2), i = idx % (D / 2);
    const int pa = HALF ? i : 2 * i, pb = HALF ? i + D / 2 : 2 * i + 1;
    const float *v = pv.centres + (ukv * pv.columns + col) * D;
    const double va = v[pa], vb = v[pb];
    const float wa = (float)(va * s_cs[i] - vb * s_sn[i]), wb = (float)(va * s_sn[i] + vb * s_cs[i]);
    const uint32_t ha = bf16_bits(wa), hb = bf16_bits(wb);
    const uint16_t la = (uint16_t)bf16_bits(wa - __uint_as_float(ha << 16));
    const uint16_t lb = (uint16_t)bf16_bits(wb - __uint_as_float(hb << 16));
    s_wh[col][pa] = (uint16_t)ha;
    s_wh[col][pb] = (uint16_t)hb;
    s_wl[col][pa] = la;
    s_wl[col][pb] = lb;
  }
  __syncthreads();
  // centre fragments (the A operand): column T*16 + m, dims s*32 + r*8 .. +8, held in registers
  u32x4 bh[NT][KS], bl[NT][KS];
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bh[T][s] = *(const u32x4 *)&s_wh[T * 16 + m][s * 32 + r * 8];
      bl[T][s] = *(const u32x4 *)&s_wl[T * 16 + m][s * 32 + r * 8];
    }
  if constexpr (XT) {
    // columns 64 + T*16 + m: each lane builds its own fragments (dims s*32 + r*8 .. +8 with their rotary partners,
    // read from the centres in global memory) into the staging bytes, which every lane has finished reading
    __syncthreads();
#pragma unroll 1
    for (int T = 0; T < 4; ++T) {
      const float *v = pv.centres + (ukv * pv.columns + 64 + T * 16 + m) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float w2[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int dim = s * 32 + r * 8 + 2 * e + q;
            const int i = HALF ? (dim < D / 2 ? dim : dim - D / 2) : dim / 2;   // rotary pair of the dim
            const bool first = HALF ? dim < D / 2 : (dim & 1) == 0;
            const int pa = HALF ? i : 2 * i, pb = HALF ? i + D / 2 : 2 * i + 1;
            const double va = v[pa], vb = v[pb];
            w2[q] = first ? (float)(va * s_cs[i] - vb * s_sn[i]) : (float)(va * s_sn[i] + vb * s_cs[i]);
          }
          const uint32_t h0 = bf16_bits(w2[0]), h1 = bf16_bits(w2[1]);
          const uint32_t l0 = bf16_bits(w2[0] - __uint_as_float(h0 << 16)), l1 = bf16_bits(w2[1] - __uint_as_float(h1 << 16));
          hi[e] = h0 | (h1 << 16);
          lo[e] = l0 | (l1 << 16);
        }
        s_xf[((T * KS + s) * 2 + 0) * 64 + lane] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        s_xf[((T * KS + s) * 2 + 1) * 64 + lane] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
    __syncthreads();
  }
  // norm coefficients of the lane's pairs
  constexpr int NPAIR = 4 * KS;                    // 8 dims per step, 2 elements per pair
  float cr[NPAIR];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (HALF) {   // pairs (j, j + D/2): steps s < KS/2 hold the first elements
        if (s < KS / 2) {
          cr[s * 8 + e] = s_c[s * 32 + r * 8 + e];
          cr[s * 8 + 4 + e] = s_c[s * 32 + r * 8 + 4 + e];
        }
      } else {                // pairs (2i, 2i + 1) within the lane's 8 dims
        cr[s * 4 + e] = s_c[(s * 32 + r * 8) / 2 + e];
      }
    }
  const float inv_g = 1.0f / (float)pv.group;
  float *out = scores + unit * score_stride;
  float smin = __builtin_huge_valf(), smax = -__builtin_huge_valf();

  // Accumulator start values: 0 for real columns, -inf for padding (columns past the group or the offsets), so
  // every max below can run over all 16 columns of a tile.  Lane l's accumulator i of tile T is column
  // c = T*16 + (l/16)*4 + i, that of query head c / dpad and offset c % dpad.
  f32x4 acc0[NTT];
#pragma unroll
  for (int T = 0; T < NTT; ++T)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = T * 16 + r * 4 + i;
      acc0[T][i] = (c / pv.dpad < pv.group && c % pv.dpad < pv.n_offsets) ? 0.f : -__builtin_huge_valf();
    }
  const int tph = pv.dpad / 16;                    // column tiles per query head

  auto step = [&](int g, const u32x4 (&raw)[KS]) {
    u32x4 cur[KS];   // lane (m, r): key m, dims s*32 + r*8 .. +8
    if constexpr (COAL) {
      // Through this wave's LDS block: written as loaded, read back at key m's chunk (s*4 + r) ^ (m % CPR).
      // LDS operations of one wave complete in order, so the reads see these writes and the next step's writes
      // land after these reads.
      u32x4 *kb = s_kb + (tid >> 6) * (16 * CPR);
#pragma unroll
      for (int s = 0; s < KS; ++s) kb[s * 64 + lane] = raw[s];
#pragma unroll
      for (int s = 0; s < KS; ++s) cur[s] = kb[m * CPR + ((s * 4 + r) ^ (m & (CPR - 1)))];
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) cur[s] = raw[s];
    }
    const int row0 = step_row(g);
    {
      // logits: D[column][key] = W_column . K_key, centres as the A operand, keys as the B operand
      f32x4 acc[NTT];
#pragma unroll
      for (int T = 0; T < NTT; ++T) acc[T] = acc0[T];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, cur[s]);
#pragma unroll
        for (int T = 0; T < NT; ++T) {
          acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bh[T][s]), kf, acc[T], 0, 0, 0);
          acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bl[T][s]), kf, acc[T], 0, 0, 0);
        }
        if constexpr (XT) {
#pragma unroll
          for (int T = 0; T < 4; ++T) {
            const u32x4 xh = s_xf[((T * KS + s) * 2 + 0) * 64 + lane], xl = s_xf[((T * KS + s) * 2 + 1) * 64 + lane];
            acc[NT + T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xh), kf, acc[NT + T], 0, 0, 0);
            acc[NT + T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xl), kf, acc[NT + T], 0, 0, 0);
          }
        }
      }
      // norm term of key m from this lane's pairs (packed pairs, one dot2 per |z|^2)
      float nrm = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (HALF) {
            if (s < KS / 2) {
              const uint32_t p0 = pack_lo(cur[s][e], cur[s + KS / 2][e]), p1 = pack_hi(cur[s][e], cur[s + KS / 2][e]);
              nrm = fmaf(cr[s * 8 + 2 * e], __builtin_amdgcn_sqrtf(dot2(p0, p0, 0.f)), nrm);
              nrm = fmaf(cr[s * 8 + 2 * e + 1], __builtin_amdgcn_sqrtf(dot2(p1, p1, 0.f)), nrm);
            }
          } else {
            nrm = fmaf(cr[s * 4 + e], __builtin_amdgcn_sqrtf(dot2(cur[s][e], cur[s][e], 0.f)), nrm);
          }
        }
      // key m's columns are spread over the lanes m, m+16, m+32, m+48: reduce in-lane, then across those lanes
      float dist;
      if constexpr (AGG == TRI_AGG_MAX) {
        float x = acc[0][0];
#pragma unroll
        for (int T = 0; T < NTT; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaxf(x, acc[T][i]);
        dist = max_xor32(max_xor16(x));
      } else {
        // per query head the max over its tph tiles, then the mean over the group's heads
        float sum = 0.f, hm = -__builtin_huge_valf();
#pragma unroll
        for (int T = 0; T < NTT; ++T) {
          const float x = max_xor32(max_xor16(fmaxf(fmaxf(acc[T][0], acc[T][1]), fmaxf(acc[T][2], acc[T][3]))));
          hm = fmaxf(hm, x);
          if ((T + 1) % tph == 0) {
            sum += T / tph < pv.group ? hm : 0.f;   // tiles past the group hold only padding
            hm = -__builtin_huge_valf();
          }
        }
        dist = sum * inv_g;
      }
      nrm = add_xor32(add_xor16(nrm));
      const float sc = dist + nrm;
      // Every lane stores: the four lanes of a key hold the same score, and a lane past the end computed the last
      // key's score from the same data, so it writes that same value there.
      const bool valid = row0 + m < L;
      out[min(row0 + m, L - 1)] = sc;
      smin = fminf(smin, valid ? sc : __builtin_huge_valf());
      smax = fmaxf(smax, valid ? sc : -__builtin_huge_valf());
    }
  };
  static_assert(STEPS % NB == 0, "the ring phase repeats every tile");
#pragma unroll 1
  for (int k = 0; k < nk; ++k) {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int g = k * STEPS + st;
      // the tail re-loads the last step rather than branching around the load
      if constexpr (PAGED) {
        const int32_t blk = blk_next;
        blk_next = table(g + NB);
        load_step(min(g + NB - 1, nsteps - 1), blk, ring[(st + NB - 1) % NB]);
      } else {
        load_step(min(g + NB - 1, nsteps - 1), 0, ring[(st + NB - 1) % NB]);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the loads above this step's waits (else they sink below them)
      step(g, ring[st % NB]);
    }
    // The wave's score range of tile j + k*cols, as order keys, into LDS (every lane writes the same two words); a
    // wave without keys in the tile leaves the neutral pair (key(+inf), key(-inf)).
    if (range != nullptr) {
      const uint32_t kmax = wave_max(order_key(smax)), kmin = wave_min(order_key(smin));
      *(uint2 *)s_rng[k][tid >> 6] = make_uint2(kmin, kmax);
    }
    smin = __builtin_huge_valf();
    smax = -__builtin_huge_valf();
  }
  // Once all tiles are done: the range of this part of every tile it walked, into slot [unit][tile][part].
  if (range != nullptr) {
    __syncthreads();
    if (tid < nk) {
      uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
      for (int w = 0; w < kVarWaves; ++w) {
        lo = min(lo, s_rng[tid][w][0]);
        hi = max(hi, s_rng[tid][w][1]);
      }
      *(uint2 *)(range + 2 * ((unit * tiles + j + tid * cols) * kRangeParts + part)) = make_uint2(lo, hi);
    }
  }
}

// ------------------------------------------------------------------------------------ select

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at most 1024); `total`
// receives the sum.  Every thread of the workgroup must call it.  smem: 33 words.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *smem, uint32_t *total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) smem[w] = inc;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = lane < nw ? smem[lane] : 0u;
    const uint32_t ti = wave_incl_scan(t, lane);
    if (lane < nw) smem[lane] = ti - t;
    if (lane == nw - 1) smem[32] = ti;
  }
  __syncthreads();
  const uint32_t r = smem[w] + inc - v;
  *total = smem[32];
  __syncthreads();
  return r;
}

// Digit search shared by the radix passes: given histogram(s) of the current digit (nsub copies of nb
// bins), find the bin holding the krem-th largest remaining key.  Bins are scanned from the top; thread t
// owns bins nb-1-t*bpt ... ; exactly one thread finds the bin.  Returns (digit, new krem) via shared words.
__device__ void find_digit(const uint32_t *hist, int nb, int nsub, uint32_t krem, uint32_t *scan_smem,
                           uint32_t *s_digit, uint32_t *s_krem) {
  const int tid = threadIdx.x;
  const int bpt = nb / (int)blockDim.x;
  uint32_t loc = 0u;
  for (int k = 0; k < bpt; ++k)
    for (int q = 0; q < nsub; ++q) loc += hist[q * 2048 + nb - 1 - (tid * bpt + k)];
  uint32_t tot;
  uint32_t cum = block_excl_scan(loc, scan_smem, &tot);
  for (int k = 0; k < bpt; ++k) {
    const int bin = nb - 1 - (tid * bpt + k);
    uint32_t hc = 0u;
    for (int q = 0; q < nsub; ++q) hc += hist[q * 2048 + bin];
    if (cum < krem && krem <= cum + hc) {
      *s_digit = (uint32_t)bin;
      *s_krem = krem - cum;
    }
    cum += hc;
  }
  __syncthreads();
}

// Bin of a score in the first selection pass: fma(v, scale, -vmin*scale) clamped to [0, 2047] and truncated.
// Each step is monotone non-decreasing in v (a fused multiply-add with scale >= 0 rounds monotonically, max/min
// and truncation preserve order, and NaN -- from a NaN score or 0*inf -- becomes 0 through max), so a score in
// a higher bin is strictly larger than every score in a lower bin whatever vmin and scale are.  The range
// only decides how evenly the scores spread over the bins, never the result.
__device__ __forceinline__ uint32_t value_bin(float v, float scale, float offset) {
  const float t = fminf(fmaxf(fmaf(v, scale, offset), 0.f), 2047.f);
  return (uint32_t)t;
}

constexpr uint32_t kNoBin = 0xffffu;  // marks slots that are not candidates
constexpr int kSelectList = 4096;     // members of the threshold bin gathered into LDS
constexpr int kRankMax = 2048;        // up to this many members are ranked directly

// ------------------------------------------------------------------------------------ compact

__global__ void k_reset(uint32_t *flags, int64_t n, uint32_t *counter, int64_t units) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) flags[i] = 0u;
  if (i < units) counter[i] = 0u;
}

constexpr int kCompactThreads = 512;   // threads of a compaction workgroup
constexpr int kSelectInflight = 64;    // scores per thread loaded before the first histogram update

// Row moves are non-temporal both ways: a moved row is not read again by the pass.
template <typename T>
__device__ __forceinline__ T move_load(const T *p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void move_store(T *p, T v) {
  __builtin_nontemporal_store(v, p);
}

// New block table row and freed blocks of sequence b (paged caches; called by one workgroup per b).
__device__ void write_tables(const CacheView &cv, const PassView &pv, int b, int32_t *table_out, int32_t *freed,
                             int32_t *n_freed, uint32_t *smem) {
  const int bs = cv.block_size, B = pv.budget;
  const int L = pv.lengths[b];
  const int nb_old = (L + bs - 1) / bs, nb_new = (min(L, B) + bs - 1) / bs;
  const int out_stride = (B + bs - 1) / bs;
  const int32_t *row = cv.block_table + (int64_t)b * cv.max_blocks;
  for (int i = threadIdx.x; i < nb_new; i += blockDim.x) table_out[(int64_t)b * out_stride + i] = row[i];
  uint32_t part = 0u;
  for (int bb = threadIdx.x; bb < b; bb += blockDim.x) {
    const int Lb = pv.lengths[bb];
    part += (uint32_t)((Lb + bs - 1) / bs - (min(Lb, B) + bs - 1) / bs);
  }
  uint32_t prefix;
  block_excl_scan(part, smem, &prefix);
  for (int i = nb_new + threadIdx.x; i < nb_old; i += blockDim.x) freed[prefix + (i - nb_new)] = row[i];
  if (b == cv.batch - 1 && threadIdx.x == 0) *n_freed = (int32_t)(prefix + (nb_old - nb_new));
}

// Moves of one unit in place ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 step 5: later attention reads
// the compressed cache), by the workgroup that selected them: row j of K and V and pos[j] become those of slot
// s_keep[j] for j < Ln, in ascending chunks of kMovePasses * (THREADS / lanes per row) destinations.  keep is
// ascending with keep[j] >= j, so the sources of a chunk lie past every destination of the chunks before it: the
// only hazard is inside a chunk, and every load of a chunk completes before the barrier that precedes its stores.
// The next chunk's loads are issued before the current chunk's stores (two register buffers).  Every load and
// store is unconditional: a destination that keeps its own row, and a lane past the end of the keep list (it takes
// a row r >= Ln, never a destination, of which it is then the only writer), copy a row onto itself -- a write of
// the value it holds -- so the compiler can count exactly which loads are still in flight.  Paged caches read the
// unit's block-table row from LDS (s_tab, staged by the caller).
// 16-byte loads of K (and as many of V) per lane per chunk and buffer: with two buffers 16 loads per lane in flight
// (≈116 VGPRs, two 512-thread workgroups per compute unit), which measured faster than 2 per buffer at three
// workgroups per compute unit (a third more bytes in flight per CU, half the chunk barriers).
constexpr int kMovePasses = 4;
// The selecting-and-moving kernel keeps four histogram copies like the selecting-only one (at two workgroups per
// compute unit the LDS has room: ≈70 KB each); its histograms hold the keep list afterwards, up to 8192 slots.
constexpr int kHistCopiesMove = 4;
constexpr int kMoveKeepMax = kHistCopiesMove * 2048;  // longest keep list it holds in LDS to move rows itself
constexpr int kMoveTableMax = 2 * 4096; // most block-table entries per sequence it stages in LDS (paged)

template <int THREADS, int PAGED, int POW2>
__device__ void move_unit(const CacheView &cv, int l, int b, int h, const int32_t *s_keep, int Ln, int L,
                          const int32_t *s_tab) {
  const int tid = threadIdx.x;
  const int64_t esz = cv.dtype == TRI_BF16 ? 2 : 4;
  const int rb = cv.head_dim * (int)esz;                  // 128, 256 or 512 bytes per row
  const int lsh = rb == 128 ? 3 : (rb == 256 ? 4 : 5);    // log2 of the lanes per row
  const int seg = tid & ((1 << lsh) - 1), rr = tid >> lsh;
  const int rpp = THREADS >> lsh;                         // rows per pass
  const int chunk = kMovePasses * rpp;
  const int H = cv.heads;
  const int64_t lb = (int64_t)l * cv.layer_stride * esz;
  const char *kbase = (const char *)cv.k + lb + seg * 16;
  const char *vbase = (const char *)cv.v + lb + seg * 16;
  int32_t *pbase = cv.pos + (int64_t)l * cv.pos_layer_stride;
  const int bs = cv.block_size, bsh = cv.block_shift;
  // byte offset of slot sl's row from the layer's base (paged: through the staged table), and its position index
  auto row_of = [&](int sl) -> int64_t {
    if constexpr (PAGED) {
      const int bi = POW2 ? sl >> bsh : sl / bs;
      return (int64_t)s_tab[bi] * bs + (sl - bi * bs);
    } else {
      return sl;
    }
  };
  auto row_off = [&](int64_t r) -> int64_t {
    if constexpr (PAGED) return (r * H + h) * (int64_t)rb;
    else return ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h + r * cv.stride_s) * esz;
  };
  auto pos_off = [&](int64_t r) -> int64_t {
    if constexpr (PAGED) return r * H + h;
    else return (int64_t)b * cv.pos_stride_b + (int64_t)h * cv.pos_stride_h + r;
  };
  // destination and source slot of lane slot j: past the keep list a lane copies a row r >= Ln onto itself (r < L)
  auto dst_of = [&](int j) -> int { return j < Ln ? j : min(j, L - 1); };
  auto src_of = [&](int j) -> int { return j < Ln ? s_keep[j] : min(j, L - 1); };

  struct Buf {
    u32x4 k[kMovePasses], v[kMovePasses];
    int32_t p[kMovePasses];
  };
  auto issue = [&](int j0, Buf &x) {
#pragma unroll
    for (int q = 0; q < kMovePasses; ++q) {
      const int64_t r = row_of(src_of(j0 + q * rpp + rr));
      const int64_t o = row_off(r);
      x.k[q] = move_load((const u32x4 *)(kbase + o));
      x.v[q] = move_load((const u32x4 *)(vbase + o));
      x.p[q] = pbase[pos_off(r)];   // every lane of the row reads (and later writes) the same position id
    }
  };
  auto settle = [&](const Buf &x) {   // this lane's loads of x have returned; then every lane's have
#pragma unroll
    for (int q = 0; q < kMovePasses; ++q) asm volatile("" ::"v"(x.k[q]), "v"(x.v[q]), "v"(x.p[q]));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto drain = [&](int j0, const Buf &x) {
#pragma unroll
    for (int q = 0; q < kMovePasses; ++q) {
      const int64_t r = row_of(dst_of(j0 + q * rpp + rr));
      const int64_t o = row_off(r);
      move_store((u32x4 *)(kbase + o), x.k[q]);
      move_store((u32x4 *)(vbase + o), x.v[q]);
      pbase[pos_off(r)] = x.p[q];
    }
  };
  // Chunk 0 is peeled so that, wherever a buffer's loads are awaited, exactly one chunk's stores were issued after
  // them on every path that reaches the wait (the compiler then waits for those loads only, not the stores).
  const int nch = (Ln + chunk - 1) / chunk;
  Buf a, c;
  issue(0, a);
  settle(a);
  if (nch > 1) issue(chunk, c);   // sources of chunk 1 lie past every destination of chunk 0
  drain(0, a);
#pragma unroll 1
  for (int ch = 1; ch < nch; ch += 2) {
    settle(c);
    if (ch + 1 < nch) issue((ch + 1) * chunk, a);
    drain(ch * chunk, c);
    if (ch + 1 >= nch) break;
    settle(a);
    if (ch + 2 < nch) issue((ch + 2) * chunk, c);
    drain((ch + 1) * chunk, a);
  }
}

// One workgroup per unit (grid = units; with MOVE on a paged cache, xcd_grouped_grid): 512 threads for up to 32K
// slots, 1024 threads beyond.  Thread t owns slots [t*EPT, (t+1)*EPT), so slot order is (thread, element) order
// and the emitted keep list is ascending.
// Finding the K-th largest key among candidate slots [0, n):
//   1. the range [vmin, vmax] of the unit's scores -- reduced from the per-tile ranges the scoring kernel
//      published when `range` is given, else from a first read of the scores -- defines 2048 equal-width
//      value bins; each thread keeps only the bin of each of its slots (two per register) and histograms them
//      into four LDS copies (one per group of waves, to spread atomic contention);
//   2. a suffix scan finds the bin b* holding the K-th largest; the exact keys of its members are gathered
//      into an LDS list (re-read from the cache-resident scores);
//   3. an exact rank of the members (few, the usual case) or an exact radix select (11/11/10-bit digits) over
//      them gives the threshold key tau and the number krem of its ties to keep; ties are kept from the lowest
//      slot up.
// MOVE: the same workgroup then compacts the unit (move_unit) from a copy of the keep list in LDS, so one unit's
// selection latency overlaps other units' row moves; paged caches also get their new tables and freed list.
template <int THREADS, int EPT, int MOVE>
__global__ __launch_bounds__(THREADS, 4) void k_select(CacheView cv, PassView pv, const float *__restrict__ scores,
                                                       int64_t score_stride, int32_t *__restrict__ keep,
                                                       int32_t *__restrict__ new_lengths, uint32_t *flags,
                                                       uint32_t *counter, int chunks_per_unit, const uint32_t *range,
                                                       int tiles, int32_t *table_out, int32_t *freed,
                                                       int32_t *n_freed) {
  static_assert(EPT % 4 == 0, "float4 loads");
  constexpr int HC = MOVE ? kHistCopiesMove : 4;   // histogram copies (atomic contention spread over wave groups)
  constexpr int INFL = MOVE ? kSelectInflight / 2 : kSelectInflight;   // scores per thread loaded at once
  __shared__ uint32_t hist[HC * 2048];
  __shared__ uint32_t lists[2 * kSelectList];
  uint32_t *const list = lists;                  // member keys
  uint32_t *const lslot = lists + kSelectList;   // member slots
  __shared__ unsigned long long kbits[THREADS];   // per thread: which of its slots in bin b* are kept
  __shared__ uint32_t scan_smem[33];
  __shared__ uint32_t s_red[2][THREADS / 64];
  __shared__ uint32_t s_digit, s_krem, s_nlist;
  static_assert(EPT <= 64, "one 64-bit member mask per thread");
  // MOVE: the keep list, written where the histograms were once the threshold is known
  int32_t *const s_keep = reinterpret_cast<int32_t *>(hist);
  static_assert(sizeof(hist) >= kMoveKeepMax * sizeof(int32_t), "keep list in LDS");
  // MOVE, paged: the sequence's block-table row, where the member lists were
  int32_t *const s_tab = reinterpret_cast<int32_t *>(lists);
  static_assert(sizeof(lists) >= kMoveTableMax * sizeof(int32_t), "table row in LDS");

  if (checks_failed(pv)) return;
  const int H = cv.heads;
  const int unit = MOVE && cv.paged ? xcd_grouped_unit(blockIdx.x, H, cv.layers * cv.batch) : (int)blockIdx.x;
  if (unit < 0) return;
  const int h = unit % H;
  const int b = (unit / H) % cv.batch;
  const int l = unit / (H * cv.batch);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = pv.lengths[b], B = pv.budget, R = pv.recent;
  const int n = L - R, K = B - R;

  if (flags != nullptr) {  // compaction control words of this unit start at zero
    for (int c = tid; c < chunks_per_unit; c += blockDim.x) flags[(int64_t)unit * chunks_per_unit + c] = 0u;
    if (tid == 0) counter[unit] = 0u;
  }
  if (l == 0 && h == 0 && tid == 0) new_lengths[b] = min(L, B);
  if constexpr (MOVE) {
    if (cv.paged && l == 0 && h == 0) write_tables(cv, pv, b, table_out, freed, n_freed, scan_smem);
  }
  int32_t *out = keep + (int64_t)unit * B;
  // emit one kept slot at place j of the keep list
  auto emit = [&](uint32_t j, int slot) {
    out[j] = slot;
    if constexpr (MOVE) s_keep[j] = slot;
  };

  auto select = [&]() {
    uint32_t kmax = 0u, kmin = 0xffffffffu;
    if (range != nullptr) {  // ranges published by the scoring kernel for this unit's tiles
      const int nparts = min((L + kScoreTile - 1) / kScoreTile, tiles) * kRangeParts;
      const uint32_t *part = range + 2 * (int64_t)unit * tiles * kRangeParts;
      for (int i = tid; i < nparts; i += blockDim.x) {
        kmin = min(kmin, part[2 * i]);
        kmax = max(kmax, part[2 * i + 1]);
      }
    }
    if (L <= B) {
      for (int j = tid; j < L; j += blockDim.x) out[j] = j;
      return;
    }
    for (int j = tid; j < R; j += blockDim.x) out[K + j] = n + j;   // (MOVE: into LDS after the selection)
    if (K == 0) return;

    const float *sc = scores + (int64_t)unit * score_stride;
    const int base = tid * EPT;
    const int nv = min(max(n - base, 0), EPT);   // candidate slots of this thread (all of them but in one thread)
    auto key_at = [&](int e) -> uint32_t { return order_key(sc[base + e]); };

    for (int i = tid; i < HC * 2048; i += blockDim.x) hist[i] = 0u;
    if (tid == 0) s_nlist = 0u;
    if (range == nullptr) {  // 1a. range from a first read of the scores
      if (nv == EPT) {
#pragma unroll
        for (int q = 0; q < EPT; q += 4) {
          const float4 f = *(const float4 *)(sc + base + q);
          const uint32_t k0 = order_key(f.x), k1 = order_key(f.y), k2 = order_key(f.z), k3 = order_key(f.w);
          kmin = min(kmin, min(min(k0, k1), min(k2, k3)));
          kmax = max(kmax, max(max(k0, k1), max(k2, k3)));
        }
      } else {
        for (int e = 0; e < nv; ++e) {
          const uint32_t k = key_at(e);
          kmin = min(kmin, k);
          kmax = max(kmax, k);
        }
      }
    }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) {
      s_red[0][wv] = kmin;
      s_red[1][wv] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
      kmin = min(kmin, s_red[0][w]);
      kmax = max(kmax, s_red[1][w]);
    }
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    float scale = vmax > vmin ? 2048.f / (vmax - vmin) : 0.f;
    if (!(scale < 3.0e38f)) scale = 0.f;                         // infinite or NaN spans
    const float offset = (scale > 0.f && vmin > -3.0e38f) ? -vmin * scale : 0.f;

    // 1b. bins and their histogram.  Every thread but (at most) one owns only candidates and takes the first
    //     branch, which has no per-slot validity logic; whole waves skip the other branch.
    uint32_t bins[EPT / 2];
    {
      const uint32_t hsub = (wv % HC) * 2048;
      if (nv == EPT) {
        // scores per load group: all of them, or a divisor of EPT no larger than INFL (a multiple of 4)
        constexpr int G = EPT <= INFL ? EPT : (EPT % INFL == 0 ? INFL : 16);
        static_assert(EPT % G == 0 && G % 4 == 0, "load groups tile the thread's slots");
#pragma unroll
        for (int g = 0; g < EPT; g += G) {
          float4 f[G / 4];
#pragma unroll
          for (int q = 0; q < G / 4; ++q) f[q] = *(const float4 *)(sc + base + g + 4 * q);   // all in flight
#pragma unroll
          for (int q = 0; q < G / 4; ++q) {
            const uint32_t b0 = value_bin(f[q].x, scale, offset), b1 = value_bin(f[q].y, scale, offset);
            const uint32_t b2 = value_bin(f[q].z, scale, offset), b3 = value_bin(f[q].w, scale, offset);
            atomicAdd(&hist[hsub + b0], 1u);
            atomicAdd(&hist[hsub + b1], 1u);
            atomicAdd(&hist[hsub + b2], 1u);
            atomicAdd(&hist[hsub + b3], 1u);
            bins[(g + 4 * q) / 2] = b0 | (b1 << 16);
            bins[(g + 4 * q) / 2 + 1] = b2 | (b3 << 16);
          }
        }
      } else {
#pragma unroll 1
        for (int q = 0; q < EPT / 2; ++q) bins[q] = kNoBin | (kNoBin << 16);
        for (int e = 0; e < nv; ++e) {
          const uint32_t bn = value_bin(sc[base + e], scale, offset);
          atomicAdd(&hist[hsub + bn], 1u);
#pragma unroll
          for (int q = 0; q < EPT / 2; ++q)   // constant register indices; the loop above is short
            if (q == e / 2) bins[q] = (e & 1) ? ((bins[q] & 0xffffu) | (bn << 16)) : ((bins[q] & 0xffff0000u) | bn);
        }
      }
    }
    auto bin_of = [&](int e) -> uint32_t { return (bins[e >> 1] >> ((e & 1) * 16)) & 0xffffu; };
    __syncthreads();

    // 2. the bin of the K-th largest, and its members as (key, slot) pairs
    find_digit(hist, 2048, HC, (uint32_t)K, scan_smem, &s_digit, &s_krem);
    const uint32_t bstar = s_digit;
    uint32_t krem = s_krem;
    kbits[tid] = 0ull;
    // members as a bit mask built without branches, then a rolled walk over its set bits
    unsigned long long mm = 0ull;
#pragma unroll
    for (int e = 0; e < EPT; ++e) mm |= (unsigned long long)(bin_of(e) == bstar) << e;
    while (mm) {
      const int e = __builtin_ctzll(mm);
      mm &= mm - 1ull;
      const uint32_t i = atomicAdd(&s_nlist, 1u);
      if (i < (uint32_t)kSelectList) lslot[i] = (uint32_t)(base + e);
    }
    __syncthreads();
    const uint32_t nlist = s_nlist;
    for (uint32_t i = tid; i < min(nlist, (uint32_t)kSelectList); i += blockDim.x) list[i] = order_key(sc[lslot[i]]);
    __syncthreads();

    if (nlist <= (uint32_t)kRankMax) {
      // 3. exact rank of every member under (key descending, slot ascending); ranks are unique, so the
      //    members ranked below krem are exactly the kept ones (ties go to the lowest slots).
      for (uint32_t i = tid; i < nlist; i += blockDim.x) {
        const uint32_t ki = list[i], si = lslot[i];
        uint32_t rank = 0u;
        for (uint32_t j = 0; j < nlist; ++j) {
          const uint32_t kj = list[j];
          rank += (kj > ki || (kj == ki && lslot[j] < si)) ? 1u : 0u;
        }
        if (rank < krem) atomicOr(&kbits[si / EPT], 1ull << (si % EPT));
      }
      __syncthreads();
      // emission: slots in bins above b* are kept, members of b* as decided
      const unsigned long long mine = kbits[tid];
      unsigned long long km = 0ull;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t bn = bin_of(e);
        const bool kept = (bn != kNoBin) & ((bn > bstar) | ((bn == bstar) & (uint32_t)((mine >> e) & 1ull)));
        km |= (unsigned long long)kept << e;
      }
      uint32_t tot;
      uint32_t dst = block_excl_scan((uint32_t)__popcll(km), scan_smem, &tot);
      while (km) {
        const int e = __builtin_ctzll(km);
        km &= km - 1ull;
        emit(dst++, base + e);
      }
      return;
    }

    // 3'. many members (heavily tied or clustered scores): exact radix select (11/11/10-bit digits) among
    //     them, then ties by a block scan.  This path re-derives membership from the scores with rolled loops
    //     so that it holds no per-slot state in registers.
    const bool in_list = nlist <= (uint32_t)kSelectList;
    auto member_key = [&](int e, uint32_t *k) -> bool {
      if (e >= nv) return false;
      const float f = sc[base + e];
      if (value_bin(f, scale, offset) != bstar) return false;
      *k = order_key(f);
      return true;
    };
    uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < nb; i += blockDim.x) hist[i] = 0u;
      __syncthreads();
      if (in_list) {
        for (uint32_t i = tid; i < nlist; i += blockDim.x) {
          const uint32_t k = list[i];
          if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      } else {
#pragma unroll 1
        for (int e = 0; e < EPT; ++e) {
          uint32_t k;
          if (member_key(e, &k) && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      find_digit(hist, nb, 1, krem, scan_smem, &s_digit, &s_krem);
      prefix |= s_digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      krem = s_krem;
    }
    const uint32_t tau = prefix;  // the K-th largest key; krem of its ties are kept, lowest slots first

    uint32_t nties = 0u;
#pragma unroll 1
    for (int e = 0; e < EPT; ++e) {
      uint32_t k;
      if (member_key(e, &k) && k == tau) ++nties;
    }
    uint32_t tot;
    const uint32_t tie0 = block_excl_scan(nties, scan_smem, &tot);
    auto kept_at = [&](int e, uint32_t &tr) -> bool {
      if (e >= nv) return false;
      const float f = sc[base + e];
      const uint32_t bn = value_bin(f, scale, offset);
      if (bn != bstar) return bn > bstar;
      const uint32_t k = order_key(f);
      const bool kept = k > tau || (k == tau && tr < krem);
      tr += k == tau ? 1u : 0u;
      return kept;
    };
    uint32_t nkeep = 0u, tr = tie0;
#pragma unroll 1
    for (int e = 0; e < EPT; ++e) nkeep += kept_at(e, tr) ? 1u : 0u;
    uint32_t dst = block_excl_scan(nkeep, scan_smem, &tot);
    tr = tie0;
#pragma unroll 1
    for (int e = 0; e < EPT; ++e)
      if (kept_at(e, tr)) emit(dst++, base + e);
  };

  select();
  if constexpr (MOVE) {
    if (L <= B) return;   // nothing evicted, nothing moves
    // the recent window's part of the keep list (the histograms it overwrites are no longer read), and for a paged
    // cache the sequence's block-table row (the member lists it overwrites are no longer read either)
    __syncthreads();
    for (int j = tid; j < R; j += THREADS) s_keep[K + j] = n + j;
    if (cv.paged) {
      const int32_t *trow = cv.block_table + (int64_t)b * cv.max_blocks;
      for (int i = tid; i < (L + cv.block_size - 1) / cv.block_size; i += THREADS) s_tab[i] = trow[i];
    }
    __syncthreads();
    if (!cv.paged) move_unit<THREADS, 0, 0>(cv, l, b, h, s_keep, B, L, nullptr);
    else if (cv.block_shift >= 0) move_unit<THREADS, 1, 1>(cv, l, b, h, s_keep, B, L, s_tab);
    else move_unit<THREADS, 1, 0>(cv, l, b, h, s_keep, B, L, s_tab);
  }
}

template <int RB, int PAGED>
__global__ __launch_bounds__(kCompactThreads) void k_compact(CacheView cv, PassView pv, const int32_t *__restrict__ keep,
                                                              int32_t *table_out, int32_t *freed, int32_t *n_freed,
                                                              uint32_t *flags, uint32_t *counter, int cpu) {
  constexpr int LPR = RB / 16;
  constexpr int RPP = kCompactThreads / LPR;      // rows per pass
  constexpr int NP = kCompactChunk / RPP;         // passes per chunk
  static_assert(NP * RPP == kCompactChunk, "chunk shape");
  __shared__ int s_ticket;
  __shared__ uint32_t smem[33];

  // Workgroups blockIdx.x / cpu belong to one unit; each takes its chunk index from that unit's ticket
  // counter, so a chunk only ever waits for chunks of its unit that are already running.
  if (checks_failed(pv)) return;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / cpu;
  if (tid == 0) s_ticket = (int)atomicAdd(&counter[unit], 1u);
  __syncthreads();
  const int c = s_ticket;
  const int H = cv.heads;
  const int h = unit % H;
  const int b = (unit / H) % cv.batch;
  const int l = unit / (H * cv.batch);
  const int L = pv.lengths[b], B = pv.budget;
  const int Ln = min(L, B);

  if constexpr (PAGED) {
    if (l == 0 && h == 0 && c == 0) write_tables(cv, pv, b, table_out, freed, n_freed, smem);
  }
  if (L <= B) return;
  const int j0 = c * kCompactChunk;
  if (j0 >= Ln) return;
  const int j1 = min(j0 + kCompactChunk, Ln);
  const int32_t *kp = keep + (int64_t)unit * B;
  const int seg = tid % LPR, rr = tid / LPR;

  const int64_t esz = RB / cv.head_dim;   // element size
  char *kb = (char *)cv.k + (int64_t)l * cv.layer_stride * esz;
  char *vb = (char *)cv.v + (int64_t)l * cv.layer_stride * esz;
  int32_t *pb = cv.pos + (int64_t)l * cv.pos_layer_stride;
  const int32_t *trow = PAGED ? cv.block_table + (int64_t)b * cv.max_blocks : nullptr;
  // Physical row of logical slot s: paged -> pool row (block*block_size + offset), contiguous -> s.
  auto row_off = [&](int64_t r) -> int64_t {
    if constexpr (PAGED) return (r * H + h) * (int64_t)RB;
    else return ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h + r * cv.stride_s) * esz;
  };
  auto pos_off = [&](int64_t r) -> int64_t {
    if constexpr (PAGED) return r * H + h;
    else return (int64_t)b * cv.pos_stride_b + (int64_t)h * cv.pos_stride_h + r;
  };
  const int bsh = cv.block_shift;
  auto blk_index = [&](int sl) -> int { return bsh >= 0 ? sl >> bsh : sl / cv.block_size; };
  auto phys = [&](int sl, int blk) -> int64_t {
    if constexpr (PAGED) return (int64_t)blk * cv.block_size + (sl - blk_index(sl) * cv.block_size);
    else return sl;
  };

  // Loads in three dependent phases, each fully parallel: keep indices, block-table entries, rows.
  u32x4 kr[NP], vr[NP];
  int src[NP], sblk[NP];
  int32_t pr[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    src[p] = j < j1 ? kp[j] : j;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    sblk[p] = 0;
    if constexpr (PAGED) {
      if (j < j1 && src[p] != j) sblk[p] = trow[blk_index(src[p])];
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    kr[p] = vr[p] = u32x4{0u, 0u, 0u, 0u};
    pr[p] = 0;
    if (j < j1 && src[p] != j) {
      const int64_t r = phys(src[p], sblk[p]);
      const int64_t o = row_off(r);
      kr[p] = move_load((const u32x4 *)(kb + o) + seg);
      vr[p] = move_load((const u32x4 *)(vb + o) + seg);
      if (seg == 0) pr[p] = pb[pos_off(r)];
    }
  }
  // Publish "my sources are loaded", then wait for earlier chunks whose sources overlap my destinations.
  // Only the completion of this workgroup's loads has to precede the flag: the empty asm consumes every
  // loaded register (the compiler waits for the loads before it), and the flag is a relaxed agent-scope
  // atomic, so no cache write-back or invalidation is needed on either side.  A waiter's stores are
  // control-dependent on the flag value it read, and GPU stores are not speculated.
#pragma unroll
  for (int p = 0; p < NP; ++p) asm volatile("" ::"v"(kr[p]), "v"(vr[p]), "v"(pr[p]));
  __syncthreads();
  if (tid == 0) {
    uint32_t *fl = flags + (int64_t)unit * cpu;
    __hip_atomic_store(&fl[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int cc = c - 1; cc >= 0; --cc) {
      if (kp[(cc + 1) * kCompactChunk - 1] < j0) break;  // keep is ascending: earlier chunks reach even less far
      while (__hip_atomic_load(&fl[cc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  int dblk[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    dblk[p] = 0;
    if constexpr (PAGED) {
      if (j < j1 && src[p] != j) dblk[p] = trow[blk_index(j)];
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    if (j < j1 && src[p] != j) {
      const int64_t r = phys(j, dblk[p]);
      const int64_t o = row_off(r);
      move_store((u32x4 *)(kb + o) + seg, kr[p]);
      move_store((u32x4 *)(vb + o) + seg, vr[p]);
      if (seg == 0) pb[pos_off(r)] = pr[p];
    }
  }
}

// ------------------------------------------------------------------------------------ fused short-cache pass

constexpr int kFusedUnroll = 4;        // rows in flight per lane in the fused pass's score phase
constexpr int kFusedMovePasses = 8;    // 16-byte loads of K (and of V) per lane in flight per move chunk

template <typename T>
__device__ __forceinline__ T fused_load(const T *p) {
  return *p;   // through the caches: the moves that follow re-read the kept K rows
}

// One workgroup per unit (paged caches: the XCD-grouped grid, xcd_grouped_unit), for caches of at most kFusedMax
// slots (the recurring pass at budget plus a few decode steps).  The unit's rows are scored into LDS as order
// keys; an exact radix select over those keys (11/11/10-bit digits) gives the threshold key and how many of its
// ties to keep from the lowest slot; the ascending keep list is built in LDS; then the same workgroup moves the
// retained rows in place, in ascending chunks.  Destination j <= source keep[j], and sources of later chunks lie beyond every earlier
// destination, so the only hazard is inside a chunk: all of its loads complete before the barrier that
// precedes its stores.  Scores and the keep list go to global memory only when the caller asks for them.
template <int DT, int D, int ROPE, int PAGED>
__global__ __launch_bounds__(kFusedThreads, 2) void k_fused(CacheView cv, PassView pv, float *__restrict__ scores,
                                                            int64_t score_stride, int32_t *__restrict__ keep_out,
                                                            int32_t *new_lengths, int32_t *table_out, int32_t *freed,
                                                            int32_t *n_freed) {
  using RS = RowScorer<DT, D, ROPE>;
  constexpr int E = RS::E, HB = RS::HB, LPR = RS::LPR;
  constexpr int RB = D * E;                            // bytes per row
  constexpr int RPW = 64 / LPR;                        // rows per wave per load
  constexpr int UNR = kFusedUnroll;
  constexpr int WAVES = kFusedThreads / 64;
  constexpr int STEP = WAVES * RPW * UNR;              // rows per workgroup step of the score phase
  constexpr int EPT = kFusedMax / kFusedThreads;       // slots per thread in the selection
  constexpr int MLPR = RB / 16;                        // lanes per row in the move phase
  constexpr int MRPP = kFusedThreads / MLPR;           // rows per move pass
  constexpr int CHUNK = MRPP * kFusedMovePasses;       // rows per move chunk
  static_assert(EPT >= 1 && EPT <= 32 && EPT * kFusedThreads == kFusedMax, "selection shape");

  __shared__ float s_w[D];
  __shared__ float s_c[D / 2];
  __shared__ uint32_t s_key[kFusedMax];                // order key of every slot's score, then the keep list
  int32_t *const s_keep = reinterpret_cast<int32_t *>(s_key);   // kept slots, ascending (written once the
                                                                 // keep bits are taken from the keys)
  __shared__ uint32_t s_hist[2048];
  __shared__ int64_t s_blk[PAGED ? kFusedBlocks : 1];  // paged: byte offset of this head's row 0 in each block
  __shared__ uint32_t s_scan[33];
  __shared__ uint32_t s_digit, s_krem;

  if (checks_failed(pv)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = cv.heads;
  const int unit = PAGED ? xcd_grouped_unit(blockIdx.x, H, cv.layers * cv.batch) : (int)blockIdx.x;
  if (unit < 0) return;
  const int h = unit % H, b = (unit / H) % cv.batch, l = unit / (H * cv.batch);
  const int L = min(pv.lengths[b], cv.capacity);       // capacity <= kFusedMax bounds every LDS index
  const int B = pv.budget, R = pv.recent;
  const int Ln = min(L, B);
  const bool evict = L > B;

  if (l == 0 && h == 0) {
    if (tid == 0) new_lengths[b] = min(pv.lengths[b], B);
    if constexpr (PAGED) write_tables(cv, pv, b, table_out, freed, n_freed, s_scan);
  }
  if (!evict && scores == nullptr) {   // nothing is evicted and no scores are wanted
    if (keep_out != nullptr)
      for (int j = tid; j < L; j += kFusedThreads) keep_out[(int64_t)unit * B + j] = j;
    return;
  }

  // Row addressing.  Paged: byte offset from the layer's pool base; contiguous: from the unit's row 0.
  const int64_t lbase = (int64_t)l * cv.layer_stride * E;
  const int64_t ubase = PAGED ? lbase : lbase + ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h) * E;
  const uint32_t rstride = (uint32_t)(cv.stride_s * E);
  const int bsh = cv.block_shift;
  auto blk_of = [&](int sl) -> int { return bsh >= 0 ? sl >> bsh : sl / cv.block_size; };
  auto row_off = [&](int sl) -> int64_t {
    if constexpr (PAGED) {
      const int bi = blk_of(sl);
      return s_blk[bi] + (int64_t)((sl - bi * cv.block_size) * H) * RB;
    } else {
      return (int64_t)((uint32_t)sl * rstride);
    }
  };
  int32_t *pbase = cv.pos + (int64_t)l * cv.pos_layer_stride +
                   (PAGED ? 0 : (int64_t)b * cv.pos_stride_b + (int64_t)h * cv.pos_stride_h);
  auto pos_idx = [&](int sl) -> int64_t {
    if constexpr (PAGED) {
      const int bi = blk_of(sl);
      return s_blk[bi] / RB + (int64_t)(sl - bi * cv.block_size) * H;
    } else {
      return sl;
    }
  };
  if constexpr (PAGED) {
    const int nblk = L > 0 ? blk_of(L - 1) + 1 : 0;
    const int32_t *trow = cv.block_table + (int64_t)b * cv.max_blocks;
    for (int i = tid; i < nblk; i += kFusedThreads) s_blk[i] = ((int64_t)trow[i] * cv.block_size * H + h) * RB;
    __syncthreads();
  }

  // ---- score every slot into s_key (and `scores` when asked)
  const char *kb = (const char *)cv.k + ubase;
  const int seg = lane % LPR, rsub = lane / LPR;
  auto load = [&](int row) -> KRow {
    KRow r;
    if (row >= L) {
      r.a = r.b = u32x4{0u, 0u, 0u, 0u};
      return r;
    }
    const char *p = kb + row_off(row) + seg * 16;
    r.a = fused_load((const u32x4 *)p);
    r.b = fused_load((const u32x4 *)(p + HB));
    return r;
  };
  const int wrow = wave * (RPW * UNR) + rsub;
  const int nsteps = (L + STEP - 1) / STEP;
  KRow cur[UNR], nxt[UNR];
  if (nsteps > 0) {
#pragma unroll
    for (int k = 0; k < UNR; ++k) cur[k] = load(wrow + k * RPW);
  }
  RS::centre(pv, (int64_t)l * H + h, pv.t[b], s_w, s_c, tid);
  __syncthreads();
  RS rs;
  rs.init(s_w, s_c, seg);
  float *out = scores != nullptr ? scores + (int64_t)unit * score_stride : nullptr;
  auto emit = [&](const KRow (&rows)[UNR], int r0) {
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const float sc = rs(rows[k]);
      const int row = r0 + k * RPW;
      if (seg == 0 && row < L) {
        s_key[row] = order_key(sc);
        if (out != nullptr) out[row] = sc;
      }
    }
  };
#pragma unroll 1
  for (int q = 0; q < nsteps; q += 2) {
    const int r0 = q * STEP + wrow;
    if (q + 1 < nsteps) {
#pragma unroll
      for (int k = 0; k < UNR; ++k) nxt[k] = load(r0 + STEP + k * RPW);
    }
    emit(cur, r0);
    if (q + 2 < nsteps) {
#pragma unroll
      for (int k = 0; k < UNR; ++k) cur[k] = load(r0 + 2 * STEP + k * RPW);
    }
    if (q + 1 < nsteps) emit(nxt, r0 + STEP);
  }
  int32_t *kout = keep_out != nullptr ? keep_out + (int64_t)unit * B : nullptr;
  if (!evict) {
    if (kout != nullptr)
      for (int j = tid; j < L; j += kFusedThreads) kout[j] = j;
    return;
  }
  __syncthreads();

  // ---- exact selection over s_key: keep the last R slots and the best K = B - R candidates of [0, n)
  const int n = L - R, K = B - R;
  const int base = tid * EPT;                 // this thread's slots: base .. base + EPT - 1
  uint32_t tau = 0xffffffffu, krem = 0u;
  if (K > 0) {
    uint32_t prefix = 0u, pmask = 0u, kr = (uint32_t)K;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < 2048; i += kFusedThreads) s_hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int sl = base + e;
        if (sl < n) {
          const uint32_t key = s_key[sl];
          if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      find_digit(s_hist, nb, 1, kr, s_scan, &s_digit, &s_krem);
      prefix |= s_digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      kr = s_krem;
    }
    tau = prefix;   // the K-th largest candidate key; keep every larger key and the first kr ties by slot
    krem = kr;
  }
  // Keep bits of this thread's slots; ties with tau are ranked across threads by one scan.
  uint32_t gt = 0u, eq = 0u, rec = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int sl = base + e;
    const uint32_t key = s_key[sl < L ? sl : 0];
    if (sl < n && K > 0) {
      gt |= (uint32_t)(key > tau) << e;
      eq |= (uint32_t)(key == tau) << e;
    } else if (sl >= n && sl < L) {
      rec |= 1u << e;
    }
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan((uint32_t)__popc(eq), s_scan, &tot);
  uint32_t keepm = gt | rec;
  {
    uint32_t m = eq;
    uint32_t r = eq_before;
    while (m != 0u && r < krem) {
      const int e = __ffs(m) - 1;
      keepm |= 1u << e;
      m &= m - 1u;
      ++r;
    }
  }
  const uint32_t dst = block_excl_scan((uint32_t)__popc(keepm), s_scan, &tot);
  {
    uint32_t m = keepm;
    uint32_t j = dst;
    while (m != 0u) {
      const int e = __ffs(m) - 1;
      s_keep[j++] = base + e;
      m &= m - 1u;
    }
  }
  __syncthreads();
  if (kout != nullptr)
    for (int j = tid; j < Ln; j += kFusedThreads) kout[j] = s_keep[j];

  // ---- move the retained rows in place, ascending chunks of CHUNK destinations
  char *kw = (char *)cv.k + ubase;
  char *vw = (char *)cv.v + ubase;
  const int mseg = tid % MLPR, mrow = tid / MLPR;
#pragma unroll 1
  for (int j0 = 0; j0 < Ln; j0 += CHUNK) {
    u32x4 kr[kFusedMovePasses], vr[kFusedMovePasses];
    int32_t pr[kFusedMovePasses];
    int src[kFusedMovePasses];
#pragma unroll
    for (int p = 0; p < kFusedMovePasses; ++p) {
      const int j = j0 + p * MRPP + mrow;
      src[p] = j < Ln ? s_keep[j] : j;
      kr[p] = vr[p] = u32x4{0u, 0u, 0u, 0u};
      pr[p] = 0;
      if (src[p] != j) {
        const int64_t o = row_off(src[p]);
        kr[p] = move_load((const u32x4 *)(kw + o) + mseg);
        vr[p] = move_load((const u32x4 *)(vw + o) + mseg);
        if (mseg == 0) pr[p] = pbase[pos_idx(src[p])];
      }
    }
    // every load of the chunk has returned before any of its stores (the asm consumes the registers)
#pragma unroll
    for (int p = 0; p < kFusedMovePasses; ++p) asm volatile("" ::"v"(kr[p]), "v"(vr[p]), "v"(pr[p]));
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kFusedMovePasses; ++p) {
      const int j = j0 + p * MRPP + mrow;
      if (src[p] != j) {
        const int64_t o = row_off(j);
        move_store((u32x4 *)(kw + o) + mseg, kr[p]);
        move_store((u32x4 *)(vw + o) + mseg, vr[p]);
        if (mseg == 0) pbase[pos_idx(j)] = pr[p];
      }
    }
  }
}

// ------------------------------------------------------------------------------------ calibration statistics


// Partial sums of one (layer, query head) over one chunk of kCalibChunk calibration tokens: for every element
// the sum of the queries, for every rotary pair the sum of |z_i(q)|, both in float64.  Lanes hold 16-byte
// chunks of both rotary halves like the scoring kernel, so half-split pairs meet inside a lane.  Output
// partial[((l*heads + h)*chunks + chunk)*(3D/2) + k]: k < D element sums, then D/2 pair-norm sums.
template <int DT, int D, int ROPE>
__global__ __launch_bounds__(512) void k_calib_partial(QueryView qv, double *__restrict__ partial, int chunks) {
  using RS = RowScorer<DT, D, ROPE>;
  constexpr int E = RS::E, HB = RS::HB, LPR = RS::LPR, VPC = RS::VPC;
  constexpr bool HALF = ROPE == TRI_ROPE_HALF;
  constexpr int RPW = 64 / LPR, WAVES = 8, RPB = RPW * WAVES;   // rows (tokens) per wave / workgroup load
  constexpr int UNR = 4;                                          // rows in flight per lane
  constexpr int NS = 2 * VPC + VPC;                               // sums per lane: 2*VPC elements, VPC pairs
  __shared__ double s_red[WAVES][LPR][NS];

  const int chunk = blockIdx.x % chunks;
  const int h = (blockIdx.x / chunks) % qv.heads;
  const int l = blockIdx.x / (chunks * qv.heads);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane % LPR, rsub = lane / LPR;
  const int64_t j0 = (int64_t)chunk * kCalibChunk;
  const int nrows = (int)min((int64_t)kCalibChunk, qv.n - j0);
  const char *base = (const char *)qv.q + ((int64_t)l * qv.stride_l + (int64_t)h * qv.stride_h) * E + seg * 16;
  const int64_t rstride = qv.stride_n * E;

  double acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0;
  auto element = [&](const u32x4 &x, int k) -> float {   // element k of a 16-byte chunk, widened exactly
    if constexpr (DT == TRI_BF16) return (k & 1) ? hi_bf16(x[k >> 1]) : lo_bf16(x[k >> 1]);
    else return __uint_as_float(x[k]);
  };
  auto add_row = [&](const u32x4 &a, const u32x4 &b) {
    float fa[VPC], fb[VPC];
#pragma unroll
    for (int k = 0; k < VPC; ++k) {
      fa[k] = element(a, k);
      fb[k] = element(b, k);
      acc[k] += (double)fa[k];
      acc[VPC + k] += (double)fb[k];
    }
    if constexpr (HALF) {
#pragma unroll
      for (int k = 0; k < VPC; ++k) acc[2 * VPC + k] += (double)__builtin_amdgcn_sqrtf(fmaf(fa[k], fa[k], fb[k] * fb[k]));
    } else {
#pragma unroll
      for (int m = 0; m < VPC / 2; ++m) {
        acc[2 * VPC + m] += (double)__builtin_amdgcn_sqrtf(fmaf(fa[2 * m], fa[2 * m], fa[2 * m + 1] * fa[2 * m + 1]));
        acc[2 * VPC + VPC / 2 + m] +=
            (double)__builtin_amdgcn_sqrtf(fmaf(fb[2 * m], fb[2 * m], fb[2 * m + 1] * fb[2 * m + 1]));
      }
    }
  };
  // Rows of this lane: wave*RPW + rsub + k*RPB for k = 0, 1, ...; UNR loads in flight.
  const int r0 = wave * RPW + rsub;
#pragma unroll 1
  for (int r = r0; r < nrows; r += UNR * RPB) {
    u32x4 a[UNR], b[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int rr = r + u * RPB;
      a[u] = b[u] = u32x4{0u, 0u, 0u, 0u};
      if (rr < nrows) {
        const char *p = base + (j0 + rr) * rstride;
        a[u] = __builtin_nontemporal_load((const u32x4 *)p);
        b[u] = __builtin_nontemporal_load((const u32x4 *)(p + HB));
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (r + u * RPB < nrows) add_row(a[u], b[u]);
  }
  // Sum over the rows of the wave (lanes with the same seg), then over the waves, in a fixed order.
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    double v = acc[k];
    for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o);
    acc[k] = v;
  }
  if (rsub == 0) {
#pragma unroll
    for (int k = 0; k < NS; ++k) s_red[wave][seg][k] = acc[k];
  }
  __syncthreads();
  double *out = partial + (((int64_t)l * qv.heads + h) * chunks + chunk) * (3 * D / 2);
  for (int t = tid; t < LPR * NS; t += blockDim.x) {
    const int sg = t / NS, k = t % NS;
    double v = 0.0;
    for (int w = 0; w < WAVES; ++w) v += s_red[w][sg][k];
    // destination: element sums by dimension, then pair-norm sums by pair
    int idx;
    if (k < VPC) idx = sg * VPC + k;                              // first half (or first chunk) element
    else if (k < 2 * VPC) idx = D / 2 + sg * VPC + (k - VPC);     // second half element
    else {
      const int m = k - 2 * VPC;
      int pair;
      if constexpr (HALF) pair = sg * VPC + m;
      else pair = m < VPC / 2 ? sg * (VPC / 2) + m : D / 4 + sg * (VPC / 2) + (m - VPC / 2);
      idx = D + pair;
    }
    out[idx] = v;
  }
}

// qbar and c of one (layer, head) from its partial sums, summed in chunk order.
template <int D, int ROPE>
__global__ __launch_bounds__(256) void k_calib_finish(QueryView qv, const double *__restrict__ partial, int chunks,
                                                      float *__restrict__ qbar, float *__restrict__ c) {
  constexpr bool HALF = ROPE == TRI_ROPE_HALF;
  __shared__ double s_mean[D];
  const int64_t lh = blockIdx.x;   // l*heads + h
  const double inv_n = 1.0 / (double)qv.n;
  const double *p = partial + lh * chunks * (3 * D / 2);
  for (int k = threadIdx.x; k < D; k += blockDim.x) {
    double v = 0.0;
    for (int ch = 0; ch < chunks; ++ch) v += p[(int64_t)ch * (3 * D / 2) + k];
    v *= inv_n;
    s_mean[k] = v;
    qbar[lh * D + k] = (float)v;
  }
  __syncthreads();   // the pair norms of the centre need every element mean
  for (int i = threadIdx.x; i < D / 2; i += blockDim.x) {
    double v = 0.0;
    for (int ch = 0; ch < chunks; ++ch) v += p[(int64_t)ch * (3 * D / 2) + D + i];
    const int pa = HALF ? i : 2 * i, pb = HALF ? i + D / 2 : 2 * i + 1;
    const double za = s_mean[pa], zb = s_mean[pb];
    c[lh * (D / 2) + i] = (float)(v * inv_n - sqrt(za * za + zb * zb));
  }
}

// ------------------------------------------------------------------------------------ decode attention


// One workgroup per (unit, split of dv.split keys, group of HG query heads): the query heads of a KV head
// attend over the unit's kept keys.  Lanes hold 16-byte chunks of both halves of a row (any split of the
// dimensions serves: the dot product sums over all of them); K and V rows stream together, and each lane group
// keeps an online softmax (running max m, sum l, weighted V sum) for its rows, merged across lane groups and
// waves at the end.  The partial (m, l, acc[D]) of every (unit, head, split) goes to `partial`.
template <int DT, int D, int HG, int PAGED>
__global__ __launch_bounds__(256) void k_decode_partial(CacheView cv, PassView pv, DecodeView dv,
                                                        float *__restrict__ partial) {
  constexpr int E = DT == TRI_BF16 ? 2 : 4;
  constexpr int HB = D * E / 2, LPR = HB / 16, VPC = 16 / E;
  constexpr int RPW = 64 / LPR, WAVES = 4, RPB = RPW * WAVES;
  constexpr int NE = 2 * VPC;                 // elements of a row held by one lane
  constexpr int UNR = 2;                      // K and V rows in flight per lane
  __shared__ int64_t s_blk[PAGED ? kDecodeSplitMax + 1 : 1];
  __shared__ float s_m[WAVES][HG], s_l[WAVES][HG];
  __shared__ float s_acc[WAVES][HG][D];

  const int ngroups = dv.group / HG;
  int bid = blockIdx.x;
  const int hgrp = bid % ngroups;
  bid /= ngroups;
  const int split = bid % dv.splits;
  const int unit = bid / dv.splits;
  const int H = cv.heads;
  const int h = unit % H, b = (unit / H) % cv.batch, l = unit / (H * cv.batch);
  const int L = min(pv.lengths[b], dv.max_length);
  const int j0 = split * dv.split;
  const int n = max(0, min(dv.split, L - j0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane % LPR, rsub = lane / LPR;

  // query slices (this lane's dims) of the HG heads, pre-multiplied by nothing: the scale applies to the dot
  const int hq0 = h * dv.group + hgrp * HG;
  const char *qb = (const char *)dv.q + (((int64_t)l * cv.batch + b) * dv.h_q + hq0) * D * E + seg * 16;
  u32x4 qa[HG], qc[HG];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    qa[g] = *(const u32x4 *)(qb + (int64_t)g * D * E);
    qc[g] = *(const u32x4 *)(qb + (int64_t)g * D * E + HB);
  }

  const int64_t lbase = (int64_t)l * cv.layer_stride * E;
  const int64_t ubase = PAGED ? lbase : lbase + ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h) * E;
  const int bsh = cv.block_shift;
  const int blk0 = PAGED && n > 0 ? (bsh >= 0 ? j0 >> bsh : j0 / cv.block_size) : 0;
  if constexpr (PAGED) {
    if (n > 0) {
      const int last = j0 + n - 1;
      const int nblk = (bsh >= 0 ? last >> bsh : last / cv.block_size) - blk0 + 1;
      for (int i = tid; i < nblk; i += blockDim.x)
        s_blk[i] = ((int64_t)cv.block_table[(int64_t)b * cv.max_blocks + blk0 + i] * cv.block_size * H + h) * (D * E);
    }
    __syncthreads();
  }
  auto row_off = [&](int sl) -> int64_t {
    if constexpr (PAGED) {
      const int bi = bsh >= 0 ? sl >> bsh : sl / cv.block_size;
      return s_blk[bi - blk0] + (int64_t)((sl - bi * cv.block_size) * H) * (D * E);
    } else {
      return (int64_t)sl * cv.stride_s * E;
    }
  };
  const char *kb = (const char *)cv.k + ubase + seg * 16;
  const char *vb = (const char *)cv.v + ubase + seg * 16;
  auto dot = [&](const u32x4 &qa_, const u32x4 &qc_, const KRow &x) -> float {
    float d = 0.f;
    if constexpr (DT == TRI_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d = dot2(qa_[i], x.a[i], d);
        d = dot2(qc_[i], x.b[i], d);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d = fmaf(__uint_as_float(qa_[i]), __uint_as_float(x.a[i]), d);
        d = fmaf(__uint_as_float(qc_[i]), __uint_as_float(x.b[i]), d);
      }
    }
    return d;
  };
  auto elem = [&](const KRow &x, int k) -> float {   // element k of the lane's NE elements of a row
    const u32x4 &c = k < VPC ? x.a : x.b;
    const int kk = k < VPC ? k : k - VPC;
    if constexpr (DT == TRI_BF16) return (kk & 1) ? hi_bf16(c[kk >> 1]) : lo_bf16(c[kk >> 1]);
    else return __uint_as_float(c[kk]);
  };

  float m[HG], lsum[HG], acc[HG][NE];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    m[g] = -__builtin_huge_valf();
    lsum[g] = 0.f;
#pragma unroll
    for (int k = 0; k < NE; ++k) acc[g][k] = 0.f;
  }
  // rows of this lane group: r = wave*RPW + rsub + k*RPB
#pragma unroll 1
  for (int r0 = wave * RPW + rsub; r0 - rsub < n; r0 += UNR * RPB) {
    KRow kr[UNR], vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = r0 + u * RPB;
      kr[u].a = kr[u].b = vr[u].a = vr[u].b = u32x4{0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t o = row_off(j0 + r);
        kr[u].a = __builtin_nontemporal_load((const u32x4 *)(kb + o));
        kr[u].b = __builtin_nontemporal_load((const u32x4 *)(kb + o + HB));
        vr[u].a = __builtin_nontemporal_load((const u32x4 *)(vb + o));
        vr[u].b = __builtin_nontemporal_load((const u32x4 *)(vb + o + HB));
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (r0 + u * RPB < n) {   // uniform over the lane group
#pragma unroll
        for (int g = 0; g < HG; ++g) {
          const float sc = group_sum<LPR>(dot(qa[g], qc[g], kr[u])) * dv.scale;
          const float mn = fmaxf(m[g], sc);
          const float corr = __expf(m[g] - mn);        // 0 while m is still -inf
          const float p = __expf(sc - mn);
          lsum[g] = fmaf(lsum[g], corr, p);
#pragma unroll
          for (int k = 0; k < NE; ++k) acc[g][k] = fmaf(p, elem(vr[u], k), acc[g][k] * corr);
          m[g] = mn;
        }
      }
    }
  }
  // Merge the lane groups of a wave (lanes with the same seg), then the waves.  Weights of a side whose
  // running max is -inf (no rows) are 0.
  auto weights = [](float m1, float m2, float &c1, float &c2) -> float {
    const float mn = fmaxf(m1, m2);
    c1 = m1 == -__builtin_huge_valf() ? 0.f : __expf(m1 - mn);
    c2 = m2 == -__builtin_huge_valf() ? 0.f : __expf(m2 - mn);
    return mn;
  };
#pragma unroll
  for (int g = 0; g < HG; ++g) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m[g], o), l2 = __shfl_xor(lsum[g], o);
      float c1, c2;
      const float mn = weights(m[g], m2, c1, c2);
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const float a2 = __shfl_xor(acc[g][k], o);
        acc[g][k] = acc[g][k] * c1 + a2 * c2;
      }
      lsum[g] = lsum[g] * c1 + l2 * c2;
      m[g] = mn;
    }
    if (rsub == 0) {
      if (seg == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = lsum[g];
      }
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int dim = k < VPC ? seg * VPC + k : D / 2 + seg * VPC + (k - VPC);
        s_acc[wave][g][dim] = acc[g][k];
      }
    }
  }
  __syncthreads();
  for (int t = tid; t < HG * D; t += blockDim.x) {
    const int g = t / D, dim = t % D;
    float mm = -__builtin_huge_valf(), ll = 0.f, aa = 0.f;
    for (int w = 0; w < WAVES; ++w) {
      float c1, c2;
      const float mn = weights(mm, s_m[w][g], c1, c2);
      ll = ll * c1 + s_l[w][g] * c2;
      aa = aa * c1 + s_acc[w][g][dim] * c2;
      mm = mn;
    }
    float *o = partial + (((int64_t)unit * dv.group + hgrp * HG + g) * dv.splits + split) * (D + 2);
    o[2 + dim] = aa;
    if (dim == 0) {
      o[0] = mm;
      o[1] = ll;
    }
  }
}

// out[l][b][hq][:] from the splits' partials of (unit, head): weights exp(m_s - max m) on each split's sums.
template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(CacheView cv, DecodeView dv, const float *__restrict__ partial,
                                                      float *__restrict__ out) {
  const int ug = blockIdx.x;                       // unit * group + g
  const int g = ug % dv.group, unit = ug / dv.group;
  const int H = cv.heads;
  const int h = unit % H, b = (unit / H) % cv.batch, l = unit / (H * cv.batch);
  const float *p = partial + (int64_t)ug * dv.splits * (D + 2);
  float mx = -__builtin_huge_valf();
  for (int s = 0; s < dv.splits; ++s) mx = fmaxf(mx, p[s * (D + 2)]);
  float ll = 0.f, aa = 0.f;
  if (mx != -__builtin_huge_valf()) {
    for (int s = 0; s < dv.splits; ++s) {
      const float w = __expf(p[s * (D + 2)] - mx);   // 0 for empty splits (m = -inf)
      ll = fmaf(w, p[s * (D + 2) + 1], ll);
      aa = fmaf(w, p[s * (D + 2) + 2 + threadIdx.x], aa);
    }
  }
  out[(((int64_t)l * cv.batch + b) * dv.h_q + h * dv.group + g) * D + threadIdx.x] = ll > 0.f ? aa / ll : 0.f;
}

// ------------------------------------------------------------------------------------ precondition check

__global__ void k_check_reset(uint32_t *check, uint32_t *claims, int64_t n_claims) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *check = 0u;
  if (i < n_claims) claims[i] = 0u;
}

// One workgroup per sequence: its length and decode position, then its used block-table entries (paged); the
// violated bits are OR-ed into *check.  claims: one bit per pool block, set by the entry that uses it.
__global__ __launch_bounds__(256) void k_check(CacheView cv, PassView pv, int32_t capacity, int32_t max_length,
                                               int32_t num_blocks, uint32_t *check, uint32_t *claims) {
  const int b = blockIdx.x;
  const int32_t *row = cv.paged ? cv.block_table + (int64_t)b * cv.max_blocks : nullptr;
  const uint32_t bits = check_entries(pv.lengths[b], pv.t[b], capacity, max_length, row, cv.block_size, num_blocks,
                                      claims != nullptr,
                                      [&](int32_t w, uint32_t bit) { return atomicOr(&claims[w], bit); },
                                      (int)threadIdx.x, (int)blockDim.x);
  if (bits != 0u) atomicOr(check, bits);
}

}  // namespace

hipError_t launch_check(const CacheView &cv, const PassView &pv, int32_t capacity, int32_t max_length,
                        int32_t num_blocks, uint32_t *check, uint32_t *claims, hipStream_t s) {
  const int64_t n_claims = claims != nullptr ? ((int64_t)num_blocks + 31) / 32 : 0;
  const int64_t n = std::max<int64_t>(n_claims, 1);
  hipLaunchKernelGGL(k_check_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, check, claims, n_claims);
  hipLaunchKernelGGL(k_check, dim3(cv.batch), dim3(256), 0, s, cv, pv, capacity, max_length, num_blocks, check, claims);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ launchers

hipError_t launch_prepare(const float *qbar, const float *c, int layers, int h_q, int h_kv, int d, double theta,
                          int rope, const int32_t *offsets_host, int n_offsets, float *u, float *c_hat,
                          hipStream_t s) {
  Offsets offs{};
  for (int i = 0; i < n_offsets; ++i) offs.v[i] = offsets_host[i];
  hipLaunchKernelGGL(k_prepare, dim3(layers * h_kv), dim3(64), 0, s, qbar, c, h_q, h_kv, d, theta, rope, offs,
                     n_offsets, u, c_hat);
  return hipGetLastError();
}

template <int DT, int D, int ROPE, int PAGED>
static void score_one(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, uint32_t *range,
                      hipStream_t s) {
  const int tiles = (cv.capacity + kScoreTile - 1) / kScoreTile;
  const int64_t grid = (int64_t)cv.layers * cv.batch * tiles * cv.heads;
  // keys of the pass (at most: every unit at the launch bound) that fit in the 256 MB infinity cache with room to
  // spare are loaded through it
  const int64_t key_bytes = (int64_t)cv.layers * cv.batch * cv.heads * cv.capacity * D * (DT == TRI_BF16 ? 2 : 4);
  const dim3 g((unsigned)(grid * kRangeParts)), blk(64 * kRangeWaves);
  if (key_bytes <= kTemporalKeyBytes)
    hipLaunchKernelGGL((k_score<DT, D, ROPE, PAGED, 1>), g, blk, 0, s, cv, pv, scores, stride, tiles, range);
  else
    hipLaunchKernelGGL((k_score<DT, D, ROPE, PAGED, 0>), g, blk, 0, s, cv, pv, scores, stride, tiles, range);
}

template <int DT, int D, int ROPE>
static void score_layout(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, uint32_t *range,
                         hipStream_t s) {
  if (cv.paged) score_one<DT, D, ROPE, 1>(cv, pv, scores, stride, range, s);
  else score_one<DT, D, ROPE, 0>(cv, pv, scores, stride, range, s);
}

template <int DT, int D>
static void score_rope(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, uint32_t *range,
                       hipStream_t s) {
  if (cv.rope == TRI_ROPE_HALF) score_layout<DT, D, TRI_ROPE_HALF>(cv, pv, scores, stride, range, s);
  else score_layout<DT, D, TRI_ROPE_INTERLEAVED>(cv, pv, scores, stride, range, s);
}

template <int D, int ROPE>
static void score_var(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, uint32_t *range,
                      hipStream_t s) {
  const int tiles = (cv.capacity + kScoreTile - 1) / kScoreTile;
  const int cols = (tiles + kVarTiles - 1) / kVarTiles;   // workgroups per (unit, part), each every cols-th tile
  const int64_t grid = (int64_t)cv.layers * cv.batch * cols * kVarParts * cv.heads;
  if (grid == 0) return;
  const dim3 g((unsigned)grid), t(64 * kVarWaves);
  // paged pools whose blocks hold whole 16-key steps take the whole-row loads (PAGED == 2)
  const int pg = !cv.paged ? 0 : (cv.block_size % 16 == 0 ? 2 : 1);
#define TRI_VAR_LAUNCH(P, A, X) \
  hipLaunchKernelGGL((k_score_var<D, ROPE, P, A, X>), g, t, 0, s, cv, pv, scores, stride, tiles, cols, range)
#define TRI_VAR_AGG(P, X)                                              \
  do {                                                                 \
    if (pv.agg == TRI_AGG_MAX) TRI_VAR_LAUNCH(P, TRI_AGG_MAX, X);      \
    else TRI_VAR_LAUNCH(P, TRI_AGG_HEAD_MAX, X);                       \
  } while (0)
  const bool x = pv.columns > 64;   // 128 columns: four more tiles from LDS
  if (pg == 0) { if (x) TRI_VAR_AGG(0, 1); else TRI_VAR_AGG(0, 0); }
  else if (pg == 1) { if (x) TRI_VAR_AGG(1, 1); else TRI_VAR_AGG(1, 0); }
  else { if (x) TRI_VAR_AGG(2, 1); else TRI_VAR_AGG(2, 0); }
#undef TRI_VAR_AGG
#undef TRI_VAR_LAUNCH
}

hipError_t launch_prepare_variant(const float *qbar, int layers, int h_q, int h_kv, int d, double theta, int rope,
                                  const int32_t *offsets_host, int n_offsets, float *centres, hipStream_t s) {
  Offsets offs{};
  for (int i = 0; i < n_offsets; ++i) offs.v[i] = offsets_host[i];
  const int G = h_q / h_kv;
  hipLaunchKernelGGL(k_prepare_variant, dim3(layers * h_kv), dim3(256), 0, s, qbar, h_q, h_kv, d, theta, rope, offs,
                     n_offsets, tri_variant_columns(G, n_offsets), variant_dpad(n_offsets), centres);
  return hipGetLastError();
}

hipError_t launch_score(const CacheView &cv, const PassView &pv, float *scores, int64_t score_stride, uint32_t *range,
                        hipStream_t s) {
  if (pv.agg != 0) {   // aggregation variants: bf16 caches, the host checked
    if (cv.head_dim == 128) {
      if (cv.rope == TRI_ROPE_HALF) score_var<128, TRI_ROPE_HALF>(cv, pv, scores, score_stride, range, s);
      else score_var<128, TRI_ROPE_INTERLEAVED>(cv, pv, scores, score_stride, range, s);
    } else {
      if (cv.rope == TRI_ROPE_HALF) score_var<64, TRI_ROPE_HALF>(cv, pv, scores, score_stride, range, s);
      else score_var<64, TRI_ROPE_INTERLEAVED>(cv, pv, scores, score_stride, range, s);
    }
    return hipGetLastError();
  }
  if (cv.dtype == TRI_BF16) {
    if (cv.head_dim == 128) score_rope<TRI_BF16, 128>(cv, pv, scores, score_stride, range, s);
    else score_rope<TRI_BF16, 64>(cv, pv, scores, score_stride, range, s);
  } else {
    if (cv.head_dim == 128) score_rope<TRI_F32, 128>(cv, pv, scores, score_stride, range, s);
    else score_rope<TRI_F32, 64>(cv, pv, scores, score_stride, range, s);
  }
  return hipGetLastError();
}

hipError_t launch_select(const CacheView &cv, const PassView &pv, const float *scores, int64_t score_stride,
                         int32_t *keep, int32_t *new_lengths, uint32_t *flags, uint32_t *counter, uint32_t *range,
                         hipStream_t s) {
  const int units = cv.layers * cv.batch * cv.heads;
  const int cpu = (pv.budget + kCompactChunk - 1) / kCompactChunk;
  const int cap = cv.capacity;
  const int tiles = (cap + kScoreTile - 1) / kScoreTile;
  dim3 g(units);
#define TRI_SELECT(T, EPT)                                                                                       \
  hipLaunchKernelGGL((k_select<T, EPT, 0>), g, dim3(T), 0, s, cv, pv, scores, score_stride, keep, new_lengths,   \
                     flags, counter, cpu, range, tiles, nullptr, nullptr, nullptr)
  if (cap <= 512 * 8) TRI_SELECT(512, 8);
  else if (cap <= 512 * 16) TRI_SELECT(512, 16);
  else if (cap <= 512 * 32) TRI_SELECT(512, 32);
  else if (cap <= 512 * 64) TRI_SELECT(512, 64);
  else if (cap <= 1024 * 48) TRI_SELECT(1024, 48);
  else TRI_SELECT(1024, 64);
#undef TRI_SELECT
  return hipGetLastError();
}

bool select_moves_fit(const CacheView &cv, const PassView &pv) {
  return pv.budget <= kMoveKeepMax &&
         (!cv.paged || (int64_t)(cv.capacity + cv.block_size - 1) / cv.block_size <= kMoveTableMax);
}

hipError_t launch_select_move(const CacheView &cv, const PassView &pv, const float *scores, int64_t score_stride,
                              int32_t *keep, int32_t *new_lengths, uint32_t *range, int32_t *block_table_out,
                              int32_t *freed, int32_t *n_freed, hipStream_t s) {
  const int units = cv.layers * cv.batch * cv.heads;
  const int cap = cv.capacity;
  const int tiles = (cap + kScoreTile - 1) / kScoreTile;
  dim3 g((unsigned)(cv.paged ? xcd_grouped_grid(cv.heads, cv.layers * cv.batch) : units));
#define TRI_SELECT(T, EPT)                                                                                       \
  hipLaunchKernelGGL((k_select<T, EPT, 1>), g, dim3(T), 0, s, cv, pv, scores, score_stride, keep, new_lengths,   \
                     nullptr, nullptr, 0, range, tiles, block_table_out, freed, n_freed)
  if (cap <= 512 * 8) TRI_SELECT(512, 8);
  else if (cap <= 512 * 16) TRI_SELECT(512, 16);
  else if (cap <= 512 * 32) TRI_SELECT(512, 32);
  else if (cap <= 512 * 64) TRI_SELECT(512, 64);
  else if (cap <= 1024 * 48) TRI_SELECT(1024, 48);
  else TRI_SELECT(1024, 64);
#undef TRI_SELECT
  return hipGetLastError();
}

hipError_t launch_reset(uint32_t *flags, int64_t n_flags, uint32_t *counter, int64_t units, hipStream_t s) {
  const int64_t n = std::max<int64_t>(std::max<int64_t>(n_flags, units), 1);
  hipLaunchKernelGGL(k_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, flags, n_flags, counter, units);
  return hipGetLastError();
}

hipError_t launch_compact(const CacheView &cv, const PassView &pv, const int32_t *keep, int32_t *block_table_out,
                          int32_t *freed, int32_t *n_freed, uint32_t *flags, uint32_t *counter, hipStream_t s) {
  const int units = cv.layers * cv.batch * cv.heads;
  const int cpu = (pv.budget + kCompactChunk - 1) / kCompactChunk;
  const int64_t grid = (int64_t)units * cpu;
  const int rb = cv.head_dim * (cv.dtype == TRI_BF16 ? 2 : 4);
  dim3 g((unsigned)grid), blk(kCompactThreads);
#define TRI_COMPACT(RB, P) \
  hipLaunchKernelGGL((k_compact<RB, P>), g, blk, 0, s, cv, pv, keep, block_table_out, freed, n_freed, flags, counter, cpu)
  if (cv.paged) {
    if (rb == 128) TRI_COMPACT(128, 1);
    else if (rb == 256) TRI_COMPACT(256, 1);
    else TRI_COMPACT(512, 1);
  } else {
    if (rb == 128) TRI_COMPACT(128, 0);
    else if (rb == 256) TRI_COMPACT(256, 0);
    else TRI_COMPACT(512, 0);
  }
#undef TRI_COMPACT
  return hipGetLastError();
}

bool fused_fits(const CacheView &cv) {
  if (cv.capacity > kFusedMax) return false;
  if (cv.paged && (int64_t)(cv.capacity + cv.block_size - 1) / cv.block_size > kFusedBlocks) return false;
  return true;
}

template <int DT, int D, int ROPE>
static void fused_layout(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, int32_t *keep,
                         int32_t *new_lengths, int32_t *table_out, int32_t *freed, int32_t *n_freed, hipStream_t s) {
  const dim3 g((unsigned)(cv.paged ? xcd_grouped_grid(cv.heads, cv.layers * cv.batch)
                                     : (int64_t)cv.layers * cv.batch * cv.heads)),
      blk(kFusedThreads);
  if (cv.paged)
    hipLaunchKernelGGL((k_fused<DT, D, ROPE, 1>), g, blk, 0, s, cv, pv, scores, stride, keep, new_lengths, table_out,
                       freed, n_freed);
  else
    hipLaunchKernelGGL((k_fused<DT, D, ROPE, 0>), g, blk, 0, s, cv, pv, scores, stride, keep, new_lengths, table_out,
                       freed, n_freed);
}

template <int DT, int D>
static void fused_rope(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, int32_t *keep,
                       int32_t *new_lengths, int32_t *table_out, int32_t *freed, int32_t *n_freed, hipStream_t s) {
  if (cv.rope == TRI_ROPE_HALF)
    fused_layout<DT, D, TRI_ROPE_HALF>(cv, pv, scores, stride, keep, new_lengths, table_out, freed, n_freed, s);
  else
    fused_layout<DT, D, TRI_ROPE_INTERLEAVED>(cv, pv, scores, stride, keep, new_lengths, table_out, freed, n_freed, s);
}

hipError_t launch_fused(const CacheView &cv, const PassView &pv, float *scores, int64_t score_stride, int32_t *keep,
                        int32_t *new_lengths, int32_t *block_table_out, int32_t *freed, int32_t *n_freed,
                        hipStream_t s) {
#define TRI_FUSED(DT, D) \
  fused_rope<DT, D>(cv, pv, scores, score_stride, keep, new_lengths, block_table_out, freed, n_freed, s)
  if (cv.dtype == TRI_BF16) {
    if (cv.head_dim == 128) TRI_FUSED(TRI_BF16, 128);
    else TRI_FUSED(TRI_BF16, 64);
  } else {
    if (cv.head_dim == 128) TRI_FUSED(TRI_F32, 128);
    else TRI_FUSED(TRI_F32, 64);
  }
#undef TRI_FUSED
  return hipGetLastError();
}

template <int DT, int D, int ROPE>
static void calib_one(const QueryView &qv, double *partial, float *qbar, float *c, hipStream_t s) {
  const int chunks = (int)((qv.n + kCalibChunk - 1) / kCalibChunk);
  const int64_t grid = (int64_t)qv.layers * qv.heads * chunks;
  hipLaunchKernelGGL((k_calib_partial<DT, D, ROPE>), dim3((unsigned)grid), dim3(512), 0, s, qv, partial, chunks);
  hipLaunchKernelGGL((k_calib_finish<D, ROPE>), dim3((unsigned)((int64_t)qv.layers * qv.heads)), dim3(256), 0, s, qv,
                     (const double *)partial, chunks, qbar, c);
}

template <int DT, int D>
static void calib_rope(const QueryView &qv, double *partial, float *qbar, float *c, hipStream_t s) {
  if (qv.rope == TRI_ROPE_HALF) calib_one<DT, D, TRI_ROPE_HALF>(qv, partial, qbar, c, s);
  else calib_one<DT, D, TRI_ROPE_INTERLEAVED>(qv, partial, qbar, c, s);
}

hipError_t launch_calibrate(const QueryView &qv, double *partial, float *qbar, float *c, hipStream_t s) {
  if (qv.dtype == TRI_BF16) {
    if (qv.head_dim == 128) calib_rope<TRI_BF16, 128>(qv, partial, qbar, c, s);
    else calib_rope<TRI_BF16, 64>(qv, partial, qbar, c, s);
  } else {
    if (qv.head_dim == 128) calib_rope<TRI_F32, 128>(qv, partial, qbar, c, s);
    else calib_rope<TRI_F32, 64>(qv, partial, qbar, c, s);
  }
  return hipGetLastError();
}

int decode_split(int64_t units, int max_length) {
  int split = kDecodeSplitMax;
  while (split > 512 && units * ((max_length + split - 1) / split) < 4096) split /= 2;
  return split;
}

template <int DT, int D, int HG, int PAGED>
static void decode_one(const CacheView &cv, const PassView &pv, const DecodeView &dv, float *partial, float *out,
                       hipStream_t s) {
  const int64_t units = (int64_t)cv.layers * cv.batch * cv.heads;
  const int64_t grid = units * dv.splits * (dv.group / HG);
  hipLaunchKernelGGL((k_decode_partial<DT, D, HG, PAGED>), dim3((unsigned)grid), dim3(256), 0, s, cv, pv, dv, partial);
  hipLaunchKernelGGL((k_decode_combine<D>), dim3((unsigned)(units * dv.group)), dim3(D), 0, s, cv, dv,
                     (const float *)partial, out);
}

template <int DT, int D, int HG>
static void decode_layout(const CacheView &cv, const PassView &pv, const DecodeView &dv, float *partial, float *out,
                          hipStream_t s) {
  if (cv.paged) decode_one<DT, D, HG, 1>(cv, pv, dv, partial, out, s);
  else decode_one<DT, D, HG, 0>(cv, pv, dv, partial, out, s);
}

template <int DT, int D>
static void decode_group(const CacheView &cv, const PassView &pv, const DecodeView &dv, float *partial, float *out,
                         hipStream_t s) {
  // heads per workgroup: the whole group up to 4 (larger groups take several workgroups per split)
  if (dv.group == 1) decode_layout<DT, D, 1>(cv, pv, dv, partial, out, s);
  else if (dv.group == 2) decode_layout<DT, D, 2>(cv, pv, dv, partial, out, s);
  else decode_layout<DT, D, 4>(cv, pv, dv, partial, out, s);
}

hipError_t launch_decode(const CacheView &cv, const PassView &pv, const DecodeView &dv, float *partial, float *out,
                         hipStream_t s) {
  if (cv.dtype == TRI_BF16) {
    if (cv.head_dim == 128) decode_group<TRI_BF16, 128>(cv, pv, dv, partial, out, s);
    else decode_group<TRI_BF16, 64>(cv, pv, dv, partial, out, s);
  } else {
    if (cv.head_dim == 128) decode_group<TRI_F32, 128>(cv, pv, dv, partial, out, s);
    else decode_group<TRI_F32, 64>(cv, pv, dv, partial, out, s);
  }
  return hipGetLastError();
}

}  // namespace tri
