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
//   k_score    streams K with 128-bit loads; a row of d elements is owned by an aligned group of
//              LPR = d*elem/16 lanes; the half-split rotary partner of a lane is LPR/2 lanes away
//              (one DPP row_ror:8 exchange for 16-lane rows); the row sum is a DPP butterfly.
//   k_select   one 1024-thread workgroup per unit; keys stay in registers; three LDS radix
//              histogram passes (11/11/10 bits) find the threshold; ties go to the lower slot;
//              two block scans emit the ascending keep list.
//   k_compact  workgroups take ordered tickets for (unit, destination chunk); each loads the rows it
//              moves, publishes "sources loaded", waits only for earlier chunks of its unit whose
//              sources reach into its destination range, then stores.  Destination j <= source
//              keep[j] makes that the only hazard of the in-place move.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kDppRor8 = 0x128;       // row_ror:8  (== lane ^ 8 inside a 16-lane row)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Value held by lane ^ (LPR/2).
template <int LPR>
__device__ __forceinline__ uint32_t partner_u32(uint32_t x) {
  if constexpr (LPR == 16) return dpp_u32<kDppRor8>(x);
  else return (uint32_t)__shfl_xor((int)x, LPR / 2);
}

// Sum over each aligned group of LPR lanes (LPR in {8, 16, 32}); every lane gets the sum.
// After the two quad steps the four lanes of a quad agree, so the mirrors act as xor 4 / xor 8.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_f32<kDppMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

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

// ------------------------------------------------------------------------------------ score

constexpr int kScoreWaves = 4;
constexpr int kScoreUnroll = 8;

// Grid: ((layer*batch + seq)*tiles + tile)*heads + head.  One workgroup scores kScoreTile rows of one
// unit; each wave owns a contiguous quarter of the tile.
template <int DT, int D, int ROPE, int PAGED>
__global__ __launch_bounds__(256) void k_score(CacheView cv, PassView pv, float *__restrict__ scores,
                                                int64_t score_stride, int tiles) {
  constexpr int E = DT == TRI_BF16 ? 2 : 4;
  constexpr int LPR = D * E / 16;            // lanes per row
  constexpr int VPL = 16 / E;                // elements per lane
  constexpr int RPW = 64 / LPR;              // rows per wave per load
  constexpr int ROWS_PER_WAVE = kScoreTile / kScoreWaves;
  constexpr int STEP = RPW * kScoreUnroll;
  constexpr int ITERS = ROWS_PER_WAVE / STEP;
  constexpr bool HALF = ROPE == TRI_ROPE_HALF;
  static_assert(ITERS * STEP == ROWS_PER_WAVE, "tile shape");

  __shared__ float s_w[D];
  __shared__ float s_c[D / 2];

  const int H = cv.heads;
  int bid = blockIdx.x;
  const int h = bid % H;
  bid /= H;
  const int tile = bid % tiles;
  bid /= tiles;
  const int b = bid % cv.batch;
  const int l = bid / cv.batch;
  const int L = pv.lengths[b];
  const int tile0 = tile * kScoreTile;
  if (tile0 >= L) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane % LPR, rsub = lane / LPR;
  const int rbase = tile0 + wave * ROWS_PER_WAVE + rsub;

  const char *kbase = (const char *)cv.k + (int64_t)l * cv.layer_stride * E;
  auto load_row = [&](int row) -> u32x4 {
    if (row >= L) return u32x4{0u, 0u, 0u, 0u};
    const char *p;
    if constexpr (PAGED) {
      const int blk = cv.block_table[(int64_t)b * cv.max_blocks + row / cv.block_size];
      const int o = row % cv.block_size;
      p = kbase + (((int64_t)blk * cv.block_size + o) * H + h) * (int64_t)(D * E);
    } else {
      p = kbase + ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h + (int64_t)row * cv.stride_s) * E;
    }
    return __builtin_nontemporal_load((const u32x4 *)p + seg);
  };

  // First batch of loads goes out before the prologue so its latency hides the float64 math.
  u32x4 cur[kScoreUnroll];
#pragma unroll
  for (int k = 0; k < kScoreUnroll; ++k) cur[k] = load_row(rbase + k * RPW);

  const int64_t ukv = (int64_t)l * H + h;
  if (tid < D / 2) {
    const int i = tid;
    const double om = pow(pv.theta, -2.0 * i / D);
    double sn, cs;
    sincos((double)pv.t[b] * om, &sn, &cs);
    const int pa = HALF ? i : 2 * i;
    const int pb = HALF ? i + D / 2 : 2 * i + 1;
    const double ua = pv.u[ukv * D + pa], ub = pv.u[ukv * D + pb];
    s_w[pa] = (float)(ua * cs - ub * sn);
    s_w[pb] = (float)(ua * sn + ub * cs);
    s_c[i] = pv.c_hat[ukv * (D / 2) + i];
  }
  __syncthreads();

  const bool first = seg < LPR / 2;
  float wr[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) wr[k] = s_w[seg * VPL + k];
  float cr[VPL / 2];
  const int cbase = HALF ? (first ? seg * VPL : (seg - LPR / 2) * VPL + VPL / 2) : seg * (VPL / 2);
#pragma unroll
  for (int k = 0; k < VPL / 2; ++k) cr[k] = s_c[cbase + k];

  auto row_score = [&](u32x4 x) -> float {
    float dot = 0.f, nrm = 0.f;
    if constexpr (DT == TRI_BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dot = fmaf(wr[2 * k], lo_bf16(x[k]), dot);
        dot = fmaf(wr[2 * k + 1], hi_bf16(x[k]), dot);
      }
      if constexpr (HALF) {
        const uint32_t q0 = partner_u32<LPR>(first ? x[2] : x[0]);
        const uint32_t q1 = partner_u32<LPR>(first ? x[3] : x[1]);
        const uint32_t a0 = first ? x[0] : x[2], a1 = first ? x[1] : x[3];
        float p, r;
        p = lo_bf16(a0); r = lo_bf16(q0); nrm = fmaf(cr[0], __builtin_amdgcn_sqrtf(fmaf(p, p, r * r)), nrm);
        p = hi_bf16(a0); r = hi_bf16(q0); nrm = fmaf(cr[1], __builtin_amdgcn_sqrtf(fmaf(p, p, r * r)), nrm);
        p = lo_bf16(a1); r = lo_bf16(q1); nrm = fmaf(cr[2], __builtin_amdgcn_sqrtf(fmaf(p, p, r * r)), nrm);
        p = hi_bf16(a1); r = hi_bf16(q1); nrm = fmaf(cr[3], __builtin_amdgcn_sqrtf(fmaf(p, p, r * r)), nrm);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float p = lo_bf16(x[k]), r = hi_bf16(x[k]);
          nrm = fmaf(cr[k], __builtin_amdgcn_sqrtf(fmaf(p, p, r * r)), nrm);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) dot = fmaf(wr[k], __uint_as_float(x[k]), dot);
      if constexpr (HALF) {
        const float q0 = __uint_as_float(partner_u32<LPR>(first ? x[2] : x[0]));
        const float q1 = __uint_as_float(partner_u32<LPR>(first ? x[3] : x[1]));
        const float a0 = __uint_as_float(first ? x[0] : x[2]), a1 = __uint_as_float(first ? x[1] : x[3]);
        nrm = fmaf(cr[0], __builtin_amdgcn_sqrtf(fmaf(a0, a0, q0 * q0)), nrm);
        nrm = fmaf(cr[1], __builtin_amdgcn_sqrtf(fmaf(a1, a1, q1 * q1)), nrm);
      } else {
        const float f0 = __uint_as_float(x[0]), f1 = __uint_as_float(x[1]);
        const float f2 = __uint_as_float(x[2]), f3 = __uint_as_float(x[3]);
        nrm = fmaf(cr[0], __builtin_amdgcn_sqrtf(fmaf(f0, f0, f1 * f1)), nrm);
        nrm = fmaf(cr[1], __builtin_amdgcn_sqrtf(fmaf(f2, f2, f3 * f3)), nrm);
      }
    }
    return group_sum<LPR>(dot + nrm);
  };

  float *out = scores + ((int64_t)(l * cv.batch + b) * H + h) * score_stride;
#pragma unroll 1
  for (int it = 0; it < ITERS; ++it) {
    const int r0 = rbase + it * STEP;
    u32x4 nxt[kScoreUnroll];
    if (it + 1 < ITERS) {
#pragma unroll
      for (int k = 0; k < kScoreUnroll; ++k) nxt[k] = load_row(r0 + STEP + k * RPW);
    }
#pragma unroll
    for (int k = 0; k < kScoreUnroll; ++k) {
      const float s = row_score(cur[k]);
      const int row = r0 + k * RPW;
      if (seg == 0 && row < L) out[row] = s;
    }
    if (it + 1 < ITERS) {
#pragma unroll
      for (int k = 0; k < kScoreUnroll; ++k) cur[k] = nxt[k];
    }
  }
}

// ------------------------------------------------------------------------------------ select

// Order-preserving map of a float score to uint32: larger score -> larger key.  NaN ranks as -inf
// and -0 as +0, so equal keys mean equal rank values.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) x = 0xff800000u;
  if (x == 0x80000000u) x = 0u;
  return (x & 0x80000000u) ? ~x : (x | 0x80000000u);
}

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

// One workgroup per unit (grid = units).  Thread t owns slots [t*EPT, (t+1)*EPT) so that slot order
// is (thread, element) order and the emitted keep list is ascending.
template <int EPT>
__global__ __launch_bounds__(kSelectThreads) void k_select(CacheView cv, PassView pv, const float *__restrict__ scores,
                                                           int64_t score_stride, int32_t *__restrict__ keep,
                                                           int32_t *__restrict__ new_lengths, uint32_t *flags,
                                                           uint32_t *counter, int chunks_per_unit) {
  static_assert(EPT % 4 == 0, "float4 loads");
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan_smem[33];
  __shared__ uint32_t s_digit, s_krem;

  const int unit = blockIdx.x;
  const int H = cv.heads;
  const int h = unit % H;
  const int b = (unit / H) % cv.batch;
  const int l = unit / (H * cv.batch);
  const int tid = threadIdx.x;
  const int L = pv.lengths[b], B = pv.budget, R = pv.recent;

  if (flags != nullptr) {  // compaction control words of this unit start at zero
    for (int c = tid; c < chunks_per_unit; c += blockDim.x) flags[(int64_t)unit * chunks_per_unit + c] = 0u;
    if (unit == 0 && tid == 0) *counter = 0u;
  }
  if (l == 0 && h == 0 && tid == 0) new_lengths[b] = min(L, B);

  int32_t *out = keep + (int64_t)unit * B;
  if (L <= B) {
    for (int j = tid; j < L; j += blockDim.x) out[j] = j;
    return;
  }
  const int n = L - R, K = B - R;
  for (int j = tid; j < R; j += blockDim.x) out[K + j] = n + j;
  if (K == 0) return;

  const float *sc = scores + (int64_t)unit * score_stride;
  const int base = tid * EPT;
  uint32_t key[EPT];
#pragma unroll
  for (int q = 0; q < EPT; q += 4) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (base + q < n) f = *(const float4 *)(sc + base + q);
    key[q] = order_key(f.x);
    key[q + 1] = order_key(f.y);
    key[q + 2] = order_key(f.z);
    key[q + 3] = order_key(f.w);
  }

  // Radix select of the K-th largest key among candidate slots [0, n): digits of 11, 11, 10 bits.
  uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (base + e < n && (key[e] & pmask) == prefix) atomicAdd(&hist[(key[e] >> shift) & (uint32_t)(nb - 1)], 1u);
    __syncthreads();
    // bins from the top: thread t owns bins nb-1-t*bpt .. nb-bpt-t*bpt
    const int bpt = nb / kSelectThreads;
    uint32_t loc = 0u;
    for (int k = 0; k < bpt; ++k) loc += hist[nb - 1 - (tid * bpt + k)];
    uint32_t tot;
    uint32_t cum = block_excl_scan(loc, scan_smem, &tot);
    for (int k = 0; k < bpt; ++k) {
      const int bin = nb - 1 - (tid * bpt + k);
      const uint32_t hc = hist[bin];
      if (cum < krem && krem <= cum + hc) {
        s_digit = (uint32_t)bin;
        s_krem = krem - cum;
      }
      cum += hc;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem = s_krem;
  }
  const uint32_t tau = prefix;  // the K-th largest key; krem of its ties are kept, lowest slots first

  uint32_t nties = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) nties += (base + e < n && key[e] == tau) ? 1u : 0u;
  uint32_t tot;
  const uint32_t tie0 = block_excl_scan(nties, scan_smem, &tot);
  uint32_t nkeep = 0u, tr = tie0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (base + e < n) {
      const bool tie = key[e] == tau;
      nkeep += (key[e] > tau || (tie && tr < krem)) ? 1u : 0u;
      tr += tie ? 1u : 0u;
    }
  }
  uint32_t dst = block_excl_scan(nkeep, scan_smem, &tot);
  tr = tie0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (base + e < n) {
      const bool tie = key[e] == tau;
      if (key[e] > tau || (tie && tr < krem)) out[dst++] = base + e;
      tr += tie ? 1u : 0u;
    }
  }
}

// ------------------------------------------------------------------------------------ compact

__global__ void k_reset(uint32_t *flags, int64_t n, uint32_t *counter) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) flags[i] = 0u;
  if (i == 0) *counter = 0u;
}

constexpr int kCompactThreads = 256;

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

  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = (int)atomicAdd(counter, 1u);
  __syncthreads();
  const int ticket = s_ticket;
  const int unit = ticket / cpu, c = ticket % cpu;
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

  const int64_t lk = (int64_t)l * cv.layer_stride * (RB / (cv.head_dim));  // bytes to this layer
  char *kb = (char *)cv.k + lk;
  char *vb = (char *)cv.v + lk;
  int32_t *pb = cv.pos + (int64_t)l * cv.pos_layer_stride;
  auto row_off = [&](int s) -> int64_t {  // byte offset of slot s's row within the layer
    if constexpr (PAGED) {
      const int blk = cv.block_table[(int64_t)b * cv.max_blocks + s / cv.block_size];
      return (((int64_t)blk * cv.block_size + s % cv.block_size) * H + h) * (int64_t)RB;
    } else {
      return ((int64_t)b * cv.stride_b + (int64_t)h * cv.stride_h + (int64_t)s * cv.stride_s) * (RB / cv.head_dim);
    }
  };
  auto pos_off = [&](int s) -> int64_t {
    if constexpr (PAGED) {
      const int blk = cv.block_table[(int64_t)b * cv.max_blocks + s / cv.block_size];
      return ((int64_t)blk * cv.block_size + s % cv.block_size) * H + h;
    } else {
      return (int64_t)b * cv.pos_stride_b + (int64_t)h * cv.pos_stride_h + s;
    }
  };

  u32x4 kr[NP], vr[NP];
  int src[NP];
  int32_t pr[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    kr[p] = vr[p] = u32x4{0u, 0u, 0u, 0u};
    pr[p] = 0;
    src[p] = j;
    if (j < j1) {
      const int s = kp[j];
      src[p] = s;
      if (s != j) {
        const int64_t o = row_off(s);
        kr[p] = *((const u32x4 *)(kb + o) + seg);
        vr[p] = *((const u32x4 *)(vb + o) + seg);
        if (seg == 0) pr[p] = pb[pos_off(s)];
      }
    }
  }
  // Publish "my sources are loaded", then wait for earlier chunks whose sources overlap my destinations.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t *fl = flags + (int64_t)unit * cpu;
    __hip_atomic_store(&fl[c], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    for (int cc = c - 1; cc >= 0; --cc) {
      if (kp[(cc + 1) * kCompactChunk - 1] < j0) break;  // keep is ascending: earlier chunks reach even less far
      while (__hip_atomic_load(&fl[cc], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int j = j0 + p * RPP + rr;
    if (j < j1 && src[p] != j) {
      const int64_t o = row_off(j);
      *((u32x4 *)(kb + o) + seg) = kr[p];
      *((u32x4 *)(vb + o) + seg) = vr[p];
      if (seg == 0) pb[pos_off(j)] = pr[p];
    }
  }
}

}  // namespace

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
static void score_one(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, hipStream_t s) {
  const int tiles = (cv.capacity + kScoreTile - 1) / kScoreTile;
  const int64_t grid = (int64_t)cv.layers * cv.batch * tiles * cv.heads;
  hipLaunchKernelGGL((k_score<DT, D, ROPE, PAGED>), dim3((unsigned)grid), dim3(256), 0, s, cv, pv, scores, stride,
                     tiles);
}

template <int DT, int D, int ROPE>
static void score_layout(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, hipStream_t s) {
  if (cv.paged) score_one<DT, D, ROPE, 1>(cv, pv, scores, stride, s);
  else score_one<DT, D, ROPE, 0>(cv, pv, scores, stride, s);
}

template <int DT, int D>
static void score_rope(const CacheView &cv, const PassView &pv, float *scores, int64_t stride, hipStream_t s) {
  if (cv.rope == TRI_ROPE_HALF) score_layout<DT, D, TRI_ROPE_HALF>(cv, pv, scores, stride, s);
  else score_layout<DT, D, TRI_ROPE_INTERLEAVED>(cv, pv, scores, stride, s);
}

hipError_t launch_score(const CacheView &cv, const PassView &pv, float *scores, int64_t score_stride, hipStream_t s) {
  if (cv.dtype == TRI_BF16) {
    if (cv.head_dim == 128) score_rope<TRI_BF16, 128>(cv, pv, scores, score_stride, s);
    else score_rope<TRI_BF16, 64>(cv, pv, scores, score_stride, s);
  } else {
    if (cv.head_dim == 128) score_rope<TRI_F32, 128>(cv, pv, scores, score_stride, s);
    else score_rope<TRI_F32, 64>(cv, pv, scores, score_stride, s);
  }
  return hipGetLastError();
}

hipError_t launch_select(const CacheView &cv, const PassView &pv, const float *scores, int64_t score_stride,
                         int32_t *keep, int32_t *new_lengths, uint32_t *flags, uint32_t *counter, hipStream_t s) {
  const int units = cv.layers * cv.batch * cv.heads;
  const int cpu = (pv.budget + kCompactChunk - 1) / kCompactChunk;
  const int cap = cv.capacity;
  dim3 g(units), blk(kSelectThreads);
#define TRI_SELECT(EPT) \
  hipLaunchKernelGGL(k_select<EPT>, g, blk, 0, s, cv, pv, scores, score_stride, keep, new_lengths, flags, counter, cpu)
  if (cap <= 4 * kSelectThreads) TRI_SELECT(4);
  else if (cap <= 8 * kSelectThreads) TRI_SELECT(8);
  else if (cap <= 16 * kSelectThreads) TRI_SELECT(16);
  else if (cap <= 32 * kSelectThreads) TRI_SELECT(32);
  else if (cap <= 48 * kSelectThreads) TRI_SELECT(48);
  else TRI_SELECT(64);
#undef TRI_SELECT
  return hipGetLastError();
}

hipError_t launch_reset(uint32_t *flags, int64_t n_flags, uint32_t *counter, hipStream_t s) {
  const int64_t n = n_flags > 0 ? n_flags : 1;
  hipLaunchKernelGGL(k_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, flags, n_flags, counter);
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

}  // namespace tri
