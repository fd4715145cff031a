/*
 * CPU oracle of the whole eviction pass in the collapsed form, float64, plain C with OpenMP over units.
 * TEST INFRASTRUCTURE ONLY: the test-suite and the CPU-baseline leg of the benchmark load it; the GPU path
 * never does and shares no code with it.
 *
 * What it computes, for every unit (one layer, sequence and KV head) independently
 * ("TriAttention：基于三角函数 KV 压缩的高效长推理", 流程详解 steps 2-5; "WeianMao/triattention", How it works):
 *   score      s(p) = w . K[p] + sum_i chat_i |z_i(K[p])|,  w = RoPE(u, t)            (steps 2 and 3)
 *              where u is the mean over the KV head's query heads g and the offsets Delta of
 *              RoPE(qbar_g, Delta): the distance series averaged over heads and offsets is linear in the
 *              stored key, so it equals this one dot product (the plain definition is cross-checked against
 *              it in the tests).  z_i is the i-th rotary pair, RoPE(x, n) turns it by n * theta^(-2i/d).
 *   selection  L <= budget: every slot.  Otherwise the last `recent` slots, plus the best budget - recent of
 *              slots 0 .. L-recent-1 by score (higher first; NaN lowest, -0 equal to +0), then position (lower
 *              first); the kept slots in ascending order                                     (step 4)
 *   gather     row j of the output K, V and pos is row keep[j] of the input, bit for bit  (step 5)
 * Keys and values are bf16 bit patterns (widened exactly to float64 for the score); positions int32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

static double bf16_to_double(uint16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return (double)x.f;
}

/* rotary pair i of a row of d elements: (x[i], x[i + d/2]) for the half-split layout, (x[2i], x[2i+1]) else */
static int pair_a(int i, int d, int half) { return half ? i : 2 * i; }
static int pair_b(int i, int d, int half) { return half ? i + d / 2 : 2 * i + 1; }

/* ranking value: NaN as -inf, -0 as +0 */
static double rank_value(double s) {
  if (isnan(s)) return -INFINITY;
  return s + 0.0;
}

typedef struct {
  double s;
  int32_t pos;
  int32_t slot;
} cand;

/* higher score first, then lower position */
static int by_score_then_position(const void *pa, const void *pb) {
  const cand *a = (const cand *)pa, *b = (const cand *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

static int ascending(const void *pa, const void *pb) {
  const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/*
 * n_units units; unit i has len[i] rows starting at row row0[i] of k, v (row-major [rows][d] bf16 bits) and pos.
 *   u     float64 [n_units][d]    the unit's centre vector (mean of RoPE(qbar_g, Delta) over heads and offsets)
 *   chat  float64 [n_units][d/2]  the unit's group-mean norm coefficients
 *   t     int32 [n_units]         decode position of the unit's sequence
 * Outputs (any may be NULL): scores float64 at the input rows; keep int32 [n_units][budget]; k_out, v_out
 * [n_units][budget][d] and pos_out [n_units][budget] (rows past min(L, budget) untouched); new_len [n_units].
 * threads: OpenMP threads (<= 0: the runtime's default).  Returns 0, or -1 on bad arguments.
 */
int tri_oracle_collapsed_pass(int n_units, const int32_t *len, const int64_t *row0, const uint16_t *k,
                              const uint16_t *v, const int32_t *pos, const double *u, const double *chat,
                              const int32_t *t, int d, double theta, int half, int budget, int recent, int threads,
                              double *scores, int32_t *keep, uint16_t *k_out, uint16_t *v_out, int32_t *pos_out,
                              int32_t *new_len) {
  if (n_units < 0 || d < 2 || d % 2 || budget < 1 || recent < 0 || recent > budget || !(theta > 0.0)) return -1;
  const int nt = threads > 0 ? threads : omp_get_max_threads();
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : bad)
  for (int ui = 0; ui < n_units; ++ui) {
    const int L = len[ui];
    const int64_t r0 = row0[ui];
    /* w = RoPE(u, t): pair i turned by t * omega_i, angles in float64 */
    double *w = (double *)malloc(sizeof(double) * d);
    double *s = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
    cand *c = (cand *)malloc(sizeof(cand) * (L > 0 ? L : 1));
    int32_t *kept = (int32_t *)malloc(sizeof(int32_t) * budget);
    if (!w || !s || !c || !kept) {
      bad = 1;
      free(w), free(s), free(c), free(kept);
      continue;
    }
    for (int i = 0; i < d / 2; ++i) {
      const double om = pow(theta, -2.0 * i / d);
      const double ang = (double)t[ui] * om;
      const double ua = u[(int64_t)ui * d + pair_a(i, d, half)], ub = u[(int64_t)ui * d + pair_b(i, d, half)];
      w[pair_a(i, d, half)] = ua * cos(ang) - ub * sin(ang);
      w[pair_b(i, d, half)] = ua * sin(ang) + ub * cos(ang);
    }
    /* score of every cached slot */
    for (int p = 0; p < L; ++p) {
      const uint16_t *row = k + (r0 + p) * d;
      double dot = 0.0, nrm = 0.0;
      for (int e = 0; e < d; ++e) dot += w[e] * bf16_to_double(row[e]);
      for (int i = 0; i < d / 2; ++i) {
        const double a = bf16_to_double(row[pair_a(i, d, half)]), b = bf16_to_double(row[pair_b(i, d, half)]);
        nrm += chat[(int64_t)ui * (d / 2) + i] * sqrt(a * a + b * b);
      }
      s[p] = dot + nrm;
      if (scores) scores[r0 + p] = s[p];
    }
    /* selection */
    int n_keep;
    if (L <= budget) {
      n_keep = L;
      for (int j = 0; j < L; ++j) kept[j] = j;
    } else {
      const int n = L - recent, K = budget - recent;
      for (int p = 0; p < n; ++p) {
        c[p].s = rank_value(s[p]);
        c[p].pos = pos[r0 + p];
        c[p].slot = p;
      }
      qsort(c, (size_t)n, sizeof(cand), by_score_then_position);
      for (int j = 0; j < K; ++j) kept[j] = c[j].slot;
      for (int j = 0; j < recent; ++j) kept[K + j] = n + j;
      qsort(kept, (size_t)budget, sizeof(int32_t), ascending);
      n_keep = budget;
    }
    /* gather */
    for (int j = 0; j < n_keep; ++j) {
      const int64_t src = r0 + kept[j];
      const int64_t dst = (int64_t)ui * budget + j;
      if (keep) keep[dst] = kept[j];
      if (k_out) memcpy(k_out + dst * d, k + src * d, sizeof(uint16_t) * d);
      if (v_out) memcpy(v_out + dst * d, v + src * d, sizeof(uint16_t) * d);
      if (pos_out) pos_out[dst] = pos[src];
    }
    if (new_len) new_len[ui] = n_keep;
    free(w), free(s), free(c), free(kept);
  }
  return bad ? -1 : 0;
}
