// Drives the C ABI's host-side validation (api.cpp, linked with launch_stubs.cpp instead of the kernels) through
// every entry point's error paths and some valid calls, under the host sanitizers.  Device pointers are fake,
// aligned addresses: the validation never dereferences them.  Exit status 0 when every call returned the expected
// status and every non-OK status left a message.  Test infrastructure only.
#include <cstdio>
#include <cstring>
#include <vector>

#include "tri.h"

extern int g_launches;

static int g_fail = 0;
#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const tri_status st_ = (call);                                                                      \
    if (st_ != (want)) {                                                                                \
      std::printf("line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, st_, (want), tri_last_error()); \
      ++g_fail;                                                                                         \
    } else if (st_ != TRI_OK && std::strlen(tri_last_error()) == 0) {                                   \
      std::printf("line %d: %s: no message\n", __LINE__, #call);                                        \
      ++g_fail;                                                                                         \
    }                                                                                                   \
  } while (0)

template <typename T>
static T *fake(uintptr_t a) { return reinterpret_cast<T *>(a); }

static tri_cache contiguous() {
  tri_cache c{};
  c.layout = TRI_CONTIGUOUS, c.dtype = TRI_BF16, c.rope = TRI_ROPE_HALF;
  c.num_layers = 2, c.batch = 3, c.num_kv_heads = 4, c.head_dim = 128, c.max_len = 5000;
  c.k = fake<void>(0x10000000), c.v = fake<void>(0x20000000), c.pos = fake<int32_t>(0x30000000);
  c.stride_s = 128, c.stride_h = 5000 * 128, c.stride_b = 4LL * 5000 * 128, c.layer_stride = 3LL * 4 * 5000 * 128;
  c.pos_stride_h = 5000, c.pos_stride_b = 4 * 5000, c.pos_layer_stride = 3 * 4 * 5000;
  return c;
}

static tri_cache paged() {
  tri_cache c{};
  c.layout = TRI_PAGED, c.dtype = TRI_BF16, c.rope = TRI_ROPE_INTERLEAVED;
  c.num_layers = 2, c.batch = 3, c.num_kv_heads = 8, c.head_dim = 128;
  c.k = fake<void>(0x10000000), c.v = fake<void>(0x20000000), c.pos = fake<int32_t>(0x30000000);
  c.layer_stride = 1000LL * 16 * 8 * 128, c.pos_layer_stride = 1000 * 16 * 8;
  c.block_size = 16, c.num_blocks = 1000, c.max_blocks_per_seq = 300;
  c.block_table = fake<const int32_t>(0x40000000);
  return c;
}

static tri_params params() {
  tri_params p{};
  p.u = fake<const float>(0x50000000), p.c_hat = fake<const float>(0x51000000);
  p.lengths = fake<const int32_t>(0x52000000), p.t = fake<const int32_t>(0x53000000);
  p.rope_theta = 1e6, p.budget = 700, p.recent = 64;
  return p;
}

int main() {
  hipStream_t s = nullptr;
  float *scores = fake<float>(0x60000000);
  int32_t *keep = fake<int32_t>(0x61000000), *nl = fake<int32_t>(0x62000000);
  int32_t *bto = fake<int32_t>(0x63000000), *fr = fake<int32_t>(0x64000000), *nf = fake<int32_t>(0x65000000);
  void *ws = fake<void>(0x70000000);

  for (int i = -1; i <= 5; ++i) (void)tri_status_string((tri_status)i);
  if (tri_score_stride(nullptr) != 0) ++g_fail;
  if (tri_workspace_bytes(nullptr, nullptr) != 0) ++g_fail;

  // valid calls reach the (stubbed) launchers
  for (tri_cache c : {contiguous(), paged()}) {
    tri_params p = params();
    const size_t need = tri_workspace_bytes(&c, &p);
    if (need == 0) ++g_fail;
    const bool pg = c.layout == TRI_PAGED;
    EXPECT(tri_score(&c, &p, scores, s), TRI_OK);
    EXPECT(tri_topk(&c, &p, scores, keep, nl, s), TRI_OK);
    EXPECT(tri_compact(&c, &p, keep, pg ? bto : nullptr, pg ? fr : nullptr, pg ? nf : nullptr, ws, need, s), TRI_OK);
    EXPECT(tri_evict_step(&c, &p, nullptr, nullptr, nl, pg ? bto : nullptr, pg ? fr : nullptr, pg ? nf : nullptr, ws,
                          need, s), TRI_OK);
    hipEvent_t ev[4] = {fake<ihipEvent_t>(8), fake<ihipEvent_t>(16), fake<ihipEvent_t>(24), fake<ihipEvent_t>(32)};
    EXPECT(tri_evict_step_profiled(&c, &p, scores, keep, nl, pg ? bto : nullptr, pg ? fr : nullptr,
                                   pg ? nf : nullptr, ws, need, s, ev), TRI_OK);
    p.max_length = 3000, p.flags = TRI_PASS_UNFUSED;
    EXPECT(tri_evict_step(&c, &p, scores, keep, nl, pg ? bto : nullptr, pg ? fr : nullptr, pg ? nf : nullptr, ws,
                          tri_workspace_bytes(&c, &p), s), TRI_OK);
    // workspace, outputs and aliasing
    EXPECT(tri_evict_step(&c, &p, scores, keep, nl, pg ? bto : nullptr, pg ? fr : nullptr, pg ? nf : nullptr, ws,
                          16, s), TRI_ERR_WORKSPACE);
    EXPECT(tri_evict_step(&c, &p, scores, keep, nl, pg ? bto : nullptr, pg ? fr : nullptr, pg ? nf : nullptr,
                          fake<void>(0x70000010), need, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_evict_step(&c, &p, scores, keep, const_cast<int32_t *>(p.lengths), pg ? bto : nullptr,
                          pg ? fr : nullptr, pg ? nf : nullptr, ws, need, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_evict_step(&c, &p, fake<float>(0x60000004), keep, nl, pg ? bto : nullptr, pg ? fr : nullptr,
                          pg ? nf : nullptr, ws, need, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_evict_step(&c, &p, scores, keep, nl, pg ? nullptr : bto, pg ? fr : nullptr, pg ? nf : nullptr, ws,
                          need, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_evict_step_profiled(&c, &p, scores, keep, nl, pg ? bto : nullptr, pg ? fr : nullptr,
                                   pg ? nf : nullptr, ws, need, s, nullptr), TRI_ERR_INVALID_ARG);
  }

  // every parameter check
  const tri_cache c0 = contiguous();
  auto bad_params = [&](void (*edit)(tri_params &), tri_status want) {
    tri_params p = params();
    edit(p);
    EXPECT(tri_score(&c0, &p, scores, s), want);
    if (tri_workspace_bytes(&c0, &p) != 0) ++g_fail;
  };
  bad_params([](tri_params &p) { p.u = nullptr; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.lengths = fake<const int32_t>(0x52000002); }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.rope_theta = -1.0; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.rope_theta = 1.0 / 0.0; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.budget = 0; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.recent = 701; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.recent = -1; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.max_length = 5001; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.flags = 3; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.flags = 64; }, TRI_ERR_INVALID_ARG);
  static tri_variant var{fake<const float>(0x80000000), TRI_AGG_MAX, 4, 13, 0};
  static tri_variant var_bad{fake<const float>(0x80000000), 7, 4, 13, 0};
  static tri_variant var_group{fake<const float>(0x80000000), TRI_AGG_MAX, 9, 13, 0};   // 144 columns
  bad_params([](tri_params &p) { p.variant = &var_bad; }, TRI_ERR_INVALID_ARG);
  bad_params([](tri_params &p) { p.variant = &var_group; }, TRI_ERR_UNSUPPORTED);
  {
    tri_params p = params();
    p.variant = &var;
    EXPECT(tri_score(&c0, &p, scores, s), TRI_OK);
  }

  // every cache check
  auto bad_cache = [&](tri_cache c, tri_status want) {
    tri_params p = params();
    EXPECT(tri_score(&c, &p, scores, s), want);
  };
  { tri_cache c = c0; c.layout = 5; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.dtype = 9; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.rope = 2; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.head_dim = 96; bad_cache(c, TRI_ERR_UNSUPPORTED); }
  { tri_cache c = c0; c.num_layers = 0; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.k = nullptr; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.v = fake<void>(0x20000008); bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.pos = fake<int32_t>(0x30000002); bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.stride_s = 100; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.stride_s = 64; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.stride_h = -8; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.max_len = 0; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = c0; c.max_len = 70000; c.stride_s = 128; bad_cache(c, TRI_ERR_UNSUPPORTED); }
  { tri_cache c = c0; c.stride_s = 1 << 20; bad_cache(c, TRI_ERR_UNSUPPORTED); }
  { tri_cache c = c0; c.batch = 1 << 20; c.num_layers = 1 << 11; bad_cache(c, TRI_ERR_UNSUPPORTED); }
  { tri_cache c = paged(); c.block_table = nullptr; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = paged(); c.block_size = 0; bad_cache(c, TRI_ERR_INVALID_ARG); }
  { tri_cache c = paged(); c.max_blocks_per_seq = 5000; bad_cache(c, TRI_ERR_UNSUPPORTED); }
  EXPECT(tri_score(nullptr, nullptr, scores, s), TRI_ERR_INVALID_ARG);
  {
    tri_params p = params();
    EXPECT(tri_score(&c0, nullptr, scores, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_score(&c0, &p, nullptr, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_topk(&c0, &p, scores, nullptr, nl, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_compact(&c0, &p, keep, nullptr, nullptr, nullptr, nullptr, 0, s), TRI_ERR_INVALID_ARG);
  }

  // centres
  const int32_t offs[3] = {1, 2, 4};
  float *u = fake<float>(0x90000000), *ch = fake<float>(0x91000000);
  const float *qb = fake<const float>(0x92000000), *cc = fake<const float>(0x93000000);
  EXPECT(tri_prepare_centres(qb, cc, 2, 32, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, ch, s), TRI_OK);
  EXPECT(tri_prepare_centres(qb, cc, 2, 30, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, ch, s), TRI_ERR_INVALID_ARG);
  EXPECT(tri_prepare_centres(qb, cc, 2, 32, 8, 128, 1e6, TRI_ROPE_HALF, offs, 0, u, ch, s), TRI_ERR_INVALID_ARG);
  EXPECT(tri_prepare_centres(qb, cc, 2, 32, 8, 128, 1e6, TRI_ROPE_HALF, offs, 65, u, ch, s), TRI_ERR_INVALID_ARG);
  EXPECT(tri_prepare_centres(qb, cc, 2, 32, 8, 80, 1e6, TRI_ROPE_HALF, offs, 3, u, ch, s), TRI_ERR_UNSUPPORTED);
  EXPECT(tri_prepare_centres(nullptr, cc, 2, 32, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, ch, s), TRI_ERR_INVALID_ARG);
  EXPECT(tri_prepare_variant_centres(qb, 2, 32, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, s), TRI_OK);
  EXPECT(tri_prepare_variant_centres(qb, 2, 64, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, s), TRI_OK);
  EXPECT(tri_prepare_variant_centres(qb, 2, 72, 8, 128, 1e6, TRI_ROPE_HALF, offs, 3, u, s), TRI_ERR_UNSUPPORTED);
  if (tri_variant_columns(4, 13) != 64 || tri_variant_columns(8, 13) != 128 || tri_variant_columns(4, 32) != 128 ||
      tri_variant_columns(8, 17) != 0 || tri_variant_columns(2, 33) != 0 || tri_variant_columns(0, 4) != 0)
    ++g_fail;
  EXPECT(tri_prepare_variant_centres(qb, 2, 32, 8, 128, 1e6, 7, offs, 3, u, s), TRI_ERR_INVALID_ARG);

  // decode attention
  {
    tri_cache c = paged();
    const size_t need = tri_decode_workspace_bytes(&c, 32, 2048);
    if (need == 0) ++g_fail;
    EXPECT(tri_decode_attention(&c, nl, 2048, fake<void>(0xa0000000), 32, 0.088f, scores, ws, need, s), TRI_OK);
    EXPECT(tri_decode_attention(&c, nl, 2048, fake<void>(0xa0000000), 24, 0.088f, scores, ws, need, s),
           TRI_ERR_UNSUPPORTED);
    EXPECT(tri_decode_attention(&c, nl, 0, fake<void>(0xa0000000), 32, 0.088f, scores, ws, need, s),
           TRI_ERR_INVALID_ARG);
    EXPECT(tri_decode_attention(&c, nl, 2048, fake<void>(0xa0000000), 32, 0.088f, scores, ws, need - 1, s),
           TRI_ERR_WORKSPACE);
    EXPECT(tri_decode_attention(&c, nl, 2048, fake<void>(0xa0000008), 32, 0.088f, scores, ws, need, s),
           TRI_ERR_INVALID_ARG);
  }
  // calibration
  {
    tri_queries q{};
    q.dtype = TRI_BF16, q.rope = TRI_ROPE_HALF, q.num_layers = 2, q.num_heads = 32, q.head_dim = 128, q.n = 4096;
    q.q = fake<const void>(0xb0000000), q.stride_n = 32 * 128, q.stride_h = 128, q.stride_l = 4096LL * 32 * 128;
    const size_t need = tri_calibrate_workspace_bytes(&q);
    if (need == 0) ++g_fail;
    EXPECT(tri_calibrate(&q, u, ch, ws, need, s), TRI_OK);
    EXPECT(tri_calibrate(&q, u, ch, ws, need - 8, s), TRI_ERR_WORKSPACE);
    q.reserved = 1;
    EXPECT(tri_calibrate(&q, u, ch, ws, need, s), TRI_ERR_INVALID_ARG);
    q.reserved = 0, q.stride_n = 3;
    EXPECT(tri_calibrate(&q, u, ch, ws, need, s), TRI_ERR_INVALID_ARG);
    EXPECT(tri_calibrate(nullptr, u, ch, ws, need, s), TRI_ERR_INVALID_ARG);
  }
  if (g_launches < 15) {
    std::printf("only %d launches reached\n", g_launches);
    ++g_fail;
  }
  std::printf("%s: %d failures, %d launches reached\n", g_fail ? "FAIL" : "ok", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
