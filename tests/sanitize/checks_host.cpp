// The device-side precondition checks (csrc/tri_checks.h, the code the check kernel runs) on the host, against
// hand-made bad inputs: lengths outside the capacity or the host bound, decode positions before the length, block
// ids out of range and used twice.  Exit status 0 when every case sets exactly the expected bits.  Test
// infrastructure only.
#include <cstdio>
#include <vector>

#include "tri_checks.h"

static int g_fail = 0;

static void expect(uint32_t got, uint32_t want, const char *what) {
  if (got != want) {
    std::printf("%s: bits %u, want %u\n", what, got, want);
    ++g_fail;
  }
}

// a whole call's check on the host: every sequence, `stride` simulated threads each, one claims bitmap
static uint32_t check_call(const std::vector<int32_t> &lengths, const std::vector<int32_t> &t, int32_t capacity,
                           int32_t max_length, const std::vector<int32_t> *table, int32_t max_blocks,
                           int32_t block_size, int32_t num_blocks, bool claims, int stride) {
  std::vector<uint32_t> bitmap((num_blocks + 31) / 32, 0u);
  auto claim_or = [&](int32_t w, uint32_t bit) {
    const uint32_t old = bitmap[w];
    bitmap[w] |= bit;
    return old;
  };
  uint32_t bits = 0u;
  for (size_t b = 0; b < lengths.size(); ++b) {
    const int32_t *row = table ? table->data() + b * max_blocks : nullptr;
    for (int th = 0; th < stride; ++th)
      bits |= tri::check_entries(lengths[b], t[b], capacity, max_length, row, block_size, num_blocks, claims, claim_or,
                                 th, stride);
  }
  return bits;
}

int main() {
  // sequences
  expect(tri::check_sequence(100, 100, 4096, 0), 0u, "valid");
  expect(tri::check_sequence(0, 0, 4096, 0), 0u, "empty");
  expect(tri::check_sequence(4096, 5000, 4096, 0), 0u, "full capacity");
  expect(tri::check_sequence(4097, 5000, 4096, 0), TRI_CHECK_LENGTH, "over capacity");
  expect(tri::check_sequence(-1, 5, 4096, 0), TRI_CHECK_LENGTH, "negative length");
  expect(tri::check_sequence(3000, 3000, 4096, 2500), TRI_CHECK_LENGTH, "over the host bound");
  expect(tri::check_sequence(2500, 2500, 4096, 2500), 0u, "at the host bound");
  expect(tri::check_sequence(100, 99, 4096, 0), TRI_CHECK_DECODE_POS, "decode position before the length");
  expect(tri::check_sequence(5000, 10, 4096, 0), TRI_CHECK_LENGTH | TRI_CHECK_DECODE_POS, "both");
  expect(tri::check_used_blocks(33, 4096, 16), 3u, "used blocks");
  expect(tri::check_used_blocks(5000, 4096, 16), 0u, "no entries read for a bad length");

  // paged calls: 3 sequences, 4 table entries each, 10 pool blocks, blocks of 16 slots
  const int32_t mb = 4, bs = 16, nb = 10, cap = mb * bs;
  const std::vector<int32_t> L = {40, 17, 64}, T = {40, 17, 64};
  std::vector<int32_t> good = {1, 2, 3, -1, 4, 5, -1, -1, 6, 7, 8, 9};
  for (int stride : {1, 2, 256}) {
    expect(check_call(L, T, cap, 0, &good, mb, bs, nb, true, stride), 0u, "valid table");
    std::vector<int32_t> t2 = good;
    t2[2] = 10;   // the third used entry of sequence 0 out of range
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, true, stride), TRI_CHECK_BLOCK_RANGE, "id == num_blocks");
    t2 = good;
    t2[9] = -3;
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, true, stride), TRI_CHECK_BLOCK_RANGE, "negative id");
    t2 = good;
    t2[3] = 9;    // an unused entry (sequence 0 uses 3 of its 4): not checked
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, true, stride), 0u, "unused entry ignored");
    t2 = good;
    t2[5] = 2;    // sequence 1's second block is sequence 0's second block
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, true, stride), TRI_CHECK_BLOCK_DUP, "block used twice");
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, false, stride), 0u, "duplicates unchecked without claims");
    t2 = good;
    t2[11] = 8;   // twice within one row
    expect(check_call(L, T, cap, 0, &t2, mb, bs, nb, true, stride), TRI_CHECK_BLOCK_DUP, "twice in one row");
    std::vector<int32_t> L2 = L;
    L2[1] = 65;   // over capacity: its entries are not read
    std::vector<int32_t> t3 = good;
    t3[6] = 99;
    expect(check_call(L2, {40, 80, 64}, cap, 0, &t3, mb, bs, nb, true, stride), TRI_CHECK_LENGTH, "bad length");
  }
  // contiguous: sequences only
  expect(check_call({10, 20}, {10, 19}, 4096, 0, nullptr, 0, 16, 0, false, 4), TRI_CHECK_DECODE_POS, "contiguous");
  std::printf("%s: %d failures\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
