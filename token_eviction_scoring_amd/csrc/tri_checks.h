// Device-side data preconditions of the pass, as plain predicates shared by the check kernel and a host test.
// The pass reads lengths, decode positions and block tables on the device only; when the caller asks for checks
// (tri_params.check), one kernel evaluates these for every sequence and table entry before anything else runs,
// and every kernel of the pass returns at entry if any failed -- so a bad entry makes the pass skip its accesses
// instead of making them out of bounds.
#pragma once
#include <stdint.h>

#include "tri.h"

#if defined(__HIPCC__)
#define TRI_HD __host__ __device__
#else
#define TRI_HD
#endif

namespace tri {

// Precondition bits of a sequence: its cached length within [0, capacity] and within the host bound max_length
// when one is given (0: none), and its decode position at least its length.
TRI_HD inline uint32_t check_sequence(int32_t length, int32_t t, int32_t capacity, int32_t max_length) {
  uint32_t bits = 0u;
  if (length < 0 || length > capacity || (max_length > 0 && length > max_length)) bits |= TRI_CHECK_LENGTH;
  if (length >= 0 && t < length) bits |= TRI_CHECK_DECODE_POS;
  return bits;
}

// Entries of a paged sequence's block-table row that hold its slots: ceil(length / block_size), none for a length
// that already failed its check.
TRI_HD inline int32_t check_used_blocks(int32_t length, int32_t capacity, int32_t block_size) {
  if (length <= 0 || length > capacity) return 0;
  return (length + block_size - 1) / block_size;
}

// Precondition bits of one used block-table entry: a block id within [0, num_blocks).
TRI_HD inline uint32_t check_block(int32_t id, int32_t num_blocks) {
  return (id < 0 || id >= num_blocks) ? TRI_CHECK_BLOCK_RANGE : 0u;
}

// A block id claimed a second time (claimed_before: the id's bit was already set in the claims bitmap when this
// entry set it) -- one pool block holding slots of two sequences.
TRI_HD inline uint32_t check_claim(bool claimed_before) { return claimed_before ? TRI_CHECK_BLOCK_DUP : 0u; }

// Bits of sequence b's checks as one thread of a group of `stride` threads sees them (thread `first`): its length
// and decode position (thread 0 only), then every stride-th used entry of its block-table row (paged; `row` null
// for a contiguous cache).  claim_or(word, bit) sets `bit` in claims word `word` and returns the word's previous
// value (an atomic or on the device); claims null: no duplicate check.
template <typename ClaimOr>
TRI_HD uint32_t check_entries(int32_t length, int32_t t, int32_t capacity, int32_t max_length, const int32_t *row,
                              int32_t block_size, int32_t num_blocks, bool claims, ClaimOr claim_or, int first,
                              int stride) {
  uint32_t bits = first == 0 ? check_sequence(length, t, capacity, max_length) : 0u;
  if (row != nullptr) {
    const int32_t n = check_used_blocks(length, capacity, block_size);
    for (int32_t i = first; i < n; i += stride) {
      const int32_t id = row[i];
      const uint32_t bad = check_block(id, num_blocks);
      bits |= bad;
      if (claims && bad == 0u) {
        const uint32_t bit = 1u << (id & 31);
        bits |= check_claim((claim_or(id >> 5, bit) & bit) != 0u);
      }
    }
  }
  return bits;
}

}  // namespace tri
