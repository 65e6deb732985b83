// Host-only validation a caller can run before a commit: that every cache
// slot a sequence's commit may write belongs to that sequence alone.  The
// accepted rows are promoted into slots that follow the sequence's committed
// boundary, inside storage the sequence owns ("BitMTP: When Multi-Token
// Prediction Meets Low-Bit Large Language Models", Sec. 3.4 M2).  A block
// table that maps one physical slot into two sequences' ranges (or twice into
// one sequence's) makes the commit either race with another sequence's
// commit or overwrite cached history that attention reads.
// Included by mtp_verify.hip only.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "mtp_verify.h"

namespace {

// A conflict is a slot in sequence b's commit range [ctx_b, ctx_b + W) that
// is also in another sequence's range [0, ctx + W), or a second time in b's
// own range [0, ctx_b + W).  Returns the smallest sequence index taking part
// in a conflict, -1 when there is none.  Logical positions
// past the block table, unmapped entries (outside [0, num_pages)) and
// sequences with a negative context are skipped: the device reports those
// as data errors itself.
int32_t first_commit_conflict(int32_t B, int32_t W, int32_t num_pages, int32_t max_pages,
                              const int32_t* block_table, const int32_t* ctx_lens) {
  const long cap = (long)max_pages * MTP_PAGE_SIZE;
  auto slot_of = [&](int32_t b, long t) -> long {
    if (t >= cap) return -1;
    const int32_t page = block_table[(size_t)b * max_pages + t / MTP_PAGE_SIZE];
    if (page < 0 || page >= num_pages) return -1;
    return (long)page * MTP_PAGE_SIZE + t % MTP_PAGE_SIZE;
  };
  // pass 1: the (last) sequence whose commit may write each slot; a slot
  // claimed twice is a conflict of the two claimants
  std::vector<int32_t> writer((size_t)num_pages * MTP_PAGE_SIZE, -1);
  int32_t bad = -1;
  auto note = [&](int32_t b) { bad = (bad < 0 || b < bad) ? b : bad; };
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = ctx_lens[b];
    if (L < 0) continue;
    for (long t = L; t < (long)L + W; ++t) {
      const long s = slot_of(b, t);
      if (s < 0) continue;
      if (writer[s] >= 0) note(writer[s]);  // writer[s] <= b
      writer[s] = b;
    }
  }
  // pass 2: a committed (read) slot that some commit writes
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = ctx_lens[b];
    for (long t = 0; t < (long)L; ++t) {
      const long s = slot_of(b, t);
      if (s < 0 || writer[s] < 0) continue;
      note(writer[s] < b ? writer[s] : b);
    }
  }
  return bad;
}

}  // namespace
