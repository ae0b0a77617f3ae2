// Index arithmetic of selected-block key sets, shared by device code and the
// host-side checks (every function is plain integer code, callable on either
// side).
//
// A vision query t (vision-local index) attends, in its selection branch, to
// the keys j <= t of the blocks chosen for it (VideoNSA paper summary page,
// "Method": the top blocks by importance score are attended token by token;
// the query's own block is causal inside). Selection lists come from the
// caller in the backward pass, so these helpers must stay inside rows 0 .. t
// whatever a list entry holds: entries are clamped into [0, t / 64] BEFORE
// any multiplication, so no product can overflow and no row can fall before
// 0 or after t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

constexpr int kSelBlk = 64;  // selection block (tokens per frame block)

// Keys of list entry b that query t sees: a whole earlier block, the part of
// its own block up to t, nothing for a pad (-1) or a block after t's own.
__host__ __device__ inline int sel_block_keys(int32_t b, int t) {
  if (b < 0 || t < 0 || b > t / kSelBlk) return 0;
  const int n = t - b * kSelBlk + 1;  // b <= t / 64, so b * 64 <= t: no overflow
  return n < kSelBlk ? n : kSelBlk;
}

// Whether list entry b names a block query t may attend (0 .. t / 64).
__host__ __device__ inline bool sel_entry_valid(int32_t b, int t) { return b >= 0 && t >= 0 && b <= t / kSelBlk; }

// Vision row of key i_in_blk (0 .. 63) of list entry b for query t, clamped
// to rows 0 .. t for any entry value (meaningful only for a valid list).
__host__ __device__ inline int sel_key_row(int32_t b, int i_in_blk, int t) {
  if (t < 0) return 0;
  int bc = b < 0 ? 0 : b;
  const int cur = t / kSelBlk;
  if (bc > cur) bc = cur;
  int r = bc * kSelBlk + (i_in_blk < 0 ? 0 : i_in_blk % kSelBlk);
  return r < t ? r : t;
}

}  // namespace nsa
