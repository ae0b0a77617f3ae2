// Per-row top-k selection shared by the prefill and decode paths.
// Top-k block selection (VideoNSA paper summary page, "Method", branch (b):
// keep the top blocks by importance score). Readings: the query's own block
// is always kept and counts toward k; the other k-1 are the highest-scoring
// complete earlier blocks, ties going to the lower block index; the result
// is emitted in ascending block order, -1 padded.
//
// One wave per row. The wave streams the row of group scores once into
// registers (non-negative floats order like their bit patterns). Fast path:
// the (k-1)-th largest of the 64 lane maxima is a lower bound T0 for the
// (k-1)-th largest score (those lane maxima are k-1 distinct scores >= T0),
// so every score of the answer is >= T0; when at most 64 scores reach T0 the
// wave compacts just those (one per lane, ascending index), finds the
// (k-1)-th largest of them, and keeps every larger one plus the lowest-index
// ones equal to it. Both order statistics come from a bitwise search over
// 64 lane values (32 ballot counts, mostly scalar work). Otherwise it finds
// the (k-1)-th largest score exactly by an MSB-first radix select over all
// scores. The chosen indices are emitted in ascending order.
#pragma once
#include "nsa_common.h"

namespace nsa {

// Orders this wave's LDS traffic: the selection runs in one wave, which may
// share its workgroup with waves that have already left.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS operations are done
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The largest T whose bits below LOW are zero with at least `need` lanes
// holding v >= T (need <= lanes with a nonzero v). With LOW = 0 it is the
// need-th largest of the 64 lane values; with LOW > 0 a lower bound of it
// found in 32 - LOW steps. Bits MSB first; each step is one ballot count,
// scalar work that the CU's one scalar unit serves for all its waves.
template <int LOW = 0, int HI = 31>
__device__ __forceinline__ uint32_t kth_largest_lane(uint32_t v, int need, uint32_t t = 0) {
#pragma unroll
  for (int b = HI; b >= LOW; --b) {
    const uint32_t c = t | (1u << b);
    if (__popcll(__ballot(v >= c)) >= need) t = c;
  }
  return t;
}

// The row's candidate keys: key = bits + 1 for candidates (so 0.0f still
// beats padding), 0 otherwise. Every load is issued before the first is
// used (no branch between them, so one wait covers all): lanes past the row
// re-read its last entry, so callers pick NPL close to ceil(f / 64). f >= 1.
template <int NPL>
__device__ __forceinline__ void topk_load_keys(const float *row, int f, uint32_t (&key)[NPL], int lane) {
#pragma unroll
  for (int s = 0; s < NPL; ++s) key[s] = __float_as_uint(row[min(s * 64 + lane, f - 1)]);
#pragma unroll
  for (int s = 0; s < NPL; ++s) key[s] = s * 64 + lane < f ? key[s] + 1u : 0u;
}

// Selects for one row of f candidate scores whose keys topk_load_keys
// produced: out[0..k-2] = the top k-1 block indices ascending (fewer: all of
// them, then -1 padding), out[k-1] = f (the own block). One wave; hist is a
// 256-entry LDS scratch of the calling wave. NPL * 64 >= f.
template <int NPL>
__device__ __forceinline__ void topk_select_keys(const uint32_t (&key)[NPL], int f, int k, int32_t *out,
                                                 uint32_t *hist, int lane) {
  const int need = k - 1;

  if (f <= need) {  // every candidate is kept
    for (int i = lane; i < k; i += 64) out[i] = i < f ? i : (i == f ? f : -1);
    return;
  }

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  {
    uint32_t lm = 0;
#pragma unroll
    for (int s = 0; s < NPL; ++s) lm = max(lm, key[s]);
    // a lower bound of the (k-1)-th largest lane maximum from its top 16
    // bits (bits below are zero): every answer score still reaches it, and
    // at most a few more candidates than with the exact value do
    const uint32_t t0 = kth_largest_lane<16>(lm, need);
    // compact the candidates (ascending index order) into LDS while counting
    // them; past 64 the slow path below takes over
    int c0 = 0;
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
      const bool cand = key[s] >= t0;
      const uint64_t cb = __ballot(cand);
      if (cand) {
        const int q = c0 + __popcll(cb & below);
        if (q < 64) {
          hist[q] = key[s];
          hist[64 + q] = (uint32_t)(s * 64 + lane);
        }
      }
      c0 += __popcll(cb);
    }
    if (c0 <= 64) {
      wave_lds_sync();
      const uint32_t ck = lane < c0 ? hist[lane] : 0u;
      const uint32_t ci = lane < c0 ? hist[64 + lane] : 0xffffffffu;
      // keep the candidates above the need-th largest key, then the
      // lowest-index ones equal to it (candidates sit in ascending index
      // order). The key's top 16 bits first: when exactly `need` candidates
      // reach that prefix they are the answer (the next one lies below it, so
      // no tie crosses the boundary) and the low bits are never searched.
      uint32_t t1 = kth_largest_lane<16>(ck, need);
      bool take;
      if (__popcll(__ballot(ck >= t1)) == need) {  // wave-uniform
        take = ck >= t1;
      } else {
        t1 = kth_largest_lane<0, 15>(ck, need, t1);
        const uint64_t gt = __ballot(ck > t1), eq = __ballot(ck == t1);
        const int rest = need - __popcll(gt);
        take = (ck > t1) || (ck == t1 && __popcll(eq & below) < rest);
      }
      const uint64_t tb = __ballot(take);
      if (take) out[__popcll(tb & below)] = (int32_t)ci;
      if (lane == 0) out[need] = f;  // own block, larger than every candidate
      return;
    }
  }

  uint32_t prefix = 0, pmask = 0;
  int rem = need;  // how many of the elements matching `prefix` are still wanted
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < NPL; ++s)
      if (key[s] != 0u && (key[s] & pmask) == prefix) atomicAdd(&hist[(key[s] >> shift) & 255u], 1u);
    wave_lds_sync();
    // lane L owns digits 255-4L .. 252-4L (descending)
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
    const uint32_t tot = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const uint64_t hit = __ballot(incl >= (uint32_t)rem);
    const int lt = __ffsll((unsigned long long)hit) - 1;
    uint32_t digit = 0, before = 0;
    if (lane == lt) {
      uint32_t cum = incl - tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum + c[i] >= (uint32_t)rem) { digit = 255 - 4 * lane - i; before = cum; break; }
        cum += c[i];
      }
    }
    digit = __shfl(digit, lt);
    before = __shfl(before, lt);
    rem -= (int)before;
    prefix |= digit << shift;
    pmask |= 255u << shift;
    wave_lds_sync();
  }

  // keys > prefix are all kept; of the keys == prefix keep the `rem` lowest indices
  int pos = 0, eq_taken = 0;
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    const bool gt = key[s] > prefix;
    const bool eq = key[s] == prefix;
    const uint64_t eqb = __ballot(eq);
    const bool eq_take = eq && (eq_taken + __popcll(eqb & below) < rem);
    const bool take = gt || eq_take;
    const uint64_t tb = __ballot(take);
    if (take) out[pos + __popcll(tb & below)] = s * 64 + lane;
    pos += __popcll(tb);
    eq_taken += __popcll(__ballot(eq_take));
  }
  if (lane == 0) out[need] = f;  // own block, larger than every candidate
}

// Selects for one row of f candidate scores (row[0..f-1], global or LDS):
// out[0..k-2] = the top k-1 block indices ascending (fewer: all of them,
// then -1 padding), out[k-1] = f (the own block). NPL loads per lane are
// issued whatever f is; a row of at most k - 1 candidates reads nothing.
template <int NPL>
__device__ __forceinline__ void select_topk_row(const float *row, int f, int k, int32_t *out, uint32_t *hist,
                                                int lane) {
  uint32_t key[NPL];
  if (f > k - 1) topk_load_keys<NPL>(row, f, key, lane);  // wave-uniform
  topk_select_keys<NPL>(key, f, k, out, hist, lane);
}

}  // namespace nsa
