// Host-side checks of the selected-block index helpers (nsa_index.h), built
// with the undefined-behaviour and address sanitizers on the host pass: any
// signed overflow or out-of-range row aborts the program. Prints "ok" and
// exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "nsa_index.h"

static int failures = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "FAIL %s: ", #cond);      \
      fprintf(stderr, __VA_ARGS__);             \
      fputc('\n', stderr);                      \
      ++failures;                               \
    }                                           \
  } while (0)

int main() {
  using nsa::sel_block_keys;
  using nsa::sel_key_row;
  const int32_t hostile[] = {INT32_MIN, -5, -2, -1, 1 << 25, (1 << 25) + 3, 1 << 30, INT32_MAX};
  const int ts[] = {0, 1, 62, 63, 64, 65, 127, 128, 4095, 4096, 131071, 524287, (1 << 30) + 7};
  for (int t : ts) {
    const int cur = t / 64;
    // any entry value: keys within [0, 64], rows within [0, t]
    int32_t entries[64];
    int n = 0;
    for (int32_t b : hostile) entries[n++] = b;
    entries[n++] = 0;
    entries[n++] = cur;
    entries[n++] = cur + 1;
    entries[n++] = cur > 0 ? cur - 1 : 0;
    for (int e = 0; e < n; ++e) {
      const int32_t b = entries[e];
      const int nk = sel_block_keys(b, t);
      CHECK(nk >= 0 && nk <= 64, "t %d b %d keys %d", t, b, nk);
      if (b < 0 || b > cur) CHECK(nk == 0, "t %d b %d keys %d (pad or later block)", t, b, nk);
      for (int i : {-3, 0, 1, 31, 63, 64, 1000}) {
        const int r = sel_key_row(b, i, t);
        CHECK(r >= 0 && r <= t, "t %d b %d i %d row %d", t, b, i, r);
      }
    }
    // the own block: keys 64*cur .. t, in order
    CHECK(sel_block_keys(cur, t) == t - 64 * cur + 1, "own block keys at t %d", t);
    for (int i = 0; i < sel_block_keys(cur, t); ++i)
      CHECK(sel_key_row(cur, i, t) == 64 * cur + i, "own block row t %d i %d", t, i);
    // an earlier block: all 64 keys, rows 64 b .. 64 b + 63
    if (cur > 0) {
      const int b = cur - 1;
      CHECK(sel_block_keys(b, t) == 64, "earlier block keys t %d", t);
      for (int i = 0; i < 64; ++i) CHECK(sel_key_row(b, i, t) == 64 * b + i, "earlier row t %d i %d", t, i);
    }
  }
  // a forward-shaped list (k - 1 earlier blocks and the own block) gives the
  // closed-form count (min(k, cur + 1) - 1) * 64 + (t - 64 cur + 1)
  for (int t : {0, 70, 640, 5000, 131071}) {
    for (int k : {1, 2, 4, 16, 32}) {
      const int cur = t / 64;
      int total = 0, taken = 0;
      for (int b = 0; b < cur && taken < k - 1; ++b, ++taken) total += sel_block_keys(b, t);
      total += sel_block_keys(cur, t);
      const int want = ((k < cur + 1 ? k : cur + 1) - 1) * 64 + (t - 64 * cur + 1);
      CHECK(total == want, "t %d k %d total %d want %d", t, k, total, want);
    }
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
