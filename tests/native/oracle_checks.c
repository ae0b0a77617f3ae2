/* Runs the fp64 oracle (oracle/nsa_oracle.c, compiled into this program) with
 * the address and undefined-behaviour sanitizers on small layouts that touch
 * every path: text before, between and after vision runs, a partial last
 * block, rows with no complete block, row subsets, injected selections,
 * decode at lengths that are and are not multiples of the block, pooling, and
 * rejected arguments. Any out-of-bounds access, leak or undefined arithmetic
 * aborts the program. Also checks that re-evaluating rows with the
 * oracle's own selection injected reproduces their outputs bit for bit.
 * Prints "ok" and exits 0 when every check holds. */
#include "../../oracle/nsa_oracle.c"

#include <stdio.h>

static int failures = 0;
#define CHECK(cond, msg)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "FAIL %s: %s\n", #cond, msg);       \
      ++failures;                                         \
    }                                                     \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static float urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  const uint64_t x = rng_state * 0x2545f4914f6cdd1dull;
  return (float)((double)(x >> 11) / 4503599627370496.0 - 1.0);
}

static float *fill(int64_t n) {
  float *a = (float *)malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) a[i] = urand();
  return a;
}

static void run_layout(const char *name, const uint8_t *isv, int64_t N, int hq, int hkv, int d, int k, int w) {
  const int B = 64;
  float *q = fill(N * hq * d), *kk = fill(N * hkv * d), *vv = fill(N * hkv * d);
  float *wk = fill((int64_t)d * d), *wv = fill((int64_t)d * d), *gates = fill(N * hq * 3);
  int64_t nv = 0;
  for (int64_t i = 0; i < N; ++i) nv += isv[i];
  const int64_t n_blk = nv / B;
  ora_desc ds = {N, hq, hkv, d, B, k, w, 0.0};
  int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
  for (int64_t i = 0; i < N; ++i) rows[i] = i;
  double *out = (double *)malloc(sizeof(double) * (size_t)(N * hq * d));
  double *lse = (double *)malloc(sizeof(double) * (size_t)(N * hq));
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N * hkv * k));
  double *oc = (double *)malloc(sizeof(double) * (size_t)(N * hq * d));
  double *os = (double *)malloc(sizeof(double) * (size_t)(N * hq * d));
  double *ow = (double *)malloc(sizeof(double) * (size_t)(N * hq * d));
  int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N * 3));
  double *sc = (double *)malloc(sizeof(double) * (size_t)(N * hkv * (n_blk > 0 ? n_blk : 1)));
  double *kc = (double *)malloc(sizeof(double) * (size_t)((n_blk > 0 ? n_blk : 1) * hkv * d));
  double *vc = (double *)malloc(sizeof(double) * (size_t)((n_blk > 0 ? n_blk : 1) * hkv * d));
  int rc = ora_prefill(&ds, q, kk, vv, isv, wk, wv, gates, rows, N, NULL, out, lse, sel, oc, os, ow, cnt, sc, kc, vc);
  CHECK(rc == ORA_OK, name);

  /* vision rows again, as a subset in reverse order, with their own
   * selection injected: identical outputs */
  int64_t nvr = 0;
  int64_t *vr = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nv > 0 ? nv : 1));
  for (int64_t i = N - 1; i >= 0; --i)
    if (isv[i]) vr[nvr++] = i;
  if (nvr > 0) {
    int32_t *inj = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nvr * hkv * k));
    for (int64_t r = 0; r < nvr; ++r) memcpy(inj + r * hkv * k, sel + vr[r] * hkv * k, sizeof(int32_t) * hkv * k);
    double *out2 = (double *)malloc(sizeof(double) * (size_t)(nvr * hq * d));
    rc = ora_prefill(&ds, q, kk, vv, isv, wk, wv, gates, vr, nvr, inj, out2, NULL, NULL, NULL, NULL, NULL, NULL,
                     NULL, NULL, NULL);
    CHECK(rc == ORA_OK, name);
    for (int64_t r = 0; r < nvr; ++r)
      CHECK(memcmp(out2 + r * hq * d, out + vr[r] * hq * d, sizeof(double) * hq * d) == 0, name);
    /* an injected block after the query's own is rejected */
    inj[0] = 100000;
    rc = ora_prefill(&ds, q, kk, vv, isv, wk, wv, gates, vr + nvr - 1, 1, inj, out2, NULL, NULL, NULL, NULL,
                     NULL, NULL, NULL, NULL, NULL);
    CHECK(rc == ORA_EINVAL, name);
    free(inj);
    free(out2);
  }
  /* a row outside the sequence is rejected */
  int64_t badrow = N;
  rc = ora_prefill(&ds, q, kk, vv, isv, wk, wv, gates, &badrow, 1, NULL, out, NULL, NULL, NULL, NULL, NULL, NULL,
                   NULL, NULL, NULL);
  CHECK(rc == ORA_EINVAL, name);
  free(q); free(kk); free(vv); free(wk); free(wv); free(gates); free(rows); free(out); free(lse); free(sel);
  free(oc); free(os); free(ow); free(cnt); free(sc); free(kc); free(vc); free(vr);
}

static void run_decode(int L, int k, int w) {
  const int bt = 3, hq = 6, hkv = 2, d = 16, B = 64;
  const int64_t nb = L / B;
  float *q = fill((int64_t)bt * hq * d), *kcache = fill((int64_t)bt * L * hkv * d), *vcache = fill((int64_t)bt * L * hkv * d);
  float *kcmp = fill((int64_t)bt * (nb > 0 ? nb : 1) * hkv * d), *vcmp = fill((int64_t)bt * (nb > 0 ? nb : 1) * hkv * d);
  float *gates = fill((int64_t)bt * hq * 3);
  ora_decode_desc ds = {bt, L, hq, hkv, d, B, k, w, 0.0};
  double *out = (double *)malloc(sizeof(double) * bt * hq * d), *lse = (double *)malloc(sizeof(double) * bt * hq);
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * bt * hkv * k);
  int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * bt * 3);
  double *sc = (double *)malloc(sizeof(double) * bt * hkv * (nb > 0 ? nb : 1));
  int rc = ora_decode(&ds, q, kcache, vcache, kcmp, vcmp, gates, NULL, out, sel, lse, NULL, NULL, NULL, cnt, sc);
  CHECK(rc == ORA_OK, "decode");
  double *out2 = (double *)malloc(sizeof(double) * bt * hq * d);
  rc = ora_decode(&ds, q, kcache, vcache, kcmp, vcmp, gates, sel, out2, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
  CHECK(rc == ORA_OK && memcmp(out, out2, sizeof(double) * bt * hq * d) == 0, "decode injection");
  free(q); free(kcache); free(vcache); free(kcmp); free(vcmp); free(gates); free(out); free(lse); free(sel);
  free(cnt); free(sc); free(out2);
}

int main(void) {
  enum { N = 420 };
  uint8_t isv[N];
  /* text 20, vision 250, text 30, vision 90, text 30 (several runs) */
  for (int i = 0; i < N; ++i) isv[i] = (i >= 20 && i < 270) || (i >= 300 && i < 390);
  run_layout("several runs", isv, N, 6, 2, 16, 3, 50);
  /* one run, partial last block, window wider than the run */
  for (int i = 0; i < N; ++i) isv[i] = i >= 7;
  run_layout("one run", isv, N, 4, 4, 8, 2, 1000);
  /* no complete block */
  for (int i = 0; i < N; ++i) isv[i] = i >= 380;
  run_layout("no complete block", isv, N, 4, 1, 8, 4, 16);
  /* text only */
  for (int i = 0; i < N; ++i) isv[i] = 0;
  run_layout("text only", isv, N, 2, 1, 8, 1, 1);
  run_decode(256, 3, 64);
  run_decode(300, 5, 300);
  run_decode(63, 2, 10);
  /* pooling, and rejected arguments */
  float *x = fill(200 * 2 * 8), *wm = fill(64);
  double pooled[3 * 2 * 8];
  CHECK(ora_cmp_pool(200, 2, 8, 64, x, wm, pooled) == ORA_OK, "pool");
  CHECK(ora_cmp_pool(200, 0, 8, 64, x, wm, pooled) == ORA_EINVAL, "pool heads");
  ora_desc bad = {N, 6, 4, 16, 64, 3, 50, 0.0}; /* 6 % 4 != 0 */
  int64_t r0 = 0;
  double o[6 * 16];
  CHECK(ora_prefill(&bad, x, x, x, isv, wm, wm, x, &r0, 1, NULL, o, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    NULL, NULL) == ORA_EINVAL, "bad heads");
  free(x); free(wm);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
