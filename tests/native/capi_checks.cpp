// Host-side checks of the C ABI's planning and validation code (include/nsa.h),
// built with the address and undefined-behaviour sanitizers on the host pass
// and no device code: every call here must return before anything is
// launched (device pointers are fake, 16-byte-aligned addresses that
// validation never dereferences). Prints "ok" and exits 0 when every status
// and workspace figure is as documented.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "nsa.h"

static int failures = 0;
#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      fprintf(stderr, "FAIL %s: ", #cond); \
      fprintf(stderr, __VA_ARGS__);        \
      fputc('\n', stderr);                 \
      ++failures;                          \
    }                                      \
  } while (0)

static void *fake(uintptr_t off = 0) { return reinterpret_cast<void *>((uintptr_t)1 << 20 | off); }

static nsa_prefill_desc pdesc(int64_t n, int hq = 28, int hkv = 4, int d = 128, int k = 16, int w = 512,
                              int dtype = NSA_DTYPE_BF16) {
  nsa_prefill_desc ds;
  memset(&ds, 0, sizeof(ds));
  ds.n_tokens = n;
  ds.n_q_heads = hq;
  ds.n_kv_heads = hkv;
  ds.head_dim = d;
  ds.block_size = 64;
  ds.top_k = k;
  ds.window = w;
  ds.scale = 0.f;
  ds.dtype = dtype;
  return ds;
}

static nsa_status prefill_call(const nsa_prefill_desc *ds, const uint8_t *mask, void *ws, size_t ws_bytes,
                               const void *q = fake()) {
  return nsa_prefill(ds, q, fake(), fake(), mask, fake(), fake(), (const float *)fake(), (float *)fake(),
                     nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, nullptr);
}

int main() {
  // status strings and version
  for (int s = 0; s <= 5; ++s) CHECK(nsa_status_string((nsa_status)s) != nullptr, "status %d", s);
  CHECK(strcmp(nsa_status_string(NSA_OK), "ok") == 0, "ok string");
  CHECK(nsa_version() && strlen(nsa_version()) >= 5, "version");

  // workspace sizes over masks: one run, text around it, several runs,
  // text only, no complete block; every figure is 256-byte aligned
  const int64_t ns[] = {1, 40, 64, 65, 1000, 4096 + 512, 36864 + 512};
  for (int64_t n : ns) {
    std::vector<uint8_t> m(n);
    for (int layout = 0; layout < 4; ++layout) {
      for (int64_t i = 0; i < n; ++i) {
        switch (layout) {
          case 0: m[i] = 1; break;
          case 1: m[i] = i >= n / 8 && i < n - n / 8; break;
          case 2: m[i] = (i / 97) % 3 != 1; break;
          default: m[i] = 0; break;
        }
      }
      nsa_prefill_desc ds = pdesc(n);
      size_t bytes = 0;
      CHECK(nsa_prefill_workspace_size(&ds, m.data(), &bytes) == NSA_OK, "ws n %lld layout %d", (long long)n, layout);
      CHECK(bytes % 256 == 0, "ws alignment n %lld", (long long)n);
      // too small a workspace is refused before anything is launched
      if (bytes > 0) CHECK(prefill_call(&ds, m.data(), fake(), bytes - 1) == NSA_ERR_WORKSPACE, "small ws");
      CHECK(prefill_call(&ds, m.data(), nullptr, bytes) == NSA_ERR_WORKSPACE, "null ws");
      CHECK(prefill_call(&ds, m.data(), fake(16), bytes) == NSA_ERR_WORKSPACE, "misaligned ws");
      CHECK(prefill_call(&ds, m.data(), fake(), bytes, fake(2)) == NSA_ERR_INVALID_ARG, "misaligned q");
      CHECK(prefill_call(&ds, m.data(), fake(), bytes, nullptr) == NSA_ERR_INVALID_ARG, "null q");
      int runs = 0;
      for (int64_t i = 0; i < n; ++i) runs += m[i] && (i == 0 || !m[i - 1]);
      size_t bb = 0;
      const nsa_status bst = nsa_prefill_backward_workspace_size(&ds, m.data(), &bb);
      CHECK(bst == (runs > 1 ? NSA_ERR_UNSUPPORTED : NSA_OK), "backward ws status %d runs %d", bst, runs);
    }
  }

  // descriptor validation
  std::vector<uint8_t> m(1024, 1);
  struct Case { nsa_prefill_desc ds; nsa_status want; } cases[] = {
      {pdesc(1024, 28, 5), NSA_ERR_INVALID_ARG},       {pdesc(1024, 28, 4, 128, 0), NSA_ERR_INVALID_ARG},
      {pdesc(1024, 28, 4, 128, 16, 0), NSA_ERR_INVALID_ARG}, {pdesc(0), NSA_ERR_INVALID_ARG},
      {pdesc(1024, 28, 4, 128, 16, 512, 9), NSA_ERR_INVALID_ARG}, {pdesc(1024, 28, 4, 96), NSA_ERR_UNSUPPORTED},
      {pdesc(1024, 36, 4, 64), NSA_ERR_UNSUPPORTED},   {pdesc(1024, 32, 4, 128), NSA_ERR_UNSUPPORTED},
      {pdesc(1024, 28, 4, 128, 65), NSA_ERR_UNSUPPORTED}, {pdesc(1024, 28, 4, 128, 16, 512, 1), NSA_ERR_UNSUPPORTED},
      {pdesc(-5), NSA_ERR_INVALID_ARG},
  };
  for (auto &c : cases) {
    size_t b = 0;
    CHECK(nsa_prefill_workspace_size(&c.ds, m.data(), &b) == c.want, "desc case");
    CHECK(prefill_call(&c.ds, m.data(), fake(), (size_t)1 << 40) == c.want, "desc case call");
  }
  {
    nsa_prefill_desc ds = pdesc(1024);
    ds.block_size = 32;
    size_t b = 0;
    CHECK(nsa_prefill_workspace_size(&ds, m.data(), &b) == NSA_ERR_UNSUPPORTED, "block 32");
    ds = pdesc(1024);
    ds.scale = __builtin_nanf("");
    CHECK(nsa_prefill_workspace_size(&ds, m.data(), &b) == NSA_ERR_INVALID_ARG, "NaN scale");
    CHECK(nsa_prefill_workspace_size(nullptr, m.data(), &b) == NSA_ERR_INVALID_ARG, "null desc");
    CHECK(nsa_prefill_workspace_size(&ds, nullptr, &b) == NSA_ERR_INVALID_ARG, "null mask");
    CHECK(nsa_prefill_workspace_size(&ds, m.data(), nullptr) == NSA_ERR_INVALID_ARG, "null bytes");
  }
  {  // more vision blocks than the kernels take
    const int64_t n = (int64_t)8193 * 64;
    std::vector<uint8_t> big(n, 1);
    nsa_prefill_desc ds = pdesc(n);
    size_t b = 0;
    CHECK(nsa_prefill_workspace_size(&ds, big.data(), &b) == NSA_ERR_UNSUPPORTED, "8193 blocks");
  }

  // varlen: cu_seqlens validation
  {
    std::vector<uint8_t> vm(3000, 1);
    nsa_prefill_desc ds = pdesc(3000);
    const int64_t good[] = {0, 1000, 3000}, bad1[] = {0, 1000, 2999}, bad2[] = {0, 1000, 1000, 3000},
                  bad3[] = {1, 1000, 3000};
    size_t b = 0;
    CHECK(nsa_prefill_varlen_workspace_size(&ds, 2, good, vm.data(), &b) == NSA_OK, "varlen good");
    CHECK(nsa_prefill_varlen_workspace_size(&ds, 2, bad1, vm.data(), &b) == NSA_ERR_INVALID_ARG, "varlen end");
    CHECK(nsa_prefill_varlen_workspace_size(&ds, 3, bad2, vm.data(), &b) == NSA_ERR_INVALID_ARG, "varlen empty seq");
    CHECK(nsa_prefill_varlen_workspace_size(&ds, 2, bad3, vm.data(), &b) == NSA_ERR_INVALID_ARG, "varlen start");
    CHECK(nsa_prefill_varlen_workspace_size(&ds, 0, good, vm.data(), &b) == NSA_ERR_INVALID_ARG, "varlen zero");
  }

  // decode
  {
    nsa_decode_desc dd;
    memset(&dd, 0, sizeof(dd));
    dd.batch = 16; dd.cache_len = 131072; dd.n_q_heads = 28; dd.n_kv_heads = 4; dd.head_dim = 128;
    dd.block_size = 64; dd.top_k = 16; dd.window = 512; dd.dtype = NSA_DTYPE_BF16;
    size_t b = 0;
    CHECK(nsa_decode_workspace_size(&dd, &b) == NSA_OK && b > 0 && b % 256 == 0, "decode ws");
    CHECK(nsa_decode(&dd, fake(), fake(), fake(), fake(), fake(), (const float *)fake(), (float *)fake(), nullptr,
                     nullptr, fake(), b - 1, nullptr) == NSA_ERR_WORKSPACE, "decode small ws");
    CHECK(nsa_decode(&dd, nullptr, fake(), fake(), fake(), fake(), (const float *)fake(), (float *)fake(), nullptr,
                     nullptr, fake(), b, nullptr) == NSA_ERR_INVALID_ARG, "decode null q");
    nsa_decode_desc bad = dd;
    bad.window = dd.cache_len + 1;
    CHECK(nsa_decode_workspace_size(&bad, &b) != NSA_OK, "decode window > L");
    bad = dd;
    bad.cache_capacity = dd.cache_len - 1;
    CHECK(nsa_decode_workspace_size(&bad, &b) != NSA_OK, "decode capacity < L");
    bad = dd;
    bad.batch = 0;
    CHECK(nsa_decode_workspace_size(&bad, &b) != NSA_OK, "decode batch 0");
    CHECK(nsa_cache_append(&dd, nullptr, fake(), fake(), fake(), fake(), fake(), fake(), fake(), nullptr) ==
              NSA_ERR_INVALID_ARG, "append null");
    // the no-allocation variant: same argument checks, and a step beyond its
    // fixed scratch is refused before any HIP call
    CHECK(nsa_decode_noalloc(&dd, nullptr, fake(), fake(), fake(), fake(), (const float *)fake(), (float *)fake(),
                             nullptr, nullptr, nullptr) == NSA_ERR_INVALID_ARG, "noalloc null q");
    CHECK(nsa_decode_noalloc(&dd, fake(), fake(), fake(), fake(), fake(), (const float *)fake(), (float *)fake(),
                             (int32_t *)fake(2), nullptr, nullptr) == NSA_ERR_INVALID_ARG, "noalloc misaligned sel");
    nsa_decode_desc huge = dd;
    huge.batch = 64;
    huge.cache_len = 524288;
    CHECK(nsa_decode_workspace_size(&huge, &b) == NSA_OK && b > NSA_DECODE_NOALLOC_SCRATCH_BYTES, "huge ws");
    CHECK(nsa_decode_noalloc(&huge, fake(), fake(), fake(), fake(), fake(), (const float *)fake(), (float *)fake(),
                             nullptr, nullptr, nullptr) == NSA_ERR_WORKSPACE, "noalloc beyond scratch");
  }

  // gate prologue
  {
    nsa_gate_desc gd;
    memset(&gd, 0, sizeof(gd));
    gd.n_tokens = 131584; gd.d_model = 3584; gd.d_hidden = 1024; gd.n_q_heads = 28;
    gd.activation = NSA_ACT_SILU; gd.dtype = NSA_DTYPE_BF16;
    size_t b = 0;
    CHECK(nsa_gate_workspace_size(&gd, &b) == NSA_OK && b == (size_t)2 * 131584 * 1024, "gate ws");
    nsa_gate_desc bad = gd;
    bad.d_model = 100;
    CHECK(nsa_gate_workspace_size(&bad, &b) == NSA_ERR_UNSUPPORTED, "gate d_model");
    bad = gd;
    bad.activation = 9;
    CHECK(nsa_gate_workspace_size(&bad, &b) == NSA_ERR_INVALID_ARG, "gate activation");
    CHECK(nsa_gate_logits(&gd, fake(), fake(), nullptr, fake(), nullptr, (float *)fake(), fake(), 10, nullptr) ==
              NSA_ERR_WORKSPACE, "gate small ws");
  }

  // dense mode and pooling argument checks
  {
    nsa_prefill_desc ds = pdesc(4096);
    size_t b = 0;
    CHECK(nsa_prefill_dense_workspace_size(&ds, &b) == NSA_OK && b % 256 == 0, "dense ws");
    CHECK(nsa_prefill_dense(&ds, fake(), fake(), fake(), (float *)fake(), nullptr, fake(), b - 1, nullptr) ==
              NSA_ERR_WORKSPACE, "dense small ws");
    CHECK(nsa_cmp_pool(4096, 4, 128, 64, NSA_DTYPE_BF16, fake(), fake(), nullptr, nullptr, nullptr) ==
              NSA_ERR_INVALID_ARG, "pool no output");
    CHECK(nsa_cmp_pool(4096, 4, 96, 64, NSA_DTYPE_BF16, fake(), fake(), fake(), nullptr, nullptr) ==
              NSA_ERR_UNSUPPORTED, "pool d 96");
  }

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
