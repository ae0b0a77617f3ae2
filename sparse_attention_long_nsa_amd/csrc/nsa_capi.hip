// C ABI of libnsa.so: argument validation, workspace planning and the launch
// sequence of the VideoNSA attention layer (declarations and contract in
// include/nsa.h).
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/nsa.h"
#include "nsa_kernels.h"
#include "nsa_timing.h"

namespace nsa {
namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxTopK = 64;
constexpr int kMaxBlocks = 8192;  // selection union bitmask / top-k register budget

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct PrefillPlan {
  int64_t N = 0, v0 = 0, v1 = 0, n_vis = 0, n_text = 0;
  bool mapped = false;  // vision tokens in several runs: rows through maps
  int hq = 0, hkv = 0, d = 0, G = 0, k = 0, w = 0;
  int n_blk = 0, n_frames = 0, n_cch = 0;
  bool fp32 = false;
  float scale = 0.f;
  int n_split = 0, chunks_per_split = 0, text_tiles = 0, n_tchunks = 0;
  size_t off_kc = 0, off_vc = 0, off_kcl = 0, off_qh = 0, off_ql = 0, off_q16 = 0, off_k16 = 0,
         off_v16 = 0;
  size_t off_kvc = 0, off_kvt = 0, off_vt = 0, off_lse = 0, off_gs = 0, off_sel = 0, off_po = 0, off_pml = 0;
  size_t off_vmap = 0, off_tmap = 0, off_tnvb = 0, off_means = 0, total = 0;
};

nsa_status plan_prefill(const nsa_prefill_desc *ds, const uint8_t *is_vision, PrefillPlan &pl) {
  if (!ds || !is_vision) return NSA_ERR_INVALID_ARG;
  if (ds->n_tokens < 1 || ds->n_q_heads < 1 || ds->n_kv_heads < 1 || ds->head_dim < 1 ||
      ds->block_size < 1 || ds->top_k < 1 || ds->window < 1)
    return NSA_ERR_INVALID_ARG;
  if (ds->n_q_heads % ds->n_kv_heads != 0) return NSA_ERR_INVALID_ARG;
  if (ds->dtype != NSA_DTYPE_BF16 && ds->dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  if (!(ds->scale == ds->scale)) return NSA_ERR_INVALID_ARG;  // NaN
  pl.N = ds->n_tokens;
  pl.hq = ds->n_q_heads;
  pl.hkv = ds->n_kv_heads;
  pl.d = ds->head_dim;
  pl.G = pl.hq / pl.hkv;
  pl.k = ds->top_k;
  pl.w = ds->window;
  pl.fp32 = ds->dtype == NSA_DTYPE_FP32;
  if (ds->block_size != kBlk) return NSA_ERR_UNSUPPORTED;
  if (!supported_heads(pl.d, pl.G, pl.fp32)) return NSA_ERR_UNSUPPORTED;
  if (pl.k > kMaxTopK) return NSA_ERR_UNSUPPORTED;
  if (pl.N > (int64_t)INT32_MAX / 2) return NSA_ERR_UNSUPPORTED;
  pl.scale = ds->scale > 0.f ? ds->scale : 1.0f / sqrtf((float)pl.d);

  // vision tokens: one run [v0, v1) addressed directly, or several runs
  // addressed through row maps
  int64_t first = -1, last = -1, runs = 0;
  for (int64_t i = 0; i < pl.N; ++i) {
    if (!is_vision[i]) continue;
    if (first < 0) first = i;
    if (i == 0 || !is_vision[i - 1]) ++runs;
    last = i;
    ++pl.n_vis;
  }
  pl.v0 = first < 0 ? 0 : first;
  pl.v1 = first < 0 ? 0 : last + 1;
  pl.mapped = runs > 1;
  pl.n_text = pl.N - pl.n_vis;
  pl.n_blk = (int)(pl.n_vis / kBlk);
  pl.n_frames = (int)((pl.n_vis + kBlk - 1) / kBlk);
  if (pl.n_frames > kMaxBlocks) return NSA_ERR_UNSUPPORTED;

  // text split-K over the packed key chunks (vision blocks, then text
  // rows): enough (tile, group, split) workgroups to fill the chip
  pl.text_tiles = (int)((pl.n_text + kBlk - 1) / kBlk);
  pl.n_tchunks = pl.text_tiles;
  if (pl.n_text > 0) {
    const int64_t want = 1024;
    const int64_t nch = (int64_t)pl.n_frames + pl.n_tchunks;
    int64_t ns = want / ((int64_t)pl.text_tiles * pl.hkv);
    if (ns < 1) ns = 1;
    int64_t cps = (nch + ns - 1) / ns;
    if (cps < 4) cps = 4;
    pl.chunks_per_split = (int)cps;
    pl.n_split = (int)((nch + cps - 1) / cps);
  }

  const size_t H = (size_t)pl.hq, Hk = (size_t)pl.hkv, D = (size_t)pl.d;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  take(sizeof(int32_t));  // offset 0: the status word (nsa_workspace_status)
  pl.off_means = take(sizeof(float) * 2 * (size_t)pl.n_blk * Hk * D);  // block means of keys, values
  pl.off_kc = take(sizeof(uint16_t) * pl.n_blk * Hk * D);
  pl.off_vc = take(sizeof(uint16_t) * pl.n_blk * Hk * D);
  if (pl.fp32) {
    pl.off_kcl = take(sizeof(uint16_t) * pl.n_blk * Hk * D);
    pl.off_qh = take(sizeof(uint16_t) * pl.N * H * D);
    pl.off_ql = take(sizeof(uint16_t) * pl.N * H * D);
    pl.off_q16 = take(sizeof(uint16_t) * pl.N * H * D);
    pl.off_k16 = take(sizeof(uint16_t) * pl.N * Hk * D);
    pl.off_v16 = take(sizeof(uint16_t) * pl.N * Hk * D);
  }
  // packed compressed key/value chunks of the compression branch (fp16 path)
  pl.n_cch = (pl.n_blk + kBlk - 1) / kBlk;
  if (!pl.fp32) pl.off_kvc = take(sizeof(uint16_t) * (size_t)pl.n_cch * Hk * packed_kv_block_elems(pl.d));
  // packed text rows of the text branch: [Hkv][n_tchunks][K tile, V^T tile]
  if (pl.n_text > 0) pl.off_kvt = take(sizeof(uint16_t) * (size_t)pl.n_tchunks * Hk * packed_kv_block_elems(pl.d));
  // packed vision blocks (window, selection and text branches): [Hkv][n_frames][K tile, V^T tile]
  pl.off_vt = take(sizeof(uint16_t) * (size_t)pl.n_frames * Hk * packed_kv_block_elems(pl.d));
  pl.off_lse = take(sizeof(float) * pl.n_vis * H);
  pl.off_gs = take(sizeof(float) * (size_t)frame_off(pl.n_frames, pl.hkv));
  pl.off_sel = take(sizeof(int32_t) * pl.n_vis * Hk * pl.k);
  pl.off_po = take(sizeof(float) * (size_t)pl.n_split * pl.n_text * H * D);
  pl.off_pml = take(sizeof(float2) * (size_t)pl.n_split * pl.n_text * H);
  if (pl.mapped) {
    pl.off_vmap = take(sizeof(int32_t) * pl.n_vis);
    pl.off_tmap = take(sizeof(int32_t) * pl.n_text);
    pl.off_tnvb = take(sizeof(int32_t) * pl.n_text);
  }
  pl.total = off;
  return NSA_OK;
}

// Dense causal GQA over all tokens (Dense-NSA mode).
struct DensePlan {
  int64_t N = 0;
  int hq = 0, hkv = 0, d = 0, G = 0, n_tiles = 0;
  bool fp32 = false;
  float scale = 0.f;
  size_t off_q16 = 0, off_k16 = 0, off_v16 = 0, off_kv = 0, total = 0;
};

nsa_status plan_dense(const nsa_prefill_desc *ds, DensePlan &pl) {
  if (!ds) return NSA_ERR_INVALID_ARG;
  if (ds->n_tokens < 1 || ds->n_q_heads < 1 || ds->n_kv_heads < 1 || ds->head_dim < 1)
    return NSA_ERR_INVALID_ARG;
  if (ds->n_q_heads % ds->n_kv_heads != 0) return NSA_ERR_INVALID_ARG;
  if (ds->dtype != NSA_DTYPE_BF16 && ds->dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  if (!(ds->scale == ds->scale)) return NSA_ERR_INVALID_ARG;  // NaN
  pl.N = ds->n_tokens;
  pl.hq = ds->n_q_heads;
  pl.hkv = ds->n_kv_heads;
  pl.d = ds->head_dim;
  pl.G = pl.hq / pl.hkv;
  pl.fp32 = ds->dtype == NSA_DTYPE_FP32;
  if (!supported_heads(pl.d, pl.G, false)) return NSA_ERR_UNSUPPORTED;
  if (pl.N > (int64_t)INT32_MAX / 2) return NSA_ERR_UNSUPPORTED;
  pl.scale = ds->scale > 0.f ? ds->scale : 1.0f / sqrtf((float)pl.d);
  pl.n_tiles = (int)((pl.N + kBlk - 1) / kBlk);
  const size_t H = (size_t)pl.hq, Hk = (size_t)pl.hkv, D = (size_t)pl.d;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  if (pl.fp32) {
    pl.off_q16 = take(sizeof(uint16_t) * pl.N * H * D);
    pl.off_k16 = take(sizeof(uint16_t) * pl.N * Hk * D);
    pl.off_v16 = take(sizeof(uint16_t) * pl.N * Hk * D);
  }
  pl.off_kv = take(sizeof(uint16_t) * (size_t)pl.n_tiles * Hk * packed_kv_block_elems(pl.d));
  pl.total = off;
  return NSA_OK;
}

template <class T> T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

constexpr int kDefaultSpinLimit = 1 << 22;  // s_sleep(1) rounds, about 0.1 s
std::atomic<int> g_spin_limit{kDefaultSpinLimit};

}  // namespace
}  // namespace nsa

using namespace nsa;

extern "C" {

const char *nsa_status_string(nsa_status s) {
  switch (s) {
    case NSA_OK: return "ok";
    case NSA_ERR_INVALID_ARG: return "invalid argument";
    case NSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case NSA_ERR_WORKSPACE: return "workspace missing or too small";
    case NSA_ERR_HIP: return "HIP launch error";
    case NSA_ERR_KERNEL: return "a kernel's bounded wait gave up: that call's outputs are invalid";
  }
  return "unknown status";
}

const char *nsa_version(void) { return "0.2.0"; }

nsa_status nsa_workspace_status(const void *workspace, void *stream, int32_t *flags) {
  if (!workspace || !flags) return NSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return NSA_ERR_INVALID_ARG;
  int32_t word = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return NSA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return NSA_ERR_HIP;
  *flags = word;
  return word ? NSA_ERR_KERNEL : NSA_OK;
}

nsa_status nsa_debug_set_spin_limit(int32_t rounds) {
  g_spin_limit.store(rounds > 0 ? rounds : kDefaultSpinLimit, std::memory_order_relaxed);
  return NSA_OK;
}

nsa_status nsa_prefill_workspace_size(const nsa_prefill_desc *desc, const uint8_t *is_vision,
                                      size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  PrefillPlan pl;
  const nsa_status st = plan_prefill(desc, is_vision, pl);
  if (st != NSA_OK) return st;
  *bytes = pl.total;
  return NSA_OK;
}

}  // extern "C"

namespace nsa {
namespace {

nsa_status check_prefill_args(const PrefillPlan &pl, const void *q, const void *k, const void *v,
                              const void *w_cmp_k, const void *w_cmp_v, const float *gate_logits,
                              float *out, float *k_cmp_out, float *v_cmp_out, int32_t *sel_idx_out,
                              float *lse_out, void *workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !gate_logits || !out) return NSA_ERR_INVALID_ARG;
  if (pl.n_blk > 0 && (!w_cmp_k || !w_cmp_v)) return NSA_ERR_INVALID_ARG;
  // tensors read or written in 16-byte pieces; gate logits, selected
  // indices and lse are accessed one 4-byte element at a time
  const void *ptrs[] = {q, k, v, w_cmp_k, w_cmp_v, out, k_cmp_out, v_cmp_out};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return NSA_ERR_INVALID_ARG;
  const void *ptrs4[] = {gate_logits, sel_idx_out, lse_out};
  for (const void *p : ptrs4)
    if (p && !aligned4(p)) return NSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return NSA_ERR_WORKSPACE;
  return NSA_OK;
}

// Enqueues the layer for one planned, validated sequence.
nsa_status enqueue_prefill(const PrefillPlan &pl, const void *q, const void *k, const void *v,
                           const uint8_t *is_vision, const void *w_cmp_k, const void *w_cmp_v,
                           const float *gate_logits, float *out, float *k_cmp_out, float *v_cmp_out,
                           int32_t *sel_idx_out, float *lse_out, void *workspace, hipStream_t s,
                           bool clear_status) {
  const int64_t H = pl.hq, Hk = pl.hkv, D = pl.d;
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const uint16_t *kb = static_cast<const uint16_t *>(k);
  const uint16_t *vb = static_cast<const uint16_t *>(v);
  const uint16_t *ql = nullptr;
  uint16_t *kc = at<uint16_t>(workspace, pl.off_kc);
  uint16_t *vc = at<uint16_t>(workspace, pl.off_vc);
  uint16_t *kcl = nullptr;
  hipError_t e = hipSuccess;
#define NSA_CHECK(expr)                      \
  do {                                       \
    e = (expr);                              \
    if (e != hipSuccess) return NSA_ERR_HIP; \
  } while (0)
#define NSA_LAUNCH(name, expr) \
  do {                         \
    Timed tm_(name, s);        \
    NSA_CHECK(expr);           \
  } while (0)

  int32_t *status = at<int32_t>(workspace, 0);
  if (clear_status) NSA_LAUNCH("status_clear", launch_status_clear(status, s));

  // fp32 inputs: block scores from split bf16 operands (q_hi, q_lo), every
  // other product in fp16
  const uint16_t *qc = qb;  // queries of the compression branch
  if (pl.fp32) {
    uint16_t *qh = at<uint16_t>(workspace, pl.off_qh), *qlo = at<uint16_t>(workspace, pl.off_ql);
    uint16_t *q16 = at<uint16_t>(workspace, pl.off_q16), *k16 = at<uint16_t>(workspace, pl.off_k16);
    uint16_t *v16 = at<uint16_t>(workspace, pl.off_v16);
    NSA_LAUNCH("split_q", launch_split_bf16(static_cast<const float *>(q), pl.N * H * D, qh, qlo, s));
    NSA_LAUNCH("to_f16_q", launch_to_f16(static_cast<const float *>(q), pl.N * H * D, q16, s, status));
    NSA_LAUNCH("to_f16_k", launch_to_f16(static_cast<const float *>(k), pl.N * Hk * D, k16, s, status));
    NSA_LAUNCH("to_f16_v", launch_to_f16(static_cast<const float *>(v), pl.N * Hk * D, v16, s, status));
    qc = qh; ql = qlo; qb = q16; kb = k16; vb = v16;
    kcl = at<uint16_t>(workspace, pl.off_kcl);
  }
  const float sl2 = pl.scale * kLog2e;

  // several vision runs: row maps from the mask, one slice per launch
  const int32_t *vmap = nullptr, *tmap = nullptr, *tnvb = nullptr;
  if (pl.mapped) {
    int32_t *vm = at<int32_t>(workspace, pl.off_vmap), *tm = at<int32_t>(workspace, pl.off_tmap);
    int32_t *tb = at<int32_t>(workspace, pl.off_tnvb);
    MaskSlice m;
    m.vis_before = 0;
    for (int64_t base = 0; base < pl.N; base += 32 * kMaskWords) {
      m.base = base;
      m.n = (int)(pl.N - base < 32 * kMaskWords ? pl.N - base : 32 * kMaskWords);
      memset(m.bits, 0, sizeof(m.bits));
      int64_t nv = 0;
      for (int j = 0; j < m.n; ++j)
        if (is_vision[base + j]) { m.bits[j >> 5] |= 1u << (j & 31); ++nv; }
      NSA_LAUNCH("row_maps", launch_row_maps(m, vm, tm, tb, s));
      m.vis_before += nv;
    }
    vmap = vm; tmap = tm; tnvb = tb;
  }

  if (pl.n_vis > 0) {
    float *lse = lse_out ? lse_out : at<float>(workspace, pl.off_lse);
    int32_t *sel = sel_idx_out ? sel_idx_out : at<int32_t>(workspace, pl.off_sel);
    float *gs = at<float>(workspace, pl.off_gs);
    const size_t esz = pl.fp32 ? sizeof(float) : sizeof(uint16_t);
    SelParams sp{qb, kb, vb, at<uint16_t>(workspace, pl.off_vt), sel, gate_logits, out, pl.v0, (int)pl.n_vis, pl.hq, pl.hkv, pl.k,
                 pl.n_frames, sl2, vmap, g_spin_limit.load(std::memory_order_relaxed), status};
    float *means = at<float>(workspace, pl.off_means);
    uint16_t *kvc = (!pl.fp32 && pl.n_cch > 0) ? at<uint16_t>(workspace, pl.off_kvc) : nullptr;
    // bf16: the block means ride in pack_kv's read of the rows, and the maps
    // write the packed compressed chunks themselves
    const int64_t C = (int64_t)pl.hkv * pl.d;
    NSA_LAUNCH("pack_kv", pl.fp32 ? launch_pack_kv(sp, pl.d, true, s)
                                  : launch_pack_kv(sp, pl.d, false, s, means, means + pl.n_blk * C, pl.n_blk));
    if (pl.n_blk > 0) {
      // compressed keys: fp16 (bf16 hi/lo for fp32 inputs); values: fp16
      const int64_t r0 = pl.mapped ? 0 : pl.v0;  // rows through vmap when mapped
      PoolJob jk{static_cast<const char *>(k) + esz * r0 * Hk * D, w_cmp_k, pl.hkv, pl.n_blk,
                 pl.fp32 ? kc : nullptr, kcl, pl.fp32 ? nullptr : kc, k_cmp_out, vmap};
      PoolJob jv{static_cast<const char *>(v) + esz * r0 * Hk * D, w_cmp_v, pl.hkv, pl.n_blk,
                 nullptr, nullptr, vc, v_cmp_out, vmap};
      jk.status = jv.status = status;
      if (pl.fp32) {
        NSA_LAUNCH("cmp_pool", launch_cmp_pool_split(jk, jv, pl.d, true, means, s));
      } else {
        jk.packed = jv.packed = kvc;
        jk.n_cch = jv.n_cch = pl.n_cch;
        jv.packed_v = 1;
        NSA_LAUNCH("cmp_pool", launch_cmp_map(jk, jv, pl.d, false, means, s));
      }
    }
    CmpAttnParams cp{qc, ql, kc, kcl, vc, kvc, pl.n_cch, gate_logits, out, lse, gs, pl.v0,
                     (int)pl.n_vis, pl.hq, pl.hkv, pl.n_frames, sl2, vmap, status};
    NSA_LAUNCH("cmp_attn", launch_cmp_attn(cp, pl.d, pl.G, pl.fp32, s));
    TopkParams tp{gs, sel, (int)pl.n_vis, pl.hkv, pl.k};
    NSA_LAUNCH("blk_score_topk", launch_topk(tp, pl.n_frames, s));
    SwaParams wp{qb, at<uint16_t>(workspace, pl.off_vt), gate_logits, out, pl.v0, (int)pl.n_vis,
                 pl.hq, pl.hkv, pl.w, pl.n_frames, sl2, vmap};
    NSA_LAUNCH("swa_attn", launch_swa_attn(wp, pl.d, pl.G, pl.fp32, s));
    NSA_LAUNCH("sel_attn", launch_sel_attn(sp, pl.d, pl.G, pl.fp32, s));
  }
  if (pl.n_text > 0) {
    uint16_t *kvt = at<uint16_t>(workspace, pl.off_kvt);
    NSA_LAUNCH("pack_text", launch_pack_tiles(kb, vb, 0, (int)pl.n_text, pl.hkv, pl.n_tchunks, kvt,
                                              pl.d, pl.fp32, s, (int)pl.v0, pl.v1 - pl.v0, tmap, status));
    TextParams tp{qb, at<uint16_t>(workspace, pl.off_vt), kvt, at<float>(workspace, pl.off_po),
                  at<float2>(workspace, pl.off_pml), out, pl.v0, pl.v1, pl.N, (int)pl.n_text,
                  pl.hq, pl.hkv, pl.n_split, pl.chunks_per_split, pl.text_tiles,
                  (int)(pl.n_vis > 0 ? pl.n_frames : 0), pl.n_tchunks, sl2, tmap, tnvb};
    NSA_LAUNCH("text_attn", launch_text_attn(tp, pl.d, pl.G, pl.fp32, s));
    NSA_LAUNCH("text_merge", launch_text_merge(tp, pl.d, s));
  }
  return NSA_OK;
}

}  // namespace
}  // namespace nsa

extern "C" {

nsa_status nsa_prefill(const nsa_prefill_desc *desc, const void *q, const void *k, const void *v,
                       const uint8_t *is_vision, const void *w_cmp_k, const void *w_cmp_v,
                       const float *gate_logits, float *out, float *k_cmp_out, float *v_cmp_out,
                       int32_t *sel_idx_out, float *lse_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
  PrefillPlan pl;
  nsa_status st = plan_prefill(desc, is_vision, pl);
  if (st != NSA_OK) return st;
  st = check_prefill_args(pl, q, k, v, w_cmp_k, w_cmp_v, gate_logits, out, k_cmp_out, v_cmp_out,
                          sel_idx_out, lse_out, workspace, workspace_bytes);
  if (st != NSA_OK) return st;
  return enqueue_prefill(pl, q, k, v, is_vision, w_cmp_k, w_cmp_v, gate_logits, out, k_cmp_out,
                         v_cmp_out, sel_idx_out, lse_out, workspace, static_cast<hipStream_t>(stream), true);
}

// Several independent sequences, one after another on the stream.
static nsa_status plan_varlen(const nsa_prefill_desc *desc, int32_t n_seqs, const int64_t *cu,
                              const uint8_t *is_vision, size_t *max_ws) {
  if (!desc || !cu || !is_vision || n_seqs < 1) return NSA_ERR_INVALID_ARG;
  if (cu[0] != 0 || cu[n_seqs] != desc->n_tokens) return NSA_ERR_INVALID_ARG;
  *max_ws = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (cu[i + 1] <= cu[i]) return NSA_ERR_INVALID_ARG;  // every sequence holds a token
    nsa_prefill_desc di = *desc;
    di.n_tokens = cu[i + 1] - cu[i];
    PrefillPlan pl;
    const nsa_status st = plan_prefill(&di, is_vision + cu[i], pl);
    if (st != NSA_OK) return st;
    if (pl.total > *max_ws) *max_ws = pl.total;
  }
  return NSA_OK;
}

nsa_status nsa_prefill_varlen_workspace_size(const nsa_prefill_desc *desc, int32_t n_seqs,
                                             const int64_t *cu_seqlens, const uint8_t *is_vision,
                                             size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  size_t need = 0;
  const nsa_status st = plan_varlen(desc, n_seqs, cu_seqlens, is_vision, &need);
  if (st != NSA_OK) return st;
  *bytes = need;
  return NSA_OK;
}

nsa_status nsa_prefill_varlen(const nsa_prefill_desc *desc, int32_t n_seqs, const int64_t *cu_seqlens,
                              const void *q, const void *k, const void *v, const uint8_t *is_vision,
                              const void *w_cmp_k, const void *w_cmp_v, const float *gate_logits,
                              float *out, float *k_cmp_out, float *v_cmp_out, int32_t *sel_idx_out,
                              float *lse_out, void *workspace, size_t workspace_bytes, void *stream) {
  size_t need = 0;
  nsa_status st = plan_varlen(desc, n_seqs, cu_seqlens, is_vision, &need);
  if (st != NSA_OK) return st;
  // validate every sequence's slice before anything is enqueued
  const size_t esz = desc->dtype == NSA_DTYPE_FP32 ? sizeof(float) : sizeof(uint16_t);
  const int64_t H = desc->n_q_heads, Hk = desc->n_kv_heads, D = desc->head_dim;
  for (int pass = 0; pass < 2; ++pass) {
    int64_t vis0 = 0, blk0 = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int64_t t0 = cu_seqlens[i];
      nsa_prefill_desc di = *desc;
      di.n_tokens = cu_seqlens[i + 1] - t0;
      PrefillPlan pl;
      st = plan_prefill(&di, is_vision + t0, pl);
      if (st != NSA_OK) return st;
      auto off = [](const void *p, int64_t bytes) -> const char * {
        return p ? static_cast<const char *>(p) + bytes : nullptr;
      };
      const void *qi = off(q, t0 * H * D * esz), *ki = off(k, t0 * Hk * D * esz), *vi = off(v, t0 * Hk * D * esz);
      const float *gi = gate_logits ? gate_logits + t0 * H * 3 : nullptr;
      float *oi = out ? out + t0 * H * D : nullptr;
      float *kci = k_cmp_out ? k_cmp_out + blk0 * Hk * D : nullptr;
      float *vci = v_cmp_out ? v_cmp_out + blk0 * Hk * D : nullptr;
      int32_t *si = sel_idx_out ? sel_idx_out + vis0 * Hk * desc->top_k : nullptr;
      float *li = lse_out ? lse_out + vis0 * H : nullptr;
      if (pass == 0) {
        st = check_prefill_args(pl, qi, ki, vi, w_cmp_k, w_cmp_v, gi, oi, kci, vci, si, li, workspace,
                                workspace_bytes);
      } else {
        st = enqueue_prefill(pl, qi, ki, vi, is_vision + t0, w_cmp_k, w_cmp_v, gi, oi, kci, vci, si, li,
                             workspace, static_cast<hipStream_t>(stream), i == 0);
      }
      if (st != NSA_OK) return st;
      vis0 += pl.n_vis;
      blk0 += pl.n_blk;
    }
  }
  return NSA_OK;
}

nsa_status nsa_cmp_pool(int64_t n_rows, int32_t n_heads, int32_t head_dim, int32_t block_size,
                        int32_t dtype, const void *x, const void *w, void *out_bf16,
                        float *out_f32, void *stream) {
  if (n_rows < 0 || n_heads < 1 || !x || !w) return NSA_ERR_INVALID_ARG;
  if (dtype != NSA_DTYPE_BF16 && dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  if (!out_bf16 && !out_f32) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {x, w, out_bf16, out_f32};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return NSA_ERR_INVALID_ARG;
  if (block_size != kBlk || (head_dim != 64 && head_dim != 128)) return NSA_ERR_UNSUPPORTED;
  PoolJob j{x, w, n_heads, n_rows / kBlk, static_cast<uint16_t *>(out_bf16), nullptr, nullptr, out_f32};
  if (launch_cmp_pool(j, nullptr, head_dim, dtype == NSA_DTYPE_FP32, static_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERR_HIP;
  return NSA_OK;
}

// Backward workspace: offsets of every array of BwdParams that lives in it.
struct BwdLayout {
  int n_vtile = 0, n_ptile = 0, n_ctile = 0, mask_words = 0, n_chunk = 0, n_tsplit = 0;
  size_t status = 0, tpart = 0, kc = 0, vc = 0, kbar = 0, vbar = 0, dkc = 0, dvc = 0, kc16 = 0, vc16 = 0, tile_v = 0, tile_p = 0,
         tile_c = 0, vstat = 0, tstat = 0, selmask = 0, selcnt = 0, seloff = 0, selrows = 0, cpart = 0, total = 0;
};

static nsa_status plan_backward(const nsa_prefill_desc *ds, const uint8_t *is_vision, PrefillPlan &pl,
                                BwdLayout &L) {
  const nsa_status st = plan_prefill(ds, is_vision, pl);
  if (st != NSA_OK) return st;
  if (pl.fp32 || pl.mapped) return NSA_ERR_UNSUPPORTED;  // bf16, one vision run
  const size_t nb = (size_t)pl.n_blk * pl.hkv * pl.d;
  const int64_t n_text = pl.N - pl.n_vis;
  L.n_vtile = (int)((pl.n_vis + kBlk - 1) / kBlk);
  L.n_ptile = n_text > 0 ? (int)((pl.N + kBlk - 1) / kBlk) : 0;
  L.n_ctile = (pl.n_blk + kBlk - 1) / kBlk;
  L.mask_words = (int)((pl.n_vis + 31) / 32);
  L.n_chunk = (int)((pl.n_vis + 2047) / 2048);
  L.n_tsplit = n_text > 0 ? 8 : 0;  // text rows' key-tile splits
  const size_t tile = sizeof(uint16_t) * 2 * kBlk * (size_t)pl.d * pl.hkv;  // one tile (K, V rows), every group
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  L.status = take(sizeof(int32_t));  // offset 0: the status word (nsa_workspace_status)
  L.kc = take(sizeof(float) * nb);
  L.vc = take(sizeof(float) * nb);
  L.kbar = take(sizeof(float) * nb);
  L.vbar = take(sizeof(float) * nb);
  L.dkc = take(sizeof(float) * nb);
  L.dvc = take(sizeof(float) * nb);
  L.kc16 = take(sizeof(uint16_t) * nb);
  L.vc16 = take(sizeof(uint16_t) * nb);
  L.tile_v = take(tile * L.n_vtile);
  L.tile_p = take(tile * L.n_ptile);
  L.tile_c = take(tile * L.n_ctile);
  L.vstat = take(sizeof(float) * 6 * (size_t)pl.n_vis * pl.hq);
  L.tstat = take(sizeof(float) * 2 * (size_t)n_text * pl.hq);
  L.selmask = take(sizeof(uint32_t) * (size_t)pl.hkv * L.n_vtile * L.mask_words);
  L.selcnt = take(sizeof(int32_t) * (size_t)pl.hkv * L.n_vtile);
  L.seloff = take(sizeof(int32_t) * ((size_t)pl.hkv * L.n_vtile + 1));
  L.selrows = take(sizeof(int32_t) * (size_t)pl.n_vis * pl.hkv * pl.k);
  L.cpart = take(sizeof(float) * (size_t)L.n_ctile * L.n_chunk * pl.hkv * 2 * kBlk * pl.d);
  L.tpart = take(sizeof(float) * (size_t)L.n_tsplit * n_text * pl.hq * (pl.d + 2));
  L.total = off + kAlign;
  return NSA_OK;
}

nsa_status nsa_prefill_backward_workspace_size(const nsa_prefill_desc *desc, const uint8_t *is_vision,
                                               size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  PrefillPlan pl;
  BwdLayout L;
  const nsa_status st = plan_backward(desc, is_vision, pl, L);
  if (st != NSA_OK) return st;
  *bytes = L.total;
  return NSA_OK;
}

nsa_status nsa_prefill_backward(const nsa_prefill_desc *desc, const void *q, const void *k, const void *v,
                                const uint8_t *is_vision, const void *w_cmp_k, const void *w_cmp_v,
                                const float *gate_logits, const int32_t *sel_idx, const float *dout,
                                float *dq, float *dk, float *dv, float *dw_cmp_k, float *dw_cmp_v,
                                float *dgate, void *workspace, size_t workspace_bytes, void *stream) {
  PrefillPlan pl;
  BwdLayout L;
  const nsa_status st = plan_backward(desc, is_vision, pl, L);
  if (st != NSA_OK) return st;
  const void *req[] = {q, k, v, w_cmp_k, w_cmp_v, gate_logits, dout, dq, dk, dv, dw_cmp_k, dw_cmp_v, dgate};
  for (const void *p : req)
    if (!p || !aligned16(p)) return NSA_ERR_INVALID_ARG;
  if (pl.n_vis > 0 && (!sel_idx || !aligned16(sel_idx))) return NSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return NSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  BwdParams bp{};
  bp.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  bp.q = static_cast<const uint16_t *>(q);
  bp.k = static_cast<const uint16_t *>(k);
  bp.v = static_cast<const uint16_t *>(v);
  bp.wk = static_cast<const uint16_t *>(w_cmp_k);
  bp.wv = static_cast<const uint16_t *>(w_cmp_v);
  bp.gates = gate_logits;
  bp.dout = dout;
  bp.sel = sel_idx;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dgate = dgate;
  bp.dwk = dw_cmp_k;
  bp.dwv = dw_cmp_v;
  bp.kc = reinterpret_cast<float *>(ws + L.kc);
  bp.vc = reinterpret_cast<float *>(ws + L.vc);
  bp.kbar = reinterpret_cast<float *>(ws + L.kbar);
  bp.vbar = reinterpret_cast<float *>(ws + L.vbar);
  bp.dkc = reinterpret_cast<float *>(ws + L.dkc);
  bp.dvc = reinterpret_cast<float *>(ws + L.dvc);
  bp.kc16 = reinterpret_cast<uint16_t *>(ws + L.kc16);
  bp.vc16 = reinterpret_cast<uint16_t *>(ws + L.vc16);
  bp.tile_v = reinterpret_cast<uint16_t *>(ws + L.tile_v);
  bp.tile_p = reinterpret_cast<uint16_t *>(ws + L.tile_p);
  bp.tile_c = reinterpret_cast<uint16_t *>(ws + L.tile_c);
  bp.vstat = reinterpret_cast<float *>(ws + L.vstat);
  bp.tstat = reinterpret_cast<float *>(ws + L.tstat);
  bp.selmask = reinterpret_cast<uint32_t *>(ws + L.selmask);
  bp.selcnt = reinterpret_cast<int32_t *>(ws + L.selcnt);
  bp.seloff = reinterpret_cast<int32_t *>(ws + L.seloff);
  bp.selrows = reinterpret_cast<int32_t *>(ws + L.selrows);
  bp.cpart = reinterpret_cast<float *>(ws + L.cpart);
  bp.tpart = reinterpret_cast<float *>(ws + L.tpart);
  bp.status = reinterpret_cast<int32_t *>(ws + L.status);
  bp.n = pl.N;
  bp.v0 = pl.v0;
  bp.n_vis = pl.n_vis;
  bp.hq = pl.hq;
  bp.hkv = pl.hkv;
  bp.topk = pl.k;
  bp.window = pl.w;
  bp.n_blk = pl.n_blk;
  bp.scale = pl.scale;
  bp.n_vtile = L.n_vtile;
  bp.n_ptile = L.n_ptile;
  bp.n_ctile = L.n_ctile;
  bp.mask_words = L.mask_words;
  bp.n_chunk = L.n_chunk;
  bp.n_tsplit = L.n_tsplit;
  hipError_t e = hipSuccess;
  NSA_LAUNCH("status_clear", launch_status_clear(bp.status, s));
  NSA_LAUNCH("bwd_selclear", launch_backward(bp, pl.d, 0, s));
  NSA_LAUNCH("bwd_pool", launch_backward(bp, pl.d, 1, s));
  NSA_LAUNCH("bwd_pack", launch_backward(bp, pl.d, 2, s));
  NSA_LAUNCH("bwd_sellist", launch_backward(bp, pl.d, 3, s));
  NSA_LAUNCH("bwd_q_vis", launch_backward(bp, pl.d, 7, s));
  NSA_LAUNCH("bwd_q_text", launch_backward(bp, pl.d, 8, s));
  NSA_LAUNCH("bwd_kv", launch_backward(bp, pl.d, 9, s));
  NSA_LAUNCH("bwd_kv_cmp", launch_backward(bp, pl.d, 10, s));
  NSA_LAUNCH("bwd_cmp_sum", launch_backward(bp, pl.d, 11, s));
  NSA_LAUNCH("bwd_cmp_w", launch_backward(bp, pl.d, 12, s));
  NSA_LAUNCH("bwd_cmp_tok", launch_backward(bp, pl.d, 13, s));
  return NSA_OK;
}

static nsa_status plan_gate(const nsa_gate_desc *ds, size_t *bytes) {
  if (!ds) return NSA_ERR_INVALID_ARG;
  if (ds->n_tokens < 1 || ds->d_model < 1 || ds->d_hidden < 1 || ds->n_q_heads < 1) return NSA_ERR_INVALID_ARG;
  if (ds->activation < NSA_ACT_SILU || ds->activation > NSA_ACT_RELU) return NSA_ERR_INVALID_ARG;
  if (ds->dtype != NSA_DTYPE_BF16 && ds->dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  if (ds->dtype != NSA_DTYPE_BF16 || ds->d_model % 64 != 0 || ds->d_hidden % 128 != 0 || 3 * ds->n_q_heads > 96)
    return NSA_ERR_UNSUPPORTED;
  // launch grids: ceil(N / 256) * (d_hidden / 128) and ceil(N / 256) workgroups of 256 threads
  if (ds->n_tokens > ((int64_t)1 << 30) || ds->n_tokens * (int64_t)ds->d_hidden > ((int64_t)1 << 37))
    return NSA_ERR_UNSUPPORTED;
  *bytes = align_up(sizeof(uint16_t) * (size_t)ds->n_tokens * (size_t)ds->d_hidden);
  return NSA_OK;
}

nsa_status nsa_gate_workspace_size(const nsa_gate_desc *desc, size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  size_t need = 0;
  const nsa_status st = plan_gate(desc, &need);
  if (st != NSA_OK) return st;
  *bytes = need;
  return NSA_OK;
}

nsa_status nsa_gate_logits(const nsa_gate_desc *desc, const void *x, const void *w1, const float *b1,
                           const void *w2, const float *b2, float *gate_logits, void *workspace,
                           size_t workspace_bytes, void *stream) {
  size_t need = 0;
  const nsa_status st = plan_gate(desc, &need);
  if (st != NSA_OK) return st;
  if (!x || !w1 || !w2 || !gate_logits) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {x, w1, b1, w2, b2, gate_logits};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return NSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < need) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return NSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GateParams gp{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w1), b1,
                static_cast<const uint16_t *>(w2), b2, static_cast<uint16_t *>(workspace), gate_logits,
                desc->n_tokens, desc->d_model, desc->d_hidden, desc->n_q_heads, desc->activation};
  hipError_t e = hipSuccess;
  NSA_LAUNCH("gate_hidden", launch_gate(gp, 0, s));
  NSA_LAUNCH("gate_out", launch_gate(gp, 1, s));
  return NSA_OK;
}

nsa_status nsa_prefill_dense_workspace_size(const nsa_prefill_desc *desc, size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  DensePlan pl;
  const nsa_status st = plan_dense(desc, pl);
  if (st != NSA_OK) return st;
  *bytes = pl.total;
  return NSA_OK;
}

nsa_status nsa_prefill_dense(const nsa_prefill_desc *desc, const void *q, const void *k,
                             const void *v, float *out, float *lse_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  DensePlan pl;
  const nsa_status st = plan_dense(desc, pl);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !out) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {q, k, v, out, lse_out};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return NSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return NSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t H = pl.hq, Hk = pl.hkv, D = pl.d;
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const uint16_t *kb = static_cast<const uint16_t *>(k);
  const uint16_t *vb = static_cast<const uint16_t *>(v);
  hipError_t e = hipSuccess;
  if (pl.fp32) {  // every product in fp16, as the text rows of nsa_prefill
    uint16_t *q16 = at<uint16_t>(workspace, pl.off_q16), *k16 = at<uint16_t>(workspace, pl.off_k16);
    uint16_t *v16 = at<uint16_t>(workspace, pl.off_v16);
    NSA_LAUNCH("to_f16_q", launch_to_f16(static_cast<const float *>(q), pl.N * H * D, q16, s));
    NSA_LAUNCH("to_f16_k", launch_to_f16(static_cast<const float *>(k), pl.N * Hk * D, k16, s));
    NSA_LAUNCH("to_f16_v", launch_to_f16(static_cast<const float *>(v), pl.N * Hk * D, v16, s));
    qb = q16; kb = k16; vb = v16;
  }
  uint16_t *kv = at<uint16_t>(workspace, pl.off_kv);
  NSA_LAUNCH("pack_dense", launch_pack_tiles(kb, vb, 0, (int)pl.N, pl.hkv, pl.n_tiles, kv, pl.d,
                                             pl.fp32, s));
  DenseParams dp{qb, kv, out, lse_out, pl.N, pl.hq, pl.hkv, pl.n_tiles, pl.scale * kLog2e};
  NSA_LAUNCH("dense_attn", launch_dense_attn(dp, pl.d, pl.G, pl.fp32, s));
  return NSA_OK;
}

}  // extern "C"
