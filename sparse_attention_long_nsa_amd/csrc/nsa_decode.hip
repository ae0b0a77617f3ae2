// Decode step: one new query per sequence, at the last slot (L-1) of its
// vision cache, through the same three NSA branches and gates as prefill
// (VideoNSA paper summary page, "Method"). Every one of the L/64 compressed
// blocks is complete and visible; the query's own block (the last) is always
// selected.
//
// One query per sequence makes this HBM-bound: the compressed caches, the
// selected blocks and the window are each read once. All three branches are
// cut into items of 64 keys, one wave each, so thousands of waves stream the
// caches at once:
//   dec_item (phase 0) a chunk of 64 compressed blocks, or a 64-key slice of
//                      the window: scores of the group's heads by matrix-core
//                      products (bf16 in, fp32 out), the chunk's softmax
//                      partial (max, sum, unnormalised output); compressed
//                      chunks also keep their logits
//   dec_select         per (sequence, KV group): merged log-sum-exp and o_cmp,
//                      group importance of every earlier block, exact
//                      top-(k-1) of those scores + the own block
//   dec_item (phase 1) one selected block per item
//   dec_combine        per (sequence, query head): merge the partials of the
//                      selected and window branches, apply the gates
#include <mutex>
#include <type_traits>

#include "../../include/nsa.h"
#include "nsa_kernels.h"
#include "nsa_select.h"
#include "nsa_timing.h"

namespace nsa {

namespace {

// Threads of the selection kernel: every chunk partial, score and o_cmp
// term is loaded in one or two rounds (1,024 threads: 40.9 us per 16 x 128K
// step against 42.7 at 256); rows of more than 2,048 candidates keep 512
// threads, where the 128-register cap of 1,024 would spill.
template <int NPL>
constexpr int dec_select_threads() { return NPL <= 32 ? 1024 : 512; }
constexpr int kDecMaxBlk = 8192;
constexpr int kDecMaxK = 64;

struct DecPlan {
  int batch = 0, L = 0, hq = 0, hkv = 0, d = 0, G = 0, k = 0, w = 0;
  int n_blk = 0, n_chunk = 0, n_win = 0, n_items = 0, cap = 0;
  float scale = 0.f;
  size_t off_logits = 0, off_cmp = 0, off_ocmp = 0, off_fine = 0, off_sel = 0, total = 0;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax_nn(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------------------ dec_item
// One workgroup of four waves per item of up to 64 keys (rows key0 ..
// key0+nk-1 of a [Bt, rows, Hkv, D] cache); wave w takes keys 16w .. 16w+15.
// S^T = K Q^T on the matrix cores: a 16-column tile holds the group's G query
// heads (zero columns past G); lane l owns head l % 16 and keys
// 16w + 4 (l / 16) + i. The item's per-head max and sum combine through LDS.
// The output product runs on the vector units: lane l owns dims
// DL l .. DL l + DL - 1 (DL = D / 64) over the wave's 16 rows, so each row of
// V is one coalesced load across the wave; the four waves' sums meet in LDS.
constexpr int kItemWaves = 4;

template <int D, int G>
__global__ __launch_bounds__(64 * kItemWaves) void dec_item_kernel(DecodeParams p, int phase) {
  constexpr int DS = D / 32, DL = D / 64, KW = kBlk / kItemWaves;
  __shared__ __attribute__((aligned(16))) float pl[kBlk][16];
  __shared__ float red[2][kItemWaves][16];
  __shared__ __attribute__((aligned(16))) float osum[kItemWaves][G][D];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, row = lane & 15, grp = lane >> 4;
  const int n_it = phase == 0 ? p.n_chunk + p.n_win : p.topk;
  const int it = (int)(blockIdx.x % n_it);
  const int g = (int)((blockIdx.x / n_it) % p.hkv);
  const int bi = (int)(blockIdx.x / ((unsigned)n_it * p.hkv));
  const uint16_t *kb = p.kcache, *vb = p.vcache;
  int nrows = p.cap, key0 = 0, nk = 0;  // rows per sequence of the array read
  bool is_cmp = false;
  float *dst;
  int64_t hstride;  // floats between consecutive heads' partials
  if (phase == 0 && it < p.n_chunk) {
    kb = p.kc;
    vb = p.vc;
    nrows = p.cap_blk;
    key0 = it * kBlk;
    nk = min(kBlk, p.n_blk - key0);
    is_cmp = true;
    hstride = (int64_t)p.n_chunk * (D + 2);
    dst = p.cmp_part + ((int64_t)bi * p.hq + g * G) * hstride + (int64_t)it * (D + 2);
  } else {
    int slot;
    if (phase == 0) {
      const int j = it - p.n_chunk;
      key0 = p.L - p.window + j * kBlk;
      nk = min(kBlk, p.L - key0);
      slot = p.topk + j;
    } else {
      const int b = p.sel[((int64_t)bi * p.hkv + g) * p.topk + it];
      if (b >= 0) {
        key0 = b * kBlk;
        nk = min(kBlk, p.L - key0);  // the own block may be partial
      }
      slot = it;
    }
    hstride = (int64_t)p.n_items * (D + 2);
    dst = p.fine_part + ((int64_t)bi * p.hq + g * G) * hstride + (int64_t)slot * (D + 2);
  }
  if (nk <= 0) {  // an unused selection slot (uniform over the workgroup)
    if (tid < G) {
      dst[tid * hstride] = -INFINITY;
      dst[tid * hstride + 1] = 0.f;
    }
    return;
  }
  const int64_t rs = (int64_t)p.hkv * D;  // elements between consecutive rows
  const int64_t r0 = (((int64_t)bi * nrows + key0) * p.hkv + g) * D;
  const uint16_t *kr = kb + r0, *vr = vb + r0;
  const int j0 = KW * wv;  // this wave's first key
  // every load is issued up front; rows past nk re-read the last row (their
  // scores are masked, their probabilities are zero)
  u16x8 kf[DS];
  {
    const int key = min(j0 + row, nk - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kf[ds] = *reinterpret_cast<const u16x8 *>(kr + key * rs + 32 * ds + 8 * grp);
  }
  u16x8 qf[DS];
  {
    const uint16_t *qr = p.q + ((int64_t)bi * p.hq + g * G + (row < G ? row : 0)) * D + 8 * grp;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = row < G ? *reinterpret_cast<const u16x8 *>(qr + 32 * ds) : zero8();
  }
  using VT = typename std::conditional<DL == 2, uint32_t, uint16_t>::type;  // DL bf16 values
  VT vv[KW];
#pragma unroll
  for (int j = 0; j < KW; ++j) vv[j] = *reinterpret_cast<const VT *>(vr + min(j0 + j, nk - 1) * rs + DL * lane);

  f32x4 s = zero4();
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) s = mfma_bf16(kf[ds], qf[ds], s);
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = j0 + 4 * grp + i;
    s[i] = key < nk ? s[i] * p.sl2 : -INFINITY;
    mx = fmax_nn(mx, s[i]);
  }
  if (is_cmp && row < G) {  // logits of the compressed blocks, for the importance scores
    float *lg = p.logits + ((int64_t)bi * p.hq + g * G + row) * p.n_blk + key0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 4 * grp + i;
      if (key < nk) lg[key] = s[i];
    }
  }
  mx = grp_max(mx);
  if (lane < 16) red[0][wv][lane] = mx;
  __syncthreads();
  // key 0 is always valid: the item's max is finite
  const float m = fmax_nn(fmax_nn(red[0][0][row], red[0][1][row]), fmax_nn(red[0][2][row], red[0][3][row]));
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pv = __builtin_amdgcn_exp2f(s[i] - m);
    pl[j0 + 4 * grp + i][row] = pv;
    ls += pv;
  }
  ls = grp_sum(ls);
  if (lane < 16) red[1][wv][lane] = ls;
  __syncthreads();

  float o[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < DL; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    float v[DL];
    if constexpr (DL == 2) {
      v[0] = __uint_as_float(vv[j] << 16);
      v[1] = __uint_as_float(vv[j] & 0xffff0000u);
    } else {
      v[0] = bfbits2f(vv[j]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pj = pl[j0 + j][h];
#pragma unroll
      for (int e = 0; e < DL; ++e) o[h][e] = fmaf(pj, v[e], o[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < DL; ++e) osum[wv][h][DL * lane + e] = o[h][e];
  __syncthreads();
  for (int i = tid; i < G * D; i += 64 * kItemWaves) {
    const int h = i / D, d = i % D;
    dst[h * hstride + 2 + d] = (osum[0][h][d] + osum[1][h][d]) + (osum[2][h][d] + osum[3][h][d]);
  }
  if (tid < G) {
    dst[tid * hstride] = m;
    dst[tid * hstride + 1] = (red[1][0][tid] + red[1][1][tid]) + (red[1][2][tid] + red[1][3][tid]);
  }
}

// --------------------------------------------------------------- dec_select
// Per (sequence, KV group): merge the compressed chunks' partials into each
// head's log-sum-exp and o_cmp, score every earlier block (sum over the
// group's heads of the normalised probability) into LDS, and select the
// top k-1 of them plus the own block (select_topk_row, wave 0).
template <int D, int G, int NPL>
__global__ __launch_bounds__(dec_select_threads<NPL>()) void dec_select_kernel(DecodeParams p) {
  constexpr int kDecThreads = dec_select_threads<NPL>();
  constexpr int NO = kDecThreads - 64;             // threads of waves 1..
  constexpr int OPT = (G * D + NO - 1) / NO;       // o_cmp outputs per thread
  __shared__ float lse2s[G];
  __shared__ float sc[kDecMaxBlk];
  __shared__ uint32_t hist[256];
  __shared__ float wt[G][kDecMaxBlk / kBlk];  // chunk max, then chunk weight
  __shared__ float ls[G][kDecMaxBlk / kBlk];  // chunk sum
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = blockIdx.x % p.hkv, bi = blockIdx.x / p.hkv;
  const int64_t hr0 = (int64_t)bi * p.hq + g * G;
  const int64_t hs = (int64_t)p.n_chunk * (D + 2);  // floats per head of partials
  const float *part = p.cmp_part + hr0 * hs;
  // every chunk's (max, sum) of every head in one round of loads
  for (int i = tid; i < G * p.n_chunk; i += kDecThreads) {
    const int h = i / p.n_chunk, c = i % p.n_chunk;
    wt[h][c] = part[h * hs + (int64_t)c * (D + 2)];
    ls[h][c] = part[h * hs + (int64_t)c * (D + 2) + 1];
  }
  __syncthreads();
  for (int h = wv; h < G; h += kDecThreads / 64) {
    float M = -INFINITY;
    for (int c = lane; c < p.n_chunk; c += 64) M = fmax_nn(M, wt[h][c]);
    M = wave_max(M);
    float L = 0.f;
    for (int c = lane; c < p.n_chunk; c += 64) L += ls[h][c] * exp2f(wt[h][c] - M);
    L = wave_sum(L);
    const float inv = 1.f / L;
    for (int c = lane; c < p.n_chunk; c += 64) wt[h][c] = exp2f(wt[h][c] - M) * inv;
    if (lane == 0) {
      lse2s[h] = M + log2f(L);
      if (p.lse) p.lse[hr0 + h] = (M + log2f(L)) * (1.0f / kLog2e);
    }
  }
  __syncthreads();
  const int n_cand = p.own;  // candidates: every block before the own one
  const float *lg = p.logits + ((int64_t)bi * p.hq + g * G) * p.n_blk;
#pragma unroll 4
  for (int b = tid; b < n_cand; b += kDecThreads) {
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s += exp2f(lg[(int64_t)h * p.n_blk + b] - lse2s[h]);
    sc[b] = s;
  }
  __syncthreads();
  if (wv == 0) {
    select_topk_row<NPL>(sc, n_cand, p.topk, p.sel + ((int64_t)bi * p.hkv + g) * p.topk, hist, lane);
    return;
  }
  {
    // o_cmp, by waves 1.. while wave 0 selects: thread u owns outputs
    // u + NO j (head, dim); the chunk loop is unrolled so each thread keeps
    // many loads in flight
    const int u = tid - 64;
    float acc[OPT];
    int hh[OPT], dd[OPT];
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int i = min(u + NO * j, G * D - 1);
      hh[j] = i / D;
      dd[j] = i % D;
      acc[j] = 0.f;
    }
#pragma unroll 16
    for (int c = 0; c < p.n_chunk; ++c)
#pragma unroll
      for (int j = 0; j < OPT; ++j) acc[j] += wt[hh[j]][c] * part[hh[j] * hs + (int64_t)c * (D + 2) + 2 + dd[j]];
#pragma unroll
    for (int j = 0; j < OPT; ++j)
      if (u + NO * j < G * D) p.ocmp[(hr0 + hh[j]) * D + dd[j]] = acc[j];
  }
}

// -------------------------------------------------------------- dec_combine
template <int D>
__global__ __launch_bounds__(D) void dec_combine_kernel(DecodeParams p) {
  const int hr = blockIdx.x;  // bi * hq + h
  const int d = threadIdx.x;
  const float *part = p.fine_part + (int64_t)hr * p.n_items * (D + 2);
  float res[2];
#pragma unroll
  for (int br = 0; br < 2; ++br) {  // 0: selected blocks, 1: window
    const int i0 = br == 0 ? 0 : p.topk, i1 = br == 0 ? p.topk : p.n_items;
    float M = -INFINITY;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) M = fmax_nn(M, part[(int64_t)i * (D + 2)]);
    float L = 0.f, o = 0.f;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
      const float m = part[(int64_t)i * (D + 2)];
      // an unused selection slot carries only (-inf, 0): its output entries
      // were never written, so their values are selected away, not scaled
      // by zero (0 * a stale NaN is NaN); branch-free, so the loads batch
      const bool used = m != -INFINITY;
      const float w = used ? exp2f(m - M) : 0.f;
      L += w * part[(int64_t)i * (D + 2) + 1];
      const float ov = part[(int64_t)i * (D + 2) + 2 + d];
      o += used ? w * ov : 0.f;
    }
    res[br] = o / L;
  }
  const float *gl = p.gates + (int64_t)hr * 3;
  p.out[(int64_t)hr * D + d] = sigmoidf_(gl[0]) * p.ocmp[(int64_t)hr * D + d] +
                               sigmoidf_(gl[1]) * res[0] + sigmoidf_(gl[2]) * res[1];
}

template <int D, int G>
hipError_t run_decode(const DecodeParams &p, hipStream_t st) {
  const unsigned pairs = (unsigned)p.batch * p.hkv;
  {
    Timed t("dec_item_cmp_win", st);
    hipLaunchKernelGGL((dec_item_kernel<D, G>), dim3(pairs * (p.n_chunk + p.n_win)), dim3(64 * kItemWaves), 0,
                       st, p, 0);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    Timed t("dec_select", st);
    // candidates per lane of the selecting wave: 32 covers caches of up to
    // 2049 blocks (131,136 tokens)
    if (p.own <= 64 * 32)
      hipLaunchKernelGGL((dec_select_kernel<D, G, 32>), dim3(pairs), dim3(dec_select_threads<32>()), 0, st, p);
    else
      hipLaunchKernelGGL((dec_select_kernel<D, G, kDecMaxBlk / 64>), dim3(pairs),
                         dim3(dec_select_threads<kDecMaxBlk / 64>()), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    Timed t("dec_item_sel", st);
    hipLaunchKernelGGL((dec_item_kernel<D, G>), dim3(pairs * p.topk), dim3(64 * kItemWaves), 0, st, p, 1);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    Timed t("dec_combine", st);
    hipLaunchKernelGGL((dec_combine_kernel<D>), dim3(p.batch * p.hq), dim3(D), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

nsa_status plan_decode(const nsa_decode_desc *ds, DecPlan &pl) {
  if (!ds) return NSA_ERR_INVALID_ARG;
  if (ds->batch < 1 || ds->cache_len < 1 || ds->n_q_heads < 1 || ds->n_kv_heads < 1 ||
      ds->head_dim < 1 || ds->block_size < 1 || ds->top_k < 1 || ds->window < 1)
    return NSA_ERR_INVALID_ARG;
  if (ds->n_q_heads % ds->n_kv_heads != 0) return NSA_ERR_INVALID_ARG;
  if (ds->dtype != NSA_DTYPE_BF16 && ds->dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  if (!(ds->scale == ds->scale)) return NSA_ERR_INVALID_ARG;
  pl.batch = ds->batch;
  pl.L = ds->cache_len;
  pl.hq = ds->n_q_heads;
  pl.hkv = ds->n_kv_heads;
  pl.d = ds->head_dim;
  pl.G = pl.hq / pl.hkv;
  pl.k = ds->top_k;
  pl.w = ds->window;
  if (ds->dtype != NSA_DTYPE_BF16) return NSA_ERR_UNSUPPORTED;
  if (ds->block_size != kBlk) return NSA_ERR_UNSUPPORTED;
  if (!decode_supported(pl.d, pl.G)) return NSA_ERR_UNSUPPORTED;
  if (pl.k > kDecMaxK || pl.w > pl.L) return NSA_ERR_UNSUPPORTED;
  pl.cap = ds->cache_capacity > 0 ? ds->cache_capacity : pl.L;
  if (ds->cache_capacity < 0 || pl.cap < pl.L) return NSA_ERR_INVALID_ARG;
  pl.n_blk = pl.L / kBlk;  // complete blocks: the compressed keys
  if (pl.n_blk > kDecMaxBlk) return NSA_ERR_UNSUPPORTED;
  pl.n_chunk = (pl.n_blk + kBlk - 1) / kBlk;
  pl.n_win = (pl.w + kBlk - 1) / kBlk;
  pl.n_items = pl.k + pl.n_win;
  pl.scale = ds->scale > 0.f ? ds->scale : 1.0f / sqrtf((float)pl.d);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = (off + bytes + 255) / 256 * 256; return o; };
  const size_t BH = (size_t)pl.batch * pl.hq;
  pl.off_logits = take(sizeof(float) * BH * pl.n_blk);
  pl.off_cmp = take(sizeof(float) * BH * pl.n_chunk * (pl.d + 2));
  pl.off_ocmp = take(sizeof(float) * BH * pl.d);
  pl.off_fine = take(sizeof(float) * BH * pl.n_items * (pl.d + 2));
  pl.off_sel = take(sizeof(int32_t) * (size_t)pl.batch * pl.hkv * pl.k);
  pl.total = off;
  return NSA_OK;
}

}  // namespace

bool decode_supported(int d, int G) { return (d == 64 || d == 128) && G >= 1 && G <= 8; }

hipError_t launch_decode(const DecodeParams &p, int d, int G, hipStream_t st) {
  if (d == 64) {
    switch (G) {
      case 1: return run_decode<64, 1>(p, st);
      case 2: return run_decode<64, 2>(p, st);
      case 3: return run_decode<64, 3>(p, st);
      case 4: return run_decode<64, 4>(p, st);
      case 5: return run_decode<64, 5>(p, st);
      case 6: return run_decode<64, 6>(p, st);
      case 7: return run_decode<64, 7>(p, st);
      case 8: return run_decode<64, 8>(p, st);
    }
  } else if (d == 128) {
    switch (G) {
      case 1: return run_decode<128, 1>(p, st);
      case 2: return run_decode<128, 2>(p, st);
      case 3: return run_decode<128, 3>(p, st);
      case 4: return run_decode<128, 4>(p, st);
      case 5: return run_decode<128, 5>(p, st);
      case 6: return run_decode<128, 6>(p, st);
      case 7: return run_decode<128, 7>(p, st);
      case 8: return run_decode<128, 8>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nsa

using namespace nsa;

extern "C" {

nsa_status nsa_decode_workspace_size(const nsa_decode_desc *desc, size_t *bytes) {
  if (!bytes) return NSA_ERR_INVALID_ARG;
  DecPlan pl;
  const nsa_status st = plan_decode(desc, pl);
  if (st != NSA_OK) return st;
  *bytes = pl.total;
  return NSA_OK;
}

}  // extern "C"

namespace nsa {
namespace {

// Argument checks shared by nsa_decode and nsa_decode_noalloc (everything
// but the workspace).
nsa_status check_decode_args(const nsa_decode_desc *desc, DecPlan &pl, const void *q, const void *k_cache,
                             const void *v_cache, const void *k_cmp, const void *v_cmp,
                             const float *gate_logits, const float *out, const int32_t *sel_idx_out,
                             const float *lse_out) {
  const nsa_status st = plan_decode(desc, pl);
  if (st != NSA_OK) return st;
  if (!q || !k_cache || !v_cache || !k_cmp || !v_cmp || !gate_logits || !out) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {q, k_cache, v_cache, k_cmp, v_cmp, out};
  for (const void *p : ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return NSA_ERR_INVALID_ARG;
  const void *ptrs4[] = {gate_logits, sel_idx_out, lse_out};  // element-wise accesses
  for (const void *p : ptrs4)
    if (p && (reinterpret_cast<uintptr_t>(p) & 3u) != 0) return NSA_ERR_INVALID_ARG;
  return NSA_OK;
}

// Enqueues a validated decode step with `ws` (pl.total bytes, 256-B aligned)
// as its scratch.
nsa_status enqueue_decode(const DecPlan &pl, const void *q, const void *k_cache, const void *v_cache,
                          const void *k_cmp, const void *v_cmp, const float *gate_logits, float *out,
                          int32_t *sel_idx_out, float *lse_out, char *ws, hipStream_t stream) {
  DecodeParams p{};
  p.q = static_cast<const uint16_t *>(q);
  p.kcache = static_cast<const uint16_t *>(k_cache);
  p.vcache = static_cast<const uint16_t *>(v_cache);
  p.kc = static_cast<const uint16_t *>(k_cmp);
  p.vc = static_cast<const uint16_t *>(v_cmp);
  p.gates = gate_logits;
  p.out = out;
  p.sel = sel_idx_out ? sel_idx_out : reinterpret_cast<int32_t *>(ws + pl.off_sel);
  p.lse = lse_out;
  p.logits = reinterpret_cast<float *>(ws + pl.off_logits);
  p.cmp_part = reinterpret_cast<float *>(ws + pl.off_cmp);
  p.ocmp = reinterpret_cast<float *>(ws + pl.off_ocmp);
  p.fine_part = reinterpret_cast<float *>(ws + pl.off_fine);
  p.batch = pl.batch;
  p.L = pl.L;
  p.hq = pl.hq;
  p.hkv = pl.hkv;
  p.topk = pl.k;
  p.window = pl.w;
  p.n_blk = pl.n_blk;
  p.cap = pl.cap;
  p.cap_blk = pl.cap / kBlk;
  p.own = (pl.L - 1) / kBlk;
  p.n_chunk = pl.n_chunk;
  p.n_win = pl.n_win;
  p.n_items = pl.n_items;
  p.sl2 = pl.scale * kLog2e;
  if (launch_decode(p, pl.d, pl.G, stream) != hipSuccess) return NSA_ERR_HIP;
  return NSA_OK;
}

// Decode scratch that lives in device memory for the life of the process,
// for callers that cannot allocate (nsa_decode_noalloc). Each GPU holds its
// own copy; host code reaches it only through the address
// hipGetSymbolAddress returns on that device, never through the name.
constexpr size_t kNoallocBytes = (size_t)NSA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch, looked up once per device.
nsa_status device_scratch(char **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return NSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char *>(g_scratch_ptr[dev]);
  return NSA_OK;
}

}  // namespace
}  // namespace nsa

extern "C" {

nsa_status nsa_decode(const nsa_decode_desc *desc, const void *q, const void *k_cache,
                      const void *v_cache, const void *k_cmp, const void *v_cmp,
                      const float *gate_logits, float *out, int32_t *sel_idx_out, float *lse_out,
                      void *workspace, size_t workspace_bytes, void *stream) {
  DecPlan pl;
  const nsa_status st = check_decode_args(desc, pl, q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, out,
                                          sel_idx_out, lse_out);
  if (st != NSA_OK) return st;
  if (!workspace || workspace_bytes < pl.total) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NSA_ERR_WORKSPACE;
  return enqueue_decode(pl, q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, out, sel_idx_out, lse_out,
                        static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

nsa_status nsa_decode_noalloc(const nsa_decode_desc *desc, const void *q, const void *k_cache,
                              const void *v_cache, const void *k_cmp, const void *v_cmp,
                              const float *gate_logits, float *out, int32_t *sel_idx_out, float *lse_out,
                              void *stream) {
  DecPlan pl;
  const nsa_status st = check_decode_args(desc, pl, q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, out,
                                          sel_idx_out, lse_out);
  if (st != NSA_OK) return st;
  if (pl.total > kNoallocBytes) return NSA_ERR_WORKSPACE;  // beyond the fixed scratch
  char *ws = nullptr;
  const nsa_status sst = device_scratch(&ws);
  if (sst != NSA_OK) return sst;
  return enqueue_decode(pl, q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, out, sel_idx_out, lse_out, ws,
                        static_cast<hipStream_t>(stream));
}

nsa_status nsa_cache_append(const nsa_decode_desc *desc, const void *k_new, const void *v_new,
                            void *k_cache, void *v_cache, const void *w_cmp_k, const void *w_cmp_v,
                            void *k_cmp, void *v_cmp, void *stream) {
  if (!desc) return NSA_ERR_INVALID_ARG;
  const nsa_decode_desc &ds = *desc;
  if (ds.batch < 1 || ds.cache_len < 1 || ds.n_kv_heads < 1 || ds.head_dim < 1 || ds.cache_capacity < 0)
    return NSA_ERR_INVALID_ARG;
  if (ds.dtype != NSA_DTYPE_BF16 && ds.dtype != NSA_DTYPE_FP32) return NSA_ERR_INVALID_ARG;
  const int64_t L = ds.cache_len;
  const int64_t cap = ds.cache_capacity > 0 ? ds.cache_capacity : L;
  if (cap < L) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {k_new, v_new, k_cache, v_cache, w_cmp_k, w_cmp_v, k_cmp, v_cmp};
  for (const void *ptr : ptrs)
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0) return NSA_ERR_INVALID_ARG;
  if (ds.dtype != NSA_DTYPE_BF16 || ds.block_size != kBlk) return NSA_ERR_UNSUPPORTED;
  if (ds.head_dim != 64 && ds.head_dim != 128) return NSA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int C = ds.n_kv_heads * ds.head_dim;  // columns of one cache row
  {
    Timed tm("cache_append", s);
    if (launch_append_rows(static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
                           static_cast<uint16_t *>(k_cache), static_cast<uint16_t *>(v_cache), ds.batch, C,
                           cap, L - 1, s) != hipSuccess)
      return NSA_ERR_HIP;
  }
  if (L % kBlk == 0) {  // the token completed block L/64 - 1: pool it for every sequence
    const int64_t row0 = L - kBlk, cap_blk = cap / kBlk, b = L / kBlk - 1;
    PoolJob jk{static_cast<const uint16_t *>(k_cache) + row0 * C, w_cmp_k, ds.n_kv_heads, ds.batch,
               static_cast<uint16_t *>(k_cmp) + b * C, nullptr, nullptr, nullptr};
    PoolJob jv{static_cast<const uint16_t *>(v_cache) + row0 * C, w_cmp_v, ds.n_kv_heads, ds.batch,
               static_cast<uint16_t *>(v_cmp) + b * C, nullptr, nullptr, nullptr};
    jk.in_stride = jv.in_stride = cap;       // sequence s's block starts cap rows after s-1's
    jk.out_stride = jv.out_stride = cap_blk;
    Timed tm("cache_pool", s);
    if (launch_cmp_pool(jk, &jv, ds.head_dim, false, s) != hipSuccess) return NSA_ERR_HIP;
  }
  return NSA_OK;
}

}  // extern "C"
