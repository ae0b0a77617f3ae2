// Decode step: one new query per sequence, at the last slot (L-1) of its
// vision cache, through the same three NSA branches and gates as prefill
// (VideoNSA paper summary page, "Method"). Every one of the L/64 compressed
// blocks is complete and visible; the query's own block (the last) is always
// selected.
//
// One query per sequence makes this GEMV-shaped and HBM-bound (compressed
// cache, selected blocks and window are each read once), so the kernels use
// fp32 vector math and split the work over blocks for occupancy:
//   dec_cmp     per (sequence, KV group, chunk of 128 compressed blocks):
//               scaled logits of the group's query heads, and a softmax
//               partial (max, sum, unnormalised output) of the chunk
//   dec_select  per (sequence, KV group): merged log-sum-exp and o_cmp,
//               group importance scores, exact top-(k-1) + own block
//   dec_fine    per (sequence, KV group, item): one selected block or one
//               64-key slice of the window -> softmax partial
//   dec_combine per (sequence, query head): merge partials, apply gates
#include "../../include/nsa.h"
#include "nsa_kernels.h"
#include "nsa_timing.h"

namespace nsa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kCmpChunk = 128;     // compressed blocks per dec_cmp workgroup
constexpr int kDecMaxBlk = 8192;
constexpr int kDecMaxK = 64;

struct DecPlan {
  int batch = 0, L = 0, hq = 0, hkv = 0, d = 0, G = 0, k = 0, w = 0;
  int n_blk = 0, n_chunk = 0, n_win = 0, n_items = 0;
  float scale = 0.f;
  size_t off_logits = 0, off_cmp = 0, off_ocmp = 0, off_fine = 0, off_sel = 0, off_lse = 0, total = 0;
};

__device__ __forceinline__ float block_reduce_max(float v, float *red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  return r;
}

// ------------------------------------------------------------------ dec_cmp
template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void dec_cmp_kernel(DecodeParams p) {
  __shared__ float qs[G][D];
  __shared__ float ps[G][kCmpChunk];
  __shared__ float red[kDecThreads / 64];
  const int tid = threadIdx.x;
  const int c = blockIdx.x % p.n_chunk;
  const int g = (blockIdx.x / p.n_chunk) % p.hkv;
  const int bi = blockIdx.x / (p.n_chunk * p.hkv);
  const int b0 = c * kCmpChunk;
  const int nb = min(kCmpChunk, p.n_blk - b0);
  for (int i = tid; i < G * D; i += kDecThreads)
    qs[i / D][i % D] = bfbits2f(p.q[((int64_t)bi * p.hq + g * G + i / D) * D + i % D]);
  __syncthreads();
  // logits: one compressed block per thread
  if (tid < nb) {
    const uint16_t *kr = p.kc + (((int64_t)bi * p.n_blk + b0 + tid) * p.hkv + g) * D;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    for (int i = 0; i < D; i += 8) {
      const u16x8 x = *reinterpret_cast<const u16x8 *>(kr + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = bfbits2f(x[e]);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += kv * qs[h][i + e];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float s = acc[h] * p.sl2;
      ps[h][tid] = s;
      p.logits[((int64_t)bi * p.hq + g * G + h) * p.n_blk + b0 + tid] = s;
    }
  }
  __syncthreads();
  // chunk softmax partial per head
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = block_reduce_max(tid < nb ? ps[h][tid] : -INFINITY, red);
    const float e = tid < nb ? exp2f(ps[h][tid] - m[h]) : 0.f;
    __syncthreads();
    if (tid < nb) ps[h][tid] = e;
    l[h] = block_reduce_sum(e, red);
  }
  __syncthreads();
  // unnormalised o over the chunk: thread (dim, half of the blocks)
  const int dim = tid % D, part = tid / D, nparts = kDecThreads / D;
  float o[G];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h] = 0.f;
  for (int b = part; b < nb; b += nparts) {
    const float vv = bfbits2f(p.vc[(((int64_t)bi * p.n_blk + b0 + b) * p.hkv + g) * D + dim]);
#pragma unroll
    for (int h = 0; h < G; ++h) o[h] += ps[h][b] * vv;
  }
  __shared__ float op[kDecThreads / 64 * 64][G];
  if (nparts > 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) op[tid][h] = o[h];
    __syncthreads();
    if (part == 0)
      for (int q = 1; q < nparts; ++q)
#pragma unroll
        for (int h = 0; h < G; ++h) o[h] += op[q * D + dim][h];
  }
  if (part == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float *dst = p.cmp_part + (((int64_t)bi * p.hq + g * G + h) * p.n_chunk + c) * (D + 2);
      dst[2 + dim] = o[h];
      if (dim == 0) { dst[0] = m[h]; dst[1] = l[h]; }
    }
  }
}

// --------------------------------------------------------------- dec_select
template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void dec_select_kernel(DecodeParams p) {
  __shared__ float sc[kDecMaxBlk];
  __shared__ float lse2s[G];
  __shared__ uint32_t hist[256];
  __shared__ float red[kDecThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = blockIdx.x % p.hkv, bi = blockIdx.x / p.hkv;
  // merge the chunk partials: lse and o_cmp per head
  for (int h = 0; h < G; ++h) {
    const int64_t hr = (int64_t)bi * p.hq + g * G + h;
    const float *part = p.cmp_part + hr * p.n_chunk * (D + 2);
    float M = -INFINITY;
    for (int c = 0; c < p.n_chunk; ++c) M = fmaxf(M, part[c * (D + 2)]);
    float L = 0.f;
    for (int c = 0; c < p.n_chunk; ++c) L += part[c * (D + 2) + 1] * exp2f(part[c * (D + 2)] - M);
    if (tid < D) {
      float o = 0.f;
      for (int c = 0; c < p.n_chunk; ++c) o += part[c * (D + 2) + 2 + tid] * exp2f(part[c * (D + 2)] - M);
      p.ocmp[hr * D + tid] = o / L;
    }
    if (tid == 0) {
      lse2s[h] = M + log2f(L);
      if (p.lse) p.lse[hr] = (M + log2f(L)) * (1.0f / kLog2e);
    }
  }
  __syncthreads();
  // group importance of every candidate block (all but the query's own)
  const int n_cand = p.n_blk - 1;
  for (int b = tid; b < n_cand; b += kDecThreads) {
    float s = 0.f;
    for (int h = 0; h < G; ++h)
      s += exp2f(p.logits[((int64_t)bi * p.hq + g * G + h) * p.n_blk + b] - lse2s[h]);
    sc[b] = s;
  }
  __syncthreads();
  int32_t *out = p.sel + ((int64_t)bi * p.hkv + g) * p.topk;
  const int need = p.topk - 1;
  if (n_cand <= need) {
    for (int i = tid; i < p.topk; i += kDecThreads)
      out[i] = i < n_cand ? i : (i == n_cand ? n_cand : -1);
    return;
  }
  if (wv != 0) return;  // wave 0 selects; no barriers follow except the wave's own
  // exact radix select of the need-th largest score (key = bits + 1)
  uint32_t prefix = 0, pmask = 0;
  int rem = need;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int b = lane; b < n_cand; b += 64) {
      const uint32_t key = __float_as_uint(sc[b]) + 1u;
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint32_t cc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cc[i] = hist[255 - 4 * lane - i];
    const uint32_t tot = cc[0] + cc[1] + cc[2] + cc[3];
    uint32_t incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const uint64_t hit = __ballot(incl >= (uint32_t)rem);
    const int lt = __builtin_ctzll(hit);
    uint32_t digit = 0, before = 0;
    if (lane == lt) {
      uint32_t cum = incl - tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum + cc[i] >= (uint32_t)rem) { digit = 255 - 4 * lane - i; before = cum; break; }
        cum += cc[i];
      }
    }
    digit = __shfl(digit, lt);
    before = __shfl(before, lt);
    rem -= (int)before;
    prefix |= digit << shift;
    pmask |= 255u << shift;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  int pos = 0, eq_taken = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n_cand; base += 64) {
    const int b = base + lane;
    const uint32_t key = b < n_cand ? __float_as_uint(sc[b]) + 1u : 0u;
    const bool gt = key > prefix, eq = key == prefix;
    const uint64_t eqb = __ballot(eq);
    const bool eq_take = eq && (eq_taken + __popcll(eqb & below) < rem);
    const bool take = gt || eq_take;
    const uint64_t tb = __ballot(take);
    if (take) out[pos + __popcll(tb & below)] = b;
    pos += __popcll(tb);
    eq_taken += __popcll(__ballot(eq_take));
  }
  if (lane == 0) out[need] = n_cand;  // the query's own block
}

// ----------------------------------------------------------------- dec_fine
template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void dec_fine_kernel(DecodeParams p) {
  __shared__ float qs[G][D];
  __shared__ float ks[kBlk][D + 1];
  __shared__ float ps[G][kBlk];
  __shared__ float red[kDecThreads / 64];
  const int tid = threadIdx.x;
  const int item = blockIdx.x % p.n_items;
  const int g = (blockIdx.x / p.n_items) % p.hkv;
  const int bi = blockIdx.x / (p.n_items * p.hkv);
  // keys of this item: a selected block, or a 64-key slice of the window
  int key0 = 0, nk = 0;
  if (item < p.topk) {
    const int b = p.sel[((int64_t)bi * p.hkv + g) * p.topk + item];
    if (b >= 0) { key0 = b * kBlk; nk = kBlk; }
  } else {
    key0 = p.L - p.window + (item - p.topk) * kBlk;
    nk = min(kBlk, p.L - key0);
  }
  float *dst_base = p.fine_part + ((int64_t)bi * p.hq + g * G) * p.n_items * (D + 2);
  if (nk <= 0) {  // empty item
    for (int i = tid; i < G; i += kDecThreads) {
      float *dst = dst_base + ((int64_t)i * p.n_items + item) * (D + 2);
      dst[0] = -INFINITY;
      dst[1] = 0.f;
    }
    return;
  }
  for (int i = tid; i < G * D; i += kDecThreads)
    qs[i / D][i % D] = bfbits2f(p.q[((int64_t)bi * p.hq + g * G + i / D) * D + i % D]);
  const int64_t row0 = ((int64_t)bi * p.L + key0) * p.hkv + g;
  for (int i = tid; i < nk * D; i += kDecThreads)
    ks[i / D][i % D] = bfbits2f(p.kcache[(row0 + (int64_t)(i / D) * p.hkv) * D + i % D]);
  __syncthreads();
  for (int i = tid; i < G * kBlk; i += kDecThreads) {
    const int h = i / kBlk, j = i % kBlk;
    float s = -INFINITY;
    if (j < nk) {
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc += qs[h][e] * ks[j][e];
      s = acc * p.sl2;
    }
    ps[h][j] = s;
  }
  __syncthreads();
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = block_reduce_max(tid < kBlk ? ps[h][tid] : -INFINITY, red);
    const float e = (tid < kBlk && tid < nk) ? exp2f(ps[h][tid] - m[h]) : 0.f;
    __syncthreads();
    if (tid < kBlk) ps[h][tid] = e;
    l[h] = block_reduce_sum(e, red);
  }
  __syncthreads();
  const int dim = tid % D, part = tid / D, nparts = kDecThreads / D;
  float o[G];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h] = 0.f;
  for (int j = part; j < nk; j += nparts) {
    const float vv = bfbits2f(p.vcache[(row0 + (int64_t)j * p.hkv) * D + dim]);
#pragma unroll
    for (int h = 0; h < G; ++h) o[h] += ps[h][j] * vv;
  }
  __shared__ float op[kDecThreads][G];
  if (nparts > 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) op[tid][h] = o[h];
    __syncthreads();
    if (part == 0)
      for (int q = 1; q < nparts; ++q)
#pragma unroll
        for (int h = 0; h < G; ++h) o[h] += op[q * D + dim][h];
  }
  if (part == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float *dst = dst_base + ((int64_t)h * p.n_items + item) * (D + 2);
      dst[2 + dim] = o[h];
      if (dim == 0) { dst[0] = m[h]; dst[1] = l[h]; }
    }
  }
}

// -------------------------------------------------------------- dec_combine
template <int D>
__global__ __launch_bounds__(D) void dec_combine_kernel(DecodeParams p) {
  const int hr = blockIdx.x;  // bi * hq + h
  const int d = threadIdx.x;
  const float *part = p.fine_part + (int64_t)hr * p.n_items * (D + 2);
  float res[2];
  for (int br = 0; br < 2; ++br) {  // 0: selected blocks, 1: window
    const int i0 = br == 0 ? 0 : p.topk, i1 = br == 0 ? p.topk : p.n_items;
    float M = -INFINITY;
    for (int i = i0; i < i1; ++i) M = fmaxf(M, part[i * (D + 2)]);
    float L = 0.f, o = 0.f;
    for (int i = i0; i < i1; ++i) {
      const float m = part[i * (D + 2)];
      if (m == -INFINITY) continue;
      const float w = exp2f(m - M);
      L += w * part[i * (D + 2) + 1];
      o += w * part[i * (D + 2) + 2 + d];
    }
    res[br] = o / L;
  }
  const float *gl = p.gates + (int64_t)hr * 3;
  p.out[(int64_t)hr * D + d] = sigmoidf_(gl[0]) * p.ocmp[(int64_t)hr * D + d] +
                               sigmoidf_(gl[1]) * res[0] + sigmoidf_(gl[2]) * res[1];
}

template <int D, int G>
hipError_t run_decode(const DecodeParams &p, hipStream_t st) {
  {
    Timed t("dec_cmp", st);
    hipLaunchKernelGGL((dec_cmp_kernel<D, G>), dim3(p.batch * p.hkv * p.n_chunk), dim3(kDecThreads), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    Timed t("dec_select", st);
    hipLaunchKernelGGL((dec_select_kernel<D, G>), dim3(p.batch * p.hkv), dim3(kDecThreads), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    Timed t("dec_fine", st);
    hipLaunchKernelGGL((dec_fine_kernel<D, G>), dim3(p.batch * p.hkv * p.n_items), dim3(kDecThreads), 0, st, p);
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
  if (ds->block_size != kBlk || pl.L % kBlk != 0) return NSA_ERR_UNSUPPORTED;
  if (!decode_supported(pl.d, pl.G)) return NSA_ERR_UNSUPPORTED;
  if (pl.k > kDecMaxK || pl.w > pl.L) return NSA_ERR_UNSUPPORTED;
  pl.n_blk = pl.L / kBlk;
  if (pl.n_blk > kDecMaxBlk) return NSA_ERR_UNSUPPORTED;
  pl.n_chunk = (pl.n_blk + kCmpChunk - 1) / kCmpChunk;
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

nsa_status nsa_decode(const nsa_decode_desc *desc, const void *q, const void *k_cache,
                      const void *v_cache, const void *k_cmp, const void *v_cmp,
                      const float *gate_logits, float *out, int32_t *sel_idx_out, float *lse_out,
                      void *workspace, size_t workspace_bytes, void *stream) {
  DecPlan pl;
  const nsa_status st = plan_decode(desc, pl);
  if (st != NSA_OK) return st;
  if (!q || !k_cache || !v_cache || !k_cmp || !v_cmp || !gate_logits || !out) return NSA_ERR_INVALID_ARG;
  const void *ptrs[] = {q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, out, sel_idx_out, lse_out};
  for (const void *p : ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return NSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return NSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NSA_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
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
  p.n_chunk = pl.n_chunk;
  p.n_items = pl.n_items;
  p.sl2 = pl.scale * kLog2e;
  if (launch_decode(p, pl.d, pl.G, static_cast<hipStream_t>(stream)) != hipSuccess) return NSA_ERR_HIP;
  return NSA_OK;
}

}  // extern "C"
