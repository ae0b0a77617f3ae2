// Token-level branches with a shared key set per query tile: the sliding
// window of vision queries (VideoNSA paper summary page, "Method", branch
// (c)) and dense causal GQA for text queries (same section: text tokens use
// standard GQA).
//
// Layout H: a wave owns 16 queries and all G query heads of one KV group, so
// each K / V^T fragment read from LDS feeds G matrix-core ops.
#include "nsa_kernels.h"

namespace nsa {

namespace {

// ---------------------------------------------------------------- layout H
// Two passes over the keys: pass 1 accumulates each row's (max, sum) to get
// its exact log-sum-exp; pass 2 forms normalised probabilities and runs the
// PV product. No accumulator is ever rescaled, so the G heads' accumulators
// stay in the matrix-core register file.
constexpr int kThreadsH = 256;  // 4 waves x 16 queries

__device__ __forceinline__ void fold4(float &m, float &l, const f32x4 x) {
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  const float mn = fmaxf(m, mx);
  if (mn == -INFINITY) return;
  l = l * exp2f(m - mn) + exp2f(x[0] - mn) + exp2f(x[1] - mn) + exp2f(x[2] - mn) + exp2f(x[3] - mn);
  m = mn;
}

template <int D, int G, bool F16>
__device__ __forceinline__ void qk16(f32x4 (&s)[G], const uint16_t *ks, int kt,
                                     const u16x8 (&qf)[G][D / 32], int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const u16x8 a = k_frag<D>(ks, kt, ds, lane);
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = mfma_qk<F16>(a, qf[h][ds], s[h]);
  }
}

template <int D, int G>
__device__ __forceinline__ void load_q_h(u16x8 (&qf)[G][D / 32], const uint16_t *q, int64_t row0,
                                         bool valid, int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qf[h][ds] = valid ? q_frag_global(q + (row0 + h) * D, ds, lane) : zero8();
}

// Attends this lane's query row (all G heads) over n_chunks staged chunks.
// chunk(c, key0, src, nvalid) gives chunk c's first key index, source row
// pointer and number of rows present; valid(key) masks keys per row.
// Returns o normalised by the row sum and the row lse (log2 units).
template <int D, int G, bool F16, class Chunk, class Valid>
__device__ __forceinline__ void two_pass(f32x4 (&o)[G][D / 16], float (&lse2)[G], uint16_t *ks,
                                         uint16_t *vt, const u16x8 (&qf)[G][D / 32], float sl2,
                                         int n_chunks, int64_t kv_stride, Chunk chunk, Valid valid) {
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4;
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
  for (int c = 0; c < n_chunks; ++c) {
    int key0;
    const uint16_t *ksrc, *vsrc;
    int nvalid;
    chunk(c, key0, ksrc, vsrc, nvalid);
    __syncthreads();
    stage_k<D>(ks, ksrc, kv_stride, nvalid, tid, kThreadsH);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 s[G];
      qk16<D, G, F16>(s, ks, kt, qf, lane);
      const int kb = key0 + 16 * kt + 4 * grp;
      bool ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ok[i] = valid(kb + i);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = ok[i] ? s[h][i] * sl2 : -INFINITY;
        fold4(m[h], l[h], x);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = grp_max(m[h]);
    const float part = (m[h] == -INFINITY) ? 0.f : l[h] * exp2f(m[h] - M);
    const float L = grp_sum(part);
    lse2[h] = (L > 0.f) ? M + log2f(L) : -INFINITY;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[h][dt] = zero4();
  }
  for (int c = 0; c < n_chunks; ++c) {
    int key0;
    const uint16_t *ksrc, *vsrc;
    int nvalid;
    chunk(c, key0, ksrc, vsrc, nvalid);
    __syncthreads();
    stage_k<D>(ks, ksrc, kv_stride, nvalid, tid, kThreadsH);
    stage_vt<D, !F16>(vt, vsrc, kv_stride, nvalid, tid, kThreadsH);
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      f32x4 s[2][G];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kt = 2 * ks2 + kk;
        qk16<D, G, F16>(s[kk], ks, kt, qf, lane);
        const int kb = key0 + 16 * kt + 4 * grp;
        bool ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ok[i] = valid(kb + i);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kk][h][i] = ok[i] ? exp2f(s[kk][h][i] * sl2 - lse2[h]) : 0.f;
      }
      u16x8 pf[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pf[h] = pack_p(s[0][h], s[1][h]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const u16x8 a = v_frag<D>(vt, dt, ks2, lane);
#pragma unroll
        for (int h = 0; h < G; ++h) o[h][dt] = mfma_f16(a, pf[h], o[h][dt]);
      }
    }
  }
}

// ----------------------------------------------------------- sliding window
// Chunks start at the tile's first window key (not 64-aligned): a 64-query
// tile needs keys [t0 - w + 1, t0 + 63], i.e. ceil((w + 63) / 64) chunks.
template <int D, int G, bool F16>
__global__ __launch_bounds__(kThreadsH) void swa_attn_kernel(SwaParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[Tile<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[Tile<D>::vElems];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  const int g = blockIdx.x % p.hkv;
  const int tile = (int)(blockIdx.x / p.hkv);
  const int t0 = tile * kBlk;
  const int t = t0 + wv * 16 + (lane & 15);
  const bool tvalid = t < p.n_vis;
  const int lo = max(0, t0 - p.window + 1);
  const int hi = min(t0 + kBlk - 1, p.n_vis - 1);
  const int64_t kvs = (int64_t)p.hkv * D;
  const int wnd = p.window;

  u16x8 qf[G][D / 32];
  const int64_t qrow = (p.v0 + (tvalid ? t : 0)) * p.hq + (int64_t)g * G;
  load_q_h<D, G>(qf, p.q, qrow, tvalid, lane);
  f32x4 o[G][D / 16];
  float lse2[G];
  const uint16_t *kbase = p.k + (p.v0 * p.hkv + g) * (int64_t)D;
  const uint16_t *vbase = p.v + (p.v0 * p.hkv + g) * (int64_t)D;
  two_pass<D, G, F16>(o, lse2, ks, vt, qf, p.sl2, (hi - lo + kBlk) / kBlk, kvs,
                 [&](int c, int &key0, const uint16_t *&ksrc, const uint16_t *&vsrc, int &nvalid) {
                   key0 = lo + c * kBlk;
                   ksrc = kbase + (int64_t)key0 * kvs;
                   vsrc = vbase + (int64_t)key0 * kvs;
                   nvalid = min(kBlk, hi + 1 - key0);
                 },
                 [&](int j) { return tvalid && j <= t && j > t - wnd; });
  if (tvalid) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float gate = sigmoidf_(p.gates[(qrow + h) * 3 + 2]);
      float *dst = p.out + (qrow + h) * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 *d4 = reinterpret_cast<f32x4 *>(dst + 16 * dt);
        *d4 = *d4 + o[h][dt] * gate;
      }
    }
  }
}

// --------------------------------------------------------------- text rows
__device__ __forceinline__ int64_t text_pos(int r, int64_t v0, int64_t v1) {
  return r < v0 ? (int64_t)r : v1 + (r - v0);
}

// One (64-query tile, KV group, key split) per workgroup; writes the split's
// normalised output and lse for the merge kernel.
template <int D, int G, bool F16>
__global__ __launch_bounds__(kThreadsH) void text_attn_kernel(TextParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[Tile<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[Tile<D>::vElems];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  const int sp = blockIdx.x % p.n_split;
  const int rest = blockIdx.x / p.n_split;
  const int g = rest % p.hkv;
  const int tile = rest / p.hkv;
  const int r = tile * kBlk + wv * 16 + (lane & 15);
  const bool rvalid = r < p.n_text;
  const int pos = rvalid ? (int)text_pos(r, p.v0, p.v1) : -1;
  const int pos_last = (int)text_pos(min(tile * kBlk + kBlk - 1, p.n_text - 1), p.v0, p.v1);
  const int kb = sp * p.split_len;
  const int ke = min(kb + p.split_len, pos_last + 1);
  const int64_t kvs = (int64_t)p.hkv * D;

  u16x8 qf[G][D / 32];
  const int64_t qrow = (int64_t)(rvalid ? pos : 0) * p.hq + (int64_t)g * G;
  load_q_h<D, G>(qf, p.q, qrow, rvalid, lane);
  f32x4 o[G][D / 16];
  float lse2[G];
  const int n_chunks = ke > kb ? (ke - kb + kBlk - 1) / kBlk : 0;
  const uint16_t *kbase = p.k + (int64_t)g * D;
  const uint16_t *vbase = p.v + (int64_t)g * D;
  two_pass<D, G, F16>(o, lse2, ks, vt, qf, p.sl2, n_chunks, kvs,
                 [&](int c, int &key0, const uint16_t *&ksrc, const uint16_t *&vsrc, int &nvalid) {
                   key0 = kb + c * kBlk;
                   ksrc = kbase + (int64_t)key0 * kvs;
                   vsrc = vbase + (int64_t)key0 * kvs;
                   nvalid = min(kBlk, ke - key0);
                 },
                 [&](int j) { return rvalid && j <= pos; });
  if (rvalid) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t pr = ((int64_t)sp * p.n_text + r) * p.hq + g * G + h;
      if (grp == 0) p.part_ml[pr] = make_float2(lse2[h], 0.f);
      float *dst = p.part_o + pr * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = o[h][dt];
    }
  }
}

// Combines the key splits of every (text query, head): each split carries a
// normalised output and its lse (log2 units); weights are exp2(lse_s - LSE).
template <int D>
__global__ __launch_bounds__(D) void text_merge_kernel(TextParams p) {
  const int r = blockIdx.x / p.hq, h = blockIdx.x % p.hq, d = threadIdx.x;
  float M = -INFINITY;
  for (int sp = 0; sp < p.n_split; ++sp)
    M = fmaxf(M, p.part_ml[((int64_t)sp * p.n_text + r) * p.hq + h].x);
  float acc = 0.f, L = 0.f;
  for (int sp = 0; sp < p.n_split; ++sp) {
    const int64_t pr = ((int64_t)sp * p.n_text + r) * p.hq + h;
    const float lse = p.part_ml[pr].x;
    if (lse == -INFINITY) continue;
    const float w = exp2f(lse - M);
    L += w;
    acc += w * p.part_o[pr * D + d];
  }
  p.out[(text_pos(r, p.v0, p.v1) * p.hq + h) * D + d] = acc / L;
}

// ------------------------------------------------------------- launchers
template <int D, int G, bool F16>
hipError_t run_swa(const SwaParams &p, hipStream_t st) {
  const unsigned n = (unsigned)p.n_tiles * (unsigned)p.hkv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((swa_attn_kernel<D, G, F16>), dim3(n), dim3(kThreadsH), 0, st, p);
  return hipGetLastError();
}

template <int D, int G, bool F16>
hipError_t run_text(const TextParams &p, hipStream_t st) {
  const unsigned n = (unsigned)p.n_tiles * (unsigned)p.hkv * (unsigned)p.n_split;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((text_attn_kernel<D, G, F16>), dim3(n), dim3(kThreadsH), 0, st, p);
  return hipGetLastError();
}

#define NSA_SWITCH_G(FN, VF, ...)                               \
  if (d == 64) {                                                \
    switch (G) {                                                \
      case 1: return FN<64, 1, VF>(__VA_ARGS__);                \
      case 2: return FN<64, 2, VF>(__VA_ARGS__);                \
      case 3: return FN<64, 3, VF>(__VA_ARGS__);                \
      case 4: return FN<64, 4, VF>(__VA_ARGS__);                \
      case 5: return FN<64, 5, VF>(__VA_ARGS__);                \
      case 6: return FN<64, 6, VF>(__VA_ARGS__);                \
      case 7: return FN<64, 7, VF>(__VA_ARGS__);                \
      case 8: return FN<64, 8, VF>(__VA_ARGS__);                \
    }                                                           \
  } else if (d == 128) {                                        \
    switch (G) {                                                \
      case 1: return FN<128, 1, VF>(__VA_ARGS__);               \
      case 2: return FN<128, 2, VF>(__VA_ARGS__);               \
      case 3: return FN<128, 3, VF>(__VA_ARGS__);               \
      case 4: return FN<128, 4, VF>(__VA_ARGS__);               \
      case 5: return FN<128, 5, VF>(__VA_ARGS__);               \
      case 6: return FN<128, 6, VF>(__VA_ARGS__);               \
      case 7: return FN<128, 7, VF>(__VA_ARGS__);               \
    }                                                           \
  }                                                             \
  return hipErrorInvalidValue;

}  // namespace

hipError_t launch_swa_attn(const SwaParams &p, int d, int G, bool f16, hipStream_t st) {
  if (f16) { NSA_SWITCH_G(run_swa, true, p, st) }
  NSA_SWITCH_G(run_swa, false, p, st)
}
hipError_t launch_text_merge(const TextParams &p, int d, hipStream_t st) {
  if (p.n_text == 0) return hipSuccess;
  if (d == 64) hipLaunchKernelGGL((text_merge_kernel<64>), dim3((unsigned)(p.n_text * p.hq)), dim3(64), 0, st, p);
  else hipLaunchKernelGGL((text_merge_kernel<128>), dim3((unsigned)(p.n_text * p.hq)), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_text_attn(const TextParams &p, int d, int G, bool f16, hipStream_t st) {
  if (f16) { NSA_SWITCH_G(run_text, true, p, st) }
  NSA_SWITCH_G(run_text, false, p, st)
}
}  // namespace nsa
