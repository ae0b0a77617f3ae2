// Gate prologue: each token's hidden state -> its heads' three branch gate
// logits through a two-layer MLP (paper summary page, "Method"; model card,
// "Model Architecture": learnable per-head gates). Reading: logits =
// W2 . act(W1 . x + b1) + b2, W1 [d_hidden, d_model], W2 [3 Hq, d_hidden],
// row 3 h + c of W2 giving head h's logit for branch c; width and activation
// are the caller's (the pages give neither). The sigmoid is applied where the
// gates are used.
//
// Two matrix-core launches:
//   gate_hidden_kernel  H = act(X W1^T + b1) as fp16 [N, d_hidden]: bf16
//                       operands (exact products), fp32 accumulation, 128 x
//                       128 output tiles of 4 waves (64 x 64 each), both
//                       operand tiles staged through LDS in 64-wide k slices
//                       with 16-byte chunks swizzled per row, double-buffered
//                       through registers;
//   gate_out_kernel     logits = H W2^T + b2: fp16 operands, one wave per 16
//                       tokens and all 3 Hq outputs, operands straight from
//                       global memory (W2 stays in the L2).
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kGT = 128;  // output tile edge of the hidden layer
constexpr int kGK = 64;   // k slice staged per step
constexpr int kGThreads = 256;

__device__ __forceinline__ float act_fn(float h, int act) {
  if (act == 0) return h / (1.f + expf(-h));                       // SiLU
  if (act == 1) {                                                  // GELU (tanh form)
    const float c = 0.7978845608028654f;                           // sqrt(2 / pi)
    return 0.5f * h * (1.f + tanhf(c * (h + 0.044715f * h * h * h)));
  }
  return fmaxf(h, 0.f);                                            // ReLU
}

// Loads this thread's four 16-byte chunks of a [128 rows][64] bf16 slice
// (rows past n_rows read as zeros).
__device__ __forceinline__ void load_slice(const uint16_t *src, int64_t ld, int64_t row0, int64_t n_rows, int k0,
                                           int tid, u16x8 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + kGThreads * j;  // chunk id: row e / 8, chunk e % 8
    const int r = e >> 3, c = e & 7;
    const int64_t row = row0 + r;
    v[j] = row < n_rows ? *reinterpret_cast<const u16x8 *>(src + row * ld + k0 + 8 * c) : zero8();
  }
}

// Stores them swizzled (the K-tile layout of 128-byte rows).
__device__ __forceinline__ void store_slice(uint16_t *dst, int tid, const u16x8 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + kGThreads * j;
    const int r = e >> 3, c = e & 7;
    *reinterpret_cast<u16x8 *>(dst + r * kGK + 8 * PackedTile<kGK>::template swz<2 * kGK>(r, c)) = v[j];
  }
}

__global__ __launch_bounds__(kGThreads) void gate_hidden_kernel(GateParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][kGT * kGK], sx[2][kGT * kGK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_ht = p.d_hidden / kGT;
  const int hid0 = (int)(blockIdx.x % n_ht) * kGT;
  const int64_t tok0 = (int64_t)(blockIdx.x / n_ht) * kGT;
  const int wh = (wv & 1) * 64, wt = (wv >> 1) * 64;  // this wave's 64 x 64 quadrant
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();
  u16x8 rw[4], rx[4];
  load_slice(p.w1, p.d_model, hid0, p.d_hidden, 0, tid, rw);
  load_slice(p.x, p.d_model, tok0, p.n, 0, tid, rx);
  const int n_k = p.d_model / kGK;
  for (int s = 0; s < n_k; ++s) {
    uint16_t *cw = sw[s & 1], *cx = sx[s & 1];
    store_slice(cw, tid, rw);
    store_slice(cx, tid, rx);
    __syncthreads();
    if (s + 1 < n_k) {  // the next slice flies while this one is used
      load_slice(p.w1, p.d_model, hid0, p.d_hidden, (s + 1) * kGK, tid, rw);
      load_slice(p.x, p.d_model, tok0, p.n, (s + 1) * kGK, tid, rx);
    }
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      u16x8 fa[4], fb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) fa[a] = pk_k_frag<kGK>(cw + wh * kGK, a, ks, lane);
#pragma unroll
      for (int b = 0; b < 4; ++b) fb[b] = pk_k_frag<kGK>(cx + wt * kGK, b, ks, lane);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16(fa[a], fb[b], acc[a][b]);
    }
    // the other buffer is overwritten only after the next barrier
  }
  // acc[a][b][i]: hidden hid0 + wh + 16a + 4 (lane / 16) + i, token tok0 + wt + 16b + lane % 16
  const int grp = lane >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t tok = tok0 + wt + 16 * b + (lane & 15);
    if (tok >= p.n) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int h0 = hid0 + wh + 16 * a + 4 * grp;
      u16x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pre = acc[a][b][i] + (p.b1 ? p.b1[h0 + i] : 0.f);
        hv[i] = f2h_bits(act_fn(pre, p.act));
      }
      *reinterpret_cast<u16x4 *>(p.h + tok * p.d_hidden + h0) = hv;
    }
  }
}

// One wave per 16 tokens; 4 waves per workgroup.
constexpr int kOutTiles = 6;  // 96 outputs: 3 Hq <= 96

__global__ __launch_bounds__(256) void gate_out_kernel(GateParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + wv) * 16;
  if (tok0 >= p.n) return;
  const int n_out = 3 * p.hq;
  const int64_t tok = min(tok0 + (lane & 15), p.n - 1);  // rows past n re-read the last one
  const uint16_t *hr = p.h + tok * p.d_hidden + 8 * grp;
  f32x4 acc[kOutTiles];
#pragma unroll
  for (int a = 0; a < kOutTiles; ++a) acc[a] = zero4();
  for (int j0 = 0; j0 < p.d_hidden; j0 += 32) {
    const u16x8 fb = *reinterpret_cast<const u16x8 *>(hr + j0);
#pragma unroll
    for (int a = 0; a < kOutTiles; ++a) {
      const int o = min(16 * a + (lane & 15), n_out - 1);  // rows past 3 Hq repeat the last
      const u16x8 w = *reinterpret_cast<const u16x8 *>(p.w2 + (int64_t)o * p.d_hidden + j0 + 8 * grp);
      u16x8 wf;
#pragma unroll
      for (int e = 0; e < 8; ++e) wf[e] = bf2h_bits(w[e]);
      acc[a] = mfma_f16(wf, fb, acc[a]);
    }
  }
  // acc[a][i]: output 16a + 4 (lane / 16) + i, token tok0 + lane % 16
  const int64_t t = tok0 + (lane & 15);
  if (t >= p.n) return;
#pragma unroll
  for (int a = 0; a < kOutTiles; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = 16 * a + 4 * grp + i;
      if (o < n_out) p.logits[t * n_out + o] = acc[a][i] + (p.b2 ? p.b2[o] : 0.f);
    }
}

}  // namespace

hipError_t launch_gate(const GateParams &p, int layer, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  if (layer == 0) {
    const int64_t n_tt = (p.n + kGT - 1) / kGT;
    hipLaunchKernelGGL(gate_hidden_kernel, dim3((unsigned)(n_tt * (p.d_hidden / kGT))), dim3(kGThreads), 0, st,
                       p);
  } else {
    const int64_t n_wg = (p.n + 63) / 64;
    hipLaunchKernelGGL(gate_out_kernel, dim3((unsigned)n_wg), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace nsa
