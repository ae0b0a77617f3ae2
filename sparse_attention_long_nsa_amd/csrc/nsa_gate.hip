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
//                       256 (hidden x token) tiles of 4 waves (64 x 128
//                       each), both operands staged through a three-slot LDS
//                       ring of 64-wide k slices by direct global->LDS
//                       copies, 16-byte chunks swizzled per row;
//   gate_out_kernel     logits = H W2^T + b2: fp16 operands, one wave per 64
//                       tokens and all 3 Hq outputs, operands straight from
//                       global memory (W2 stays in the L2).
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

// Hidden layer: a workgroup computes a 128 (hidden) x 256 (token) tile of
// H^T with four waves of 64 x 128; k advances in 64-wide slices through a
// ring of kGS LDS stages filled by direct global->LDS copies, so two slices
// are in flight while one is multiplied.
constexpr int kGH = 128, kGTok = 256, kGK = 64, kGS = 3;
constexpr int kGThreads = 256;
constexpr int kStageW = kGH * kGK, kStage = (kGH + kGTok) * kGK;  // elements
constexpr int kPiecesPerWave = (kGH + kGTok) * kGK / 512 / 4;     // 1 KB copies per wave per stage

__device__ __forceinline__ float act_fn(float h, int act) {
  if (act == 0) return h / (1.f + expf(-h));                       // SiLU
  if (act == 1) {                                                  // GELU (tanh form)
    const float c = 0.7978845608028654f;                           // sqrt(2 / pi)
    return 0.5f * h * (1.f + tanhf(c * (h + 0.044715f * h * h * h)));
  }
  return fmaxf(h, 0.f);                                            // ReLU
}

// Issues this wave's share of one stage: 1 KB pieces of eight 128-byte rows
// (W1 rows hid0.., then token rows tok0..; rows past the last token re-read
// it). Each lane fetches the logical chunk whose swizzled slot it fills, so
// the stage holds the K-tile layout of 128-byte rows.
__device__ __forceinline__ void gate_stage(const GateParams &p, int hid0, int64_t tok0, int k0, uint16_t *stage,
                                           int wv, int lane) {
#pragma unroll
  for (int j = 0; j < kPiecesPerWave; ++j) {
    const int q = wv * kPiecesPerWave + j;  // piece id: rows 8q .. 8q + 7 of the stage
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const uint16_t *src;
    if (r < kGH) {
      src = p.w1 + (int64_t)(hid0 + r) * p.d_model;
    } else {
      const int64_t t = min(tok0 + (r - kGH), p.n - 1);
      src = p.x + t * p.d_model;
    }
    __builtin_amdgcn_global_load_lds(src + k0 + 8 * c, (lds_void *)(stage + 8 * q * kGK), 16, 0, 0);
  }
}

__global__ __launch_bounds__(kGThreads) void gate_hidden_kernel(GateParams p, int n_tt) {
  __shared__ __attribute__((aligned(16))) uint16_t ring[kGS * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_ht = p.d_hidden / kGH;
  // XCD-aware order: ids 8 apart run on one XCD; each XCD walks all hidden
  // tiles of one token tile before the next, so the token rows stay in its L2
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tt = (j / n_ht) * 8 + xcd;
  if (tt >= n_tt) return;
  const int hid0 = (j % n_ht) * kGH;
  const int64_t tok0 = (int64_t)tt * kGTok;
  const int wh = (wv & 1) * 64, wt = (wv >> 1) * 128;  // this wave's 64 x 128 part
  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = zero4();
  const int n_k = p.d_model / kGK;
  gate_stage(p, hid0, tok0, 0, ring, wv, lane);
  if (n_k > 1) gate_stage(p, hid0, tok0, kGK, ring + kStage, wv, lane);
  for (int s = 0; s < n_k; ++s) {
    if (s + 1 < n_k) wait_vm_c<kPiecesPerWave>();  // this wave's copies of slice s have landed
    else wait_vm_c<0>();
    bare_barrier();  // everyone's have; and slot (s - 1) % kGS is no longer read
    if (s + 2 < n_k) gate_stage(p, hid0, tok0, (s + 2) * kGK, ring + ((s + 2) % kGS) * kStage, wv, lane);
    const uint16_t *cw = ring + (s % kGS) * kStage, *cx = cw + kStageW;
    // all 24 fragments of the slice are read up front; the reads of the
    // second half are interleaved with the first half's matrix instructions
    u16x8 fa[2][4], fb[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int a = 0; a < 4; ++a) fa[ks][a] = pk_k_frag<kGK>(cw + wh * kGK, a, ks, lane);
#pragma unroll
      for (int b = 0; b < 8; ++b) fb[ks][b] = pk_k_frag<kGK>(cx + wt * kGK, b, ks, lane);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = mfma_bf16(fa[ks][a], fb[ks][b], acc[a][b]);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // the first half's LDS reads
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read of the second half
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 52, 0);
  }
  // acc[a][b][i]: hidden hid0 + wh + 16a + 4 (lane / 16) + i, token tok0 + wt + 16b + lane % 16
  const int grp = lane >> 4;
  float bias[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[a][i] = p.b1 ? p.b1[hid0 + wh + 16 * a + 4 * grp + i] : 0.f;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int64_t tok = tok0 + wt + 16 * b + (lane & 15);
    if (tok >= p.n) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int h0 = hid0 + wh + 16 * a + 4 * grp;
      u16x4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = f2h_bits(act_fn(acc[a][b][i] + bias[a][i], p.act));
      *reinterpret_cast<u16x4 *>(p.h + tok * p.d_hidden + h0) = hv;
    }
  }
}

// Output layer: one wave per 64 tokens (four 16-token column groups sharing
// each W2 fragment), all 3 Hq <= 96 outputs; W2 is read from the L2 and
// converted to fp16 once per fragment.
constexpr int kOutTiles = 6;   // 96 outputs
constexpr int kOutGroups = 4;  // 16-token groups per wave

__global__ __launch_bounds__(256) void gate_out_kernel(GateParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + wv) * (16 * kOutGroups);
  if (tok0 >= p.n) return;
  const int n_out = 3 * p.hq;
  const uint16_t *hr[kOutGroups];
#pragma unroll
  for (int g = 0; g < kOutGroups; ++g)  // rows past n re-read the last one
    hr[g] = p.h + min(tok0 + 16 * g + (lane & 15), p.n - 1) * p.d_hidden + 8 * grp;
  f32x4 acc[kOutTiles][kOutGroups];
#pragma unroll
  for (int a = 0; a < kOutTiles; ++a)
#pragma unroll
    for (int g = 0; g < kOutGroups; ++g) acc[a][g] = zero4();
  for (int j0 = 0; j0 < p.d_hidden; j0 += 32) {
    u16x8 fb[kOutGroups];
#pragma unroll
    for (int g = 0; g < kOutGroups; ++g) fb[g] = *reinterpret_cast<const u16x8 *>(hr[g] + j0);
#pragma unroll
    for (int a = 0; a < kOutTiles; ++a) {
      const int o = min(16 * a + (lane & 15), n_out - 1);  // rows past 3 Hq repeat the last
      const u16x8 w = *reinterpret_cast<const u16x8 *>(p.w2 + (int64_t)o * p.d_hidden + j0 + 8 * grp);
      u16x8 wf;
#pragma unroll
      for (int e = 0; e < 8; ++e) wf[e] = bf2h_bits(w[e]);
#pragma unroll
      for (int g = 0; g < kOutGroups; ++g) acc[a][g] = mfma_f16(wf, fb[g], acc[a][g]);
    }
  }
  // acc[a][g][i]: output 16a + 4 (lane / 16) + i, token tok0 + 16g + lane % 16
#pragma unroll
  for (int g = 0; g < kOutGroups; ++g) {
    const int64_t t = tok0 + 16 * g + (lane & 15);
    if (t >= p.n) continue;
#pragma unroll
    for (int a = 0; a < kOutTiles; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 16 * a + 4 * grp + i;
        if (o < n_out) p.logits[t * n_out + o] = acc[a][g][i] + (p.b2 ? p.b2[o] : 0.f);
      }
  }
}

}  // namespace

hipError_t launch_gate(const GateParams &p, int layer, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  if (layer == 0) {
    const int64_t n_tt = (p.n + kGTok - 1) / kGTok, n_tt8 = (n_tt + 7) / 8 * 8;
    hipLaunchKernelGGL(gate_hidden_kernel, dim3((unsigned)(n_tt8 * (p.d_hidden / kGH))), dim3(kGThreads), 0, st,
                       p, (int)n_tt);
  } else {
    const int64_t n_wg = (p.n + 4 * 16 * kOutGroups - 1) / (4 * 16 * kOutGroups);
    hipLaunchKernelGGL(gate_out_kernel, dim3((unsigned)n_wg), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace nsa
