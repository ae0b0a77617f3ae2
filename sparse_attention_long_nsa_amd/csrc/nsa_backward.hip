// Backward pass of the layer for training (model card, "Training Details";
// paper summary, "Method": the model is trained end to end through the NSA
// branches and gates). The block selection is a discrete choice with no
// gradient, so the forward's selected blocks are an input; gradients flow to
// q, k, v (all three branches and the text rows), the gate logits and both
// compression maps.
//
// A first, plain design in fp32 on the vector units (no matrix cores):
//   bwd_zero   clears the accumulated gradients
//   bwd_pool   block means and compressed keys/values, fp32
//   bwd_rows   one wave per (row, query head); per branch three passes over
//              its keys, lane = key for dot products and lane = dimension for
//              sums over keys: (1) max and sum of the exponentials, (2)
//              output o and D = dO . o (and the gate gradient), (3)
//              dS = P (dP - D): dq in registers, dk / dv (or the compressed
//              dK / dV) accumulated with float atomics
//   bwd_cmp_w  dW = sum over blocks of dK_cmp x mean^T, and each block's
//              W^T dK_cmp / 64 added to its 64 tokens' dk (dv likewise)
#include "nsa_kernels.h"
#include "nsa_select.h"

namespace nsa {

namespace {

constexpr int kBwdWaves = 4;

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__global__ void bwd_zero_kernel(float *a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a[i] = 0.f;
}

// One workgroup of D threads per (block, KV group): means of the block's 64
// vision rows and their image under W (y = W x), for keys and values.
template <int D>
__global__ __launch_bounds__(D) void bwd_pool_kernel(BwdParams p) {
  __shared__ float xm[2][D];
  const int b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv, i = threadIdx.x;
  const int64_t r0 = p.v0 + (int64_t)b * kBlk;
  float sk = 0.f, sv = 0.f;
  for (int r = 0; r < kBlk; ++r) {
    const int64_t o = ((r0 + r) * p.hkv + g) * D + i;
    sk += bfbits2f(p.k[o]);
    sv += bfbits2f(p.v[o]);
  }
  sk *= 1.f / kBlk;
  sv *= 1.f / kBlk;
  xm[0][i] = sk;
  xm[1][i] = sv;
  const int64_t ob = ((int64_t)b * p.hkv + g) * D + i;
  p.kbar[ob] = sk;
  p.vbar[ob] = sv;
  __syncthreads();
  float yk = 0.f, yv = 0.f;
  for (int j = 0; j < D; ++j) {
    yk = fmaf(bfbits2f(p.wk[i * D + j]), xm[0][j], yk);
    yv = fmaf(bfbits2f(p.wv[i * D + j]), xm[1][j], yv);
  }
  p.kc[ob] = yk;
  p.vc[ob] = yv;
}

// A branch's key set for one row: n keys; key i is row `row(i)` of either
// the token arrays (bf16, gradients into dk / dv) or the compressed arrays
// (fp32, gradients into dkc / dvc).
struct KeySet {
  int kind;      // 0 compressed blocks 0..n-1, 1 contiguous token rows, 2 selected blocks
  int n;         // number of keys
  int64_t row0;  // kind 1: first token row
  const int32_t *blocks;  // kind 2: selected blocks (ascending, -1 pads)
  int nsel, t;   // kind 2: entries, vision index of the query (keys j <= t)
};

// Token row of key i of a selected-block set (vision keys j <= t of the
// selected blocks, in block order): walks the block list.
__device__ __forceinline__ int64_t sel_row(const BwdParams &p, const KeySet &ks, int i) {
  for (int e = 0; e < ks.nsel; ++e) {
    const int b = ks.blocks[e];
    if (b < 0) continue;
    const int len = min(kBlk, ks.t - b * kBlk + 1);
    if (len <= 0) continue;
    if (i < len) return p.v0 + (int64_t)b * kBlk + i;
    i -= len;
  }
  return -1;
}

template <int D>
struct KeyRef {
  const uint16_t *kb = nullptr, *vb = nullptr;  // token rows (bf16)
  const float *kf = nullptr, *vf = nullptr;     // compressed rows (fp32)
  float *dk = nullptr, *dv = nullptr;
  __device__ __forceinline__ float k(int j) const { return kb ? bfbits2f(kb[j]) : kf[j]; }
  __device__ __forceinline__ float v(int j) const { return vb ? bfbits2f(vb[j]) : vf[j]; }
};

template <int D>
__device__ __forceinline__ KeyRef<D> key_ref(const BwdParams &p, const KeySet &ks, int i, int g) {
  KeyRef<D> r;
  if (ks.kind == 0) {
    const int64_t o = ((int64_t)i * p.hkv + g) * D;
    r.kf = p.kc + o;
    r.vf = p.vc + o;
    r.dk = p.dkc + o;
    r.dv = p.dvc + o;
  } else {
    const int64_t row = ks.kind == 1 ? ks.row0 + i : sel_row(p, ks, i);
    const int64_t o = (row * p.hkv + g) * D;
    r.kb = p.k + o;
    r.vb = p.v + o;
    r.dk = p.dk + o;
    r.dv = p.dv + o;
  }
  return r;
}

// One branch for one (row, head) held by one wave. q and dO (already scaled
// by the branch's gate) sit in LDS (qs, dos); lane owns dims lane + 64 e.
// Returns the branch output's dot with the raw output gradient (for the gate
// gradient) and adds the branch's dq into dq_acc.
template <int D>
__device__ float branch_bwd(const BwdParams &p, const KeySet &ks, int g, const float *qs, const float *dos,
                            const float *dout_s, float *pb, float *db, float (&dq_acc)[D / 64], int lane) {
  constexpr int E = D / 64;
  if (ks.n <= 0) return 0.f;
  // (1) max and sum of exp over the keys
  float m = -INFINITY, l = 0.f;
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float s = -INFINITY;
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
      float a = 0.f;
      for (int j = 0; j < D; ++j) a = fmaf(qs[j], kr.k(j), a);
      s = a * p.scale;
    }
    const float mc = wmax(s);
    const float mn = fmaxf(m, mc);
    l = l * expf(m - mn) + wsum(i < ks.n ? expf(s - mn) : 0.f);
    m = mn;
  }
  const float lse = m + logf(l);
  // (2) o = sum p v; lane owns dims lane + 64 e
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float pi = 0.f;
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
      float a = 0.f;
      for (int j = 0; j < D; ++j) a = fmaf(qs[j], kr.k(j), a);
      pi = expf(a * p.scale - lse);
    }
    pb[lane] = pi;
    wave_lds_sync();
    const int nc = min(64, ks.n - c0);
    for (int ii = 0; ii < nc; ++ii) {
      const KeyRef<D> kr = key_ref<D>(p, ks, c0 + ii, g);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pb[ii], kr.v(lane + 64 * e), o[e]);
    }
    wave_lds_sync();
  }
  float dd = 0.f, go = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dd = fmaf(dos[lane + 64 * e], o[e], dd);
    go = fmaf(dout_s[lane + 64 * e], o[e], go);
  }
  dd = wsum(dd);  // D = dO . o
  go = wsum(go);
  // (3) dS = P (dP - D); dq += scale dS k; dk += scale dS q; dv += P dO
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float pi = 0.f, dsi = 0.f;
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
      float a = 0.f, dp = 0.f;
      for (int j = 0; j < D; ++j) {
        a = fmaf(qs[j], kr.k(j), a);
        dp = fmaf(dos[j], kr.v(j), dp);
      }
      pi = expf(a * p.scale - lse);
      dsi = pi * (dp - dd);
    }
    pb[lane] = pi;
    db[lane] = dsi;
    wave_lds_sync();
    const int nc = min(64, ks.n - c0);
    for (int ii = 0; ii < nc; ++ii) {
      const KeyRef<D> kr = key_ref<D>(p, ks, c0 + ii, g);
      const float ds = db[ii] * p.scale, pw = pb[ii];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        dq_acc[e] = fmaf(ds, kr.k(j), dq_acc[e]);
        unsafeAtomicAdd(kr.dk + j, ds * qs[j]);
        unsafeAtomicAdd(kr.dv + j, pw * dos[j]);
      }
    }
    wave_lds_sync();
  }
  return go;
}

template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_rows_kernel(BwdParams p) {
  constexpr int E = D / 64;
  __shared__ float qs_[kBwdWaves][D], dos_[kBwdWaves][D], dout_[kBwdWaves][D];
  __shared__ float pb_[kBwdWaves][64], db_[kBwdWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kBwdWaves + wv;
  if (item >= p.n * p.hq) return;
  const int64_t row = item / p.hq;
  const int h = (int)(item % p.hq), g = h / (p.hq / p.hkv);
  float *qs = qs_[wv], *dos = dos_[wv], *douts = dout_[wv], *pb = pb_[wv], *db = db_[wv];
  const int64_t oq = (row * p.hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qs[lane + 64 * e] = bfbits2f(p.q[oq + lane + 64 * e]);
    douts[lane + 64 * e] = p.dout[oq + lane + 64 * e];
  }
  float dq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) dq[e] = 0.f;
  const bool vis = row >= p.v0 && row < p.v0 + p.n_vis;
  float *dg = p.dgate + (row * p.hq + h) * 3;
  if (!vis) {  // text row: dense causal over every earlier position
#pragma unroll
    for (int e = 0; e < E; ++e) dos[lane + 64 * e] = douts[lane + 64 * e];
    wave_lds_sync();
    KeySet ks{1, (int)(row + 1), 0, nullptr, 0, 0};
    branch_bwd<D>(p, ks, g, qs, dos, douts, pb, db, dq, lane);
    if (lane < 3) dg[lane] = 0.f;
  } else {
    const int t = (int)(row - p.v0);
    const float *gl = p.gates + (row * p.hq + h) * 3;
    const KeySet sets[3] = {
        KeySet{0, (t + 1) / kBlk, 0, nullptr, 0, 0},
        KeySet{2, 0, 0, p.sel + ((int64_t)t * p.hkv + g) * p.topk, p.topk, t},
        KeySet{1, min(p.window, t + 1), p.v0 + t - min(p.window, t + 1) + 1, nullptr, 0, 0}};
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      KeySet ks = sets[c];
      if (c == 1) {  // keys of the selected blocks up to t
        int n = 0;
        for (int e = 0; e < ks.nsel; ++e) {
          const int b = ks.blocks[e];
          if (b >= 0) n += max(0, min(kBlk, t - b * kBlk + 1));
        }
        ks.n = n;
      }
      const float sg = 1.f / (1.f + expf(-gl[c]));
      wave_lds_sync();
#pragma unroll
      for (int e = 0; e < E; ++e) dos[lane + 64 * e] = sg * douts[lane + 64 * e];
      wave_lds_sync();
      const float go = branch_bwd<D>(p, ks, g, qs, dos, douts, pb, db, dq, lane);
      if (lane == 0) dg[c] = go * sg * (1.f - sg);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) p.dq[oq + lane + 64 * e] = dq[e];
}

// dW = sum over (block, group) of dK_cmp (x) mean; one workgroup of D
// threads per row i of dW (k and v maps).
template <int D>
__global__ __launch_bounds__(D) void bwd_cmp_w_kernel(BwdParams p) {
  const int i = blockIdx.x % D, which = blockIdx.x / D, j = threadIdx.x;
  const float *dy = which ? p.dvc : p.dkc;
  const float *x = which ? p.vbar : p.kbar;
  float acc = 0.f;
  const int64_t rows = (int64_t)p.n_blk * p.hkv;
  for (int64_t r = 0; r < rows; ++r) acc = fmaf(dy[r * D + i], x[r * D + j], acc);
  (which ? p.dwv : p.dwk)[i * D + j] = acc;
}

// Each block's share of the tokens' gradients: W^T dK_cmp / 64 added to the
// 64 rows of dk (dv likewise); one workgroup of D threads per (block, group).
template <int D>
__global__ __launch_bounds__(D) void bwd_cmp_tok_kernel(BwdParams p) {
  __shared__ float dy[2][D];
  const int b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv, j = threadIdx.x;
  const int64_t ob = ((int64_t)b * p.hkv + g) * D;
  dy[0][j] = p.dkc[ob + j];
  dy[1][j] = p.dvc[ob + j];
  __syncthreads();
  float uk = 0.f, uv = 0.f;
  for (int i = 0; i < D; ++i) {
    uk = fmaf(bfbits2f(p.wk[i * D + j]), dy[0][i], uk);
    uv = fmaf(bfbits2f(p.wv[i * D + j]), dy[1][i], uv);
  }
  uk *= 1.f / kBlk;
  uv *= 1.f / kBlk;
  for (int r = 0; r < kBlk; ++r) {
    const int64_t o = ((p.v0 + (int64_t)b * kBlk + r) * p.hkv + g) * D + j;
    p.dk[o] += uk;
    p.dv[o] += uv;
  }
}

template <int D>
hipError_t run(const BwdParams &p, int stage, hipStream_t st) {
  switch (stage) {
    case 0: {  // clear dk, dv, dkc, dvc
      const int64_t nt = p.n * p.hkv * D, nb = (int64_t)p.n_blk * p.hkv * D;
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(1024), dim3(256), 0, st, p.dk, nt);
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(1024), dim3(256), 0, st, p.dv, nt);
      if (nb > 0) {
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(256), dim3(256), 0, st, p.dkc, nb);
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(256), dim3(256), 0, st, p.dvc, nb);
      }
      break;
    }
    case 1:
      if (p.n_blk > 0) hipLaunchKernelGGL((bwd_pool_kernel<D>), dim3(p.n_blk * p.hkv), dim3(D), 0, st, p);
      break;
    case 2: {
      const int64_t items = p.n * p.hq;
      hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3((unsigned)((items + kBwdWaves - 1) / kBwdWaves)),
                         dim3(64 * kBwdWaves), 0, st, p);
      break;
    }
    default:
      hipLaunchKernelGGL((bwd_cmp_w_kernel<D>), dim3(2 * D), dim3(D), 0, st, p);
      if (p.n_blk > 0) hipLaunchKernelGGL((bwd_cmp_tok_kernel<D>), dim3(p.n_blk * p.hkv), dim3(D), 0, st, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdParams &p, int d, int stage, hipStream_t st) {
  if (d == 64) return run<64>(p, stage, st);
  if (d == 128) return run<128>(p, stage, st);
  return hipErrorInvalidValue;
}

}  // namespace nsa
