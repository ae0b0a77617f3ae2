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
//   bwd_rows   one wave per (row, KV group) with all its query heads; per
//              branch three passes over its keys, lane = key for dot
//              products and lane = dimension for sums over keys: (1) max
//              and sum of the exponentials, (2) output o and D = dO . o (and
//              the gate gradient), (3) dS = P (dP - D): dq in registers,
//              dk / dv (or the compressed dK / dV) summed over the heads and
//              accumulated with float atomics
//   bwd_cmp_w  dW = sum over blocks of dK_cmp x mean^T, and each block's
//              W^T dK_cmp / 64 added to its 64 tokens' dk (dv likewise)
#include "nsa_kernels.h"
#include "nsa_index.h"
#include "nsa_select.h"

namespace nsa {

namespace {

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
// selected blocks, in block order). The blocks come in ascending order,
// -1 padded: every one but the last is a complete earlier block of 64 keys,
// and the last is the query's own block, cut at t; so key i is key i % 64
// of entry i / 64. Any other list (not the forward's) gives meaningless
// gradients but no access outside the rows 0 .. t.
__device__ __forceinline__ int64_t sel_row(const BwdParams &p, const KeySet &ks, int i) {
  return p.v0 + sel_key_row(ks.blocks[i / kBlk], i % kBlk, ks.t);
}

template <int D>
struct KeyRef {
  const uint16_t *kb = nullptr, *vb = nullptr;  // token rows (bf16)
  const float *kf = nullptr, *vf = nullptr;     // compressed rows (fp32)
  float *dk = nullptr, *dv = nullptr;
  __device__ __forceinline__ float k(int j) const { return kb ? bfbits2f(kb[j]) : kf[j]; }
  __device__ __forceinline__ float v(int j) const { return vb ? bfbits2f(vb[j]) : vf[j]; }
  // eight consecutive values from j (a multiple of 8) in one or two loads
  __device__ __forceinline__ static void load8(const uint16_t *b16, const float *f32, int j, float (&x)[8]) {
    if (b16) {
      const u16x8 u = *reinterpret_cast<const u16x8 *>(b16 + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bfbits2f(u[e]);
    } else {
      const float4 a = *reinterpret_cast<const float4 *>(f32 + j), c = *reinterpret_cast<const float4 *>(f32 + j + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    }
  }
  __device__ __forceinline__ void k8(int j, float (&x)[8]) const { load8(kb, kf, j, x); }
  __device__ __forceinline__ void v8(int j, float (&x)[8]) const { load8(vb, vf, j, x); }
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

// One branch for one (row, KV group) held by one wave, all G query heads of
// the group together so that every key row is read once for the group and
// its gradients are summed over the heads before the atomics. q, dO (scaled
// by each head's gate) and the raw output gradient sit in LDS; for sums over
// keys lane l owns dims l + 64 e. Adds the branch's dq into dq and returns,
// per head, the branch output's dot with the raw output gradient (go).
template <int D, int G>
__device__ void branch_bwd(const BwdParams &p, const KeySet &ks, int g, const float (*qs)[D],
                           const float (*dos)[D], const float (*douts)[D], float (*pb)[64], float (*db)[64],
                           float (&dq)[G][D / 64], float (&go)[G], int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int h = 0; h < G; ++h) go[h] = 0.f;
  if (ks.n <= 0) return;
  // (1) per head: max and sum of exp over the keys
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = -INFINITY;
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = 0.f;
      for (int j0 = 0; j0 < D; j0 += 8) {
        float kv[8];
        kr.k8(j0, kv);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int h = 0; h < G; ++h) sc[h] = fmaf(qs[h][j0 + jj], kv[jj], sc[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] *= p.scale;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], wmax(sc[h]));
      l[h] = l[h] * expf(m[h] - mn) + wsum(i < ks.n ? expf(sc[h] - mn) : 0.f);
      m[h] = mn;
    }
  }
  float lse[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lse[h] = m[h] + logf(l[h]);
  // (2) o = sum p v per head, then D = dO . o and go = dout . o
  float o[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
      for (int j0 = 0; j0 < D; j0 += 8) {
        float kv[8];
        kr.k8(j0, kv);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int h = 0; h < G; ++h) sc[h] = fmaf(qs[h][j0 + jj], kv[jj], sc[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = expf(sc[h] * p.scale - lse[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) pb[h][lane] = sc[h];
    wave_lds_sync();
    const int nc = min(64, ks.n - c0);
    for (int ii = 0; ii < nc; ++ii) {
      const KeyRef<D> kr = key_ref<D>(p, ks, c0 + ii, g);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float vv = kr.v(lane + 64 * e);
#pragma unroll
        for (int h = 0; h < G; ++h) o[h][e] = fmaf(pb[h][ii], vv, o[h][e]);
      }
    }
    wave_lds_sync();
  }
  float dd[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a = fmaf(dos[h][lane + 64 * e], o[h][e], a);
      b = fmaf(douts[h][lane + 64 * e], o[h][e], b);
    }
    dd[h] = wsum(a);
    go[h] = wsum(b);
  }
  // (3) dS = P (dP - D); dq += scale dS k; dk += scale sum_h dS q; dv += sum_h P dO
  for (int c0 = 0; c0 < ks.n; c0 += 64) {
    const int i = c0 + lane;
    float pr[G], dsr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { pr[h] = 0.f; dsr[h] = 0.f; }
    if (i < ks.n) {
      const KeyRef<D> kr = key_ref<D>(p, ks, i, g);
      float sc[G], dp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { sc[h] = 0.f; dp[h] = 0.f; }
      for (int j0 = 0; j0 < D; j0 += 8) {
        float kv[8], vv[8];
        kr.k8(j0, kv);
        kr.v8(j0, vv);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            sc[h] = fmaf(qs[h][j0 + jj], kv[jj], sc[h]);
            dp[h] = fmaf(dos[h][j0 + jj], vv[jj], dp[h]);
          }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[h] = expf(sc[h] * p.scale - lse[h]);
        dsr[h] = pr[h] * (dp[h] - dd[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pb[h][lane] = pr[h];
      db[h][lane] = dsr[h];
    }
    wave_lds_sync();
    const int nc = min(64, ks.n - c0);
    for (int ii = 0; ii < nc; ++ii) {
      const KeyRef<D> kr = key_ref<D>(p, ks, c0 + ii, g);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        const float kv = kr.k(j);
        float gk = 0.f, gv = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ds = db[h][ii] * p.scale;
          dq[h][e] = fmaf(ds, kv, dq[h][e]);
          gk = fmaf(ds, qs[h][j], gk);
          gv = fmaf(pb[h][ii], dos[h][j], gv);
        }
        unsafeAtomicAdd(kr.dk + j, gk);
        unsafeAtomicAdd(kr.dv + j, gv);
      }
    }
    wave_lds_sync();
  }
}

constexpr int kBwdWavesG = 2;  // (row, group) items per workgroup

template <int D, int G>
__global__ __launch_bounds__(64 * kBwdWavesG) void bwd_rows_kernel(BwdParams p) {
  constexpr int E = D / 64;
  __shared__ float qs_[kBwdWavesG][G][D], dos_[kBwdWavesG][G][D], dout_[kBwdWavesG][G][D];
  __shared__ float pb_[kBwdWavesG][G][64], db_[kBwdWavesG][G][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kBwdWavesG + wv;
  if (item >= p.n * p.hkv) return;
  const int64_t row = item / p.hkv;
  const int g = (int)(item % p.hkv);
  float(*qs)[D] = qs_[wv];
  float(*dos)[D] = dos_[wv];
  float(*douts)[D] = dout_[wv];
  const int64_t oq = (row * p.hq + (int64_t)g * G) * D;  // the group's first head
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qs[h][lane + 64 * e] = bfbits2f(p.q[oq + h * D + lane + 64 * e]);
      douts[h][lane + 64 * e] = p.dout[oq + h * D + lane + 64 * e];
    }
  float dq[G][E], go[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) dq[h][e] = 0.f;
  const bool vis = row >= p.v0 && row < p.v0 + p.n_vis;
  float *dg = p.dgate + (row * p.hq + (int64_t)g * G) * 3;
  if (!vis) {  // text row: dense causal over every earlier position
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) dos[h][lane + 64 * e] = douts[h][lane + 64 * e];
    wave_lds_sync();
    KeySet ks{1, (int)(row + 1), 0, nullptr, 0, 0};
    branch_bwd<D, G>(p, ks, g, qs, dos, douts, pb_[wv], db_[wv], dq, go, lane);
    if (lane < 3 * G) dg[lane] = 0.f;
  } else {
    const int t = (int)(row - p.v0);
    const float *gl = p.gates + (row * p.hq + (int64_t)g * G) * 3;
    const int32_t *blocks = p.sel + ((int64_t)t * p.hkv + g) * p.topk;
    int n_sel = 0;
    for (int e = 0; e < p.topk; ++e) {
      n_sel += sel_block_keys(blocks[e], t);
    }
    const int nw = min(p.window, t + 1);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const KeySet ks = c == 0 ? KeySet{0, (t + 1) / kBlk, 0, nullptr, 0, 0}
                      : c == 1 ? KeySet{2, n_sel, 0, blocks, p.topk, t}
                               : KeySet{1, nw, p.v0 + t - nw + 1, nullptr, 0, 0};
      float sg[G];
#pragma unroll
      for (int h = 0; h < G; ++h) sg[h] = 1.f / (1.f + expf(-gl[h * 3 + c]));
      wave_lds_sync();
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) dos[h][lane + 64 * e] = sg[h] * douts[h][lane + 64 * e];
      wave_lds_sync();
      branch_bwd<D, G>(p, ks, g, qs, dos, douts, pb_[wv], db_[wv], dq, go, lane);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) dg[h * 3 + c] = go[h] * sg[h] * (1.f - sg[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) p.dq[oq + h * D + lane + 64 * e] = dq[h][e];
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

template <int D, int G>
hipError_t run_rows(const BwdParams &p, hipStream_t st) {
  const int64_t items = p.n * p.hkv;
  hipLaunchKernelGGL((bwd_rows_kernel<D, G>), dim3((unsigned)((items + kBwdWavesG - 1) / kBwdWavesG)),
                     dim3(64 * kBwdWavesG), 0, st, p);
  return hipGetLastError();
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
    case 2:
      switch (p.hq / p.hkv) {
        case 1: return run_rows<D, 1>(p, st);
        case 2: return run_rows<D, 2>(p, st);
        case 3: return run_rows<D, 3>(p, st);
        case 4: return run_rows<D, 4>(p, st);
        case 5: return run_rows<D, 5>(p, st);
        case 6: return run_rows<D, 6>(p, st);
        case 7: return run_rows<D, 7>(p, st);
        case 8: return run_rows<D, 8>(p, st);
        default: return hipErrorInvalidValue;
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
