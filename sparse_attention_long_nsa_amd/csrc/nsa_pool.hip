// Compression-branch pooling: every complete 64-token block of keys (values)
// is averaged per KV head and mapped through the learned d x d linear map
// (VideoNSA model card, "Model Architecture": frame KV blocks are averaged;
// paper summary page, "Method": a learned map turns each block into one
// block-level key/value). Reading: y = W * mean, no bias.
//
// HBM-bound: a workgroup streams one block (64 rows x Hkv x d, contiguous in
// the token-major layout, or gathered through a row map when the vision
// tokens lie in several runs) with 16-byte loads and reduces the rows in
// fp32; W is applied from its L1/L2-resident copy. In a bf16 layer the block
// means are taken by the packing kernel that reads every block anyway, and
// only the maps run here (writing the packed compressed chunks as well); an
// fp32 layer runs the two steps as separate launches (means through the
// workspace); single calls run both in one kernel. Every form adds in the
// same order, so the results are identical.
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

__device__ __forceinline__ void load8f(const bf16 *p, float v[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = bf2f(x[i]);
}
__device__ __forceinline__ void load8f(const float *p, float v[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

constexpr int kPoolThreads = 256;

// Column sums of block b's 64 rows, then the mean: thread items (row phase,
// 16-byte column chunk) sum every P-th row, and the P partials are added in
// phase order. `mean` (LDS or global, C floats) gets the result; `part` is
// LDS scratch of P * C floats.
template <typename T, int D>
__device__ __forceinline__ void block_mean(const PoolJob &jb, int64_t b, float *part, float *mean, int tid) {
  const T *x = static_cast<const T *>(jb.x);
  const int C = jb.n_heads * D;  // columns of one token row
  const int CH = C / 8;          // 16-byte (bf16) column chunks
  const int P = CH >= kPoolThreads ? 1 : kPoolThreads / CH;  // row phases
  const T *xb = x + b * jb.in_stride * (int64_t)C;
  const int32_t *rb = jb.rows ? jb.rows + b * kBlk : nullptr;
  for (int item = tid; item < P * CH; item += kPoolThreads) {
    const int ch = item % CH, rp = item / CH;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int r = rp; r < kBlk; r += P) {  // independent row loads, many in flight
      float v[8];
      load8f((rb ? x + (int64_t)rb[r] * C : xb + (int64_t)r * C) + ch * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[rp * C + ch * 8 + i] = acc[i];
  }
  __syncthreads();
  for (int col = tid; col < C; col += kPoolThreads) {
    float s = 0.f;
    for (int rp = 0; rp < P; ++rp) s += part[rp * C + col];
    mean[col] = s * (1.0f / kBlk);
  }
}

// Output o = (head g, row r) of block b: y = W[r, :] . mean_g, in index order.
template <typename T, int D>
__device__ __forceinline__ void map_out(const PoolJob &jb, int64_t b, const float *mean, int o) {
  const T *w = static_cast<const T *>(jb.w);
  const int g = o / D, r = o % D;
  const T *wr = w + (int64_t)r * D;
  const float *mg = mean + g * D;
  float acc = 0.f;
  for (int i = 0; i < D; i += 8) {
    float wv[8];
    load8f(wr + i, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += wv[e] * mg[i + e];
  }
  const int64_t dst = (b * jb.out_stride * jb.n_heads + g) * (int64_t)D + r;
  const uint16_t hi = f2bf_bits(acc);
  if (jb.out_hi) jb.out_hi[dst] = hi;
  if (jb.out_lo) jb.out_lo[dst] = f2bf_bits(acc - bfbits2f(hi));
  if (jb.out_h16) {
    const uint16_t h = f2h_bits(acc);
    jb.out_h16[dst] = h;
    if (jb.status && h16_nonfinite(h)) atomicOr(jb.status, kStatusRange);
  }
  if (jb.out_f32) jb.out_f32[dst] = acc;
}

// Both steps in one workgroup per block (small jobs: one block per sequence
// while generating, or a cache built once).
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void cmp_pool_kernel(PoolJob j0, PoolJob j1) {
  const PoolJob &jb = blockIdx.y == 0 ? j0 : j1;
  const int C = jb.n_heads * D;
  const int CH = C / 8;
  const int P = CH >= kPoolThreads ? 1 : kPoolThreads / CH;
  extern __shared__ float smem[];
  float *part = smem;             // [P][C]
  float *mean = smem + P * C;     // [C]
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < jb.n_blk; b += gridDim.x) {
    block_mean<T, D>(jb, b, part, mean, tid);
    __syncthreads();
    for (int o = tid; o < C; o += kPoolThreads) map_out<T, D>(jb, b, mean, o);
    __syncthreads();
  }
}

// Pooling in two launches (fp32 layers), so that the streaming of the rows is
// not held up by the maps: block means into a workspace, then the maps, one
// output per thread. Same arithmetic in the same order as cmp_pool_kernel.
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_mean_kernel(PoolJob j0, PoolJob j1, float *m0, float *m1) {
  const PoolJob &jb = blockIdx.y == 0 ? j0 : j1;
  const int64_t b = blockIdx.x;
  if (b >= jb.n_blk) return;
  extern __shared__ float smem[];
  const int C = jb.n_heads * D;
  block_mean<T, D>(jb, b, smem, (blockIdx.y == 0 ? m0 : m1) + b * C, threadIdx.x);
}

// kMapBlocks blocks per workgroup of kMapThreads: W is staged once in LDS,
// transposed with a padded row (conflict-free both ways). A thread owns one
// output row r and walks eight (block, head) mean vectors at once, read with
// wave-uniform addresses (scalar loads): eight independent index-ordered
// fp32 sums, each the same as map_out's. (Measured: 4 blocks per workgroup
// is 10x slower -- every workgroup reads the same W lines at once -- and 64
// is 3.5x slower -- too few workgroups.)
constexpr int kMapBlocks = 16;
constexpr int kMapThreads = 512;

// Element (block blk, head g, dim r) of a job's packed output: row blk % 64
// of the K tile, or column blk % 64 (its key slot) of the V^T tile, in chunk
// blk / 64 of head g.
template <int D>
__device__ __forceinline__ int64_t packed_at(const PoolJob &jb, int64_t blk, int g, int r) {
  using T = PackedTile<D>;
  const int key = (int)(blk % kBlk);
  const int64_t base = ((int64_t)g * jb.n_cch + blk / kBlk) * (T::KE + T::VE);
  if (!jb.packed_v) return base + key * D + 8 * T::template swz<2 * D>(key, r / 8) + r % 8;
  const int sl = T::vslot(key);
  return base + T::KE + r * kBlk + 8 * T::template swz<2 * kBlk>(r, sl / 8) + sl % 8;
}

template <typename T, int D>
__global__ __launch_bounds__(kMapThreads) void pool_map_kernel(PoolJob j0, PoolJob j1, const float *m0,
                                                               const float *m1) {
  constexpr int WS = D + 1, NQ = 8, TPR = kMapThreads / D;
  const PoolJob &jb = blockIdx.y == 0 ? j0 : j1;
  const int hkv = jb.n_heads, C = hkv * D;
  const int64_t b0 = (int64_t)blockIdx.x * kMapBlocks;
  if (b0 >= jb.n_blk) return;
  const int nv = (int)min((int64_t)kMapBlocks, jb.n_blk - b0) * hkv;  // (block, head) vectors
  const float *means = (blockIdx.y == 0 ? m0 : m1) + b0 * C;
  extern __shared__ float wt[];  // [D][WS]: wt[i * WS + r] = W[r][i]
  const T *w = static_cast<const T *>(jb.w);
  const int tid = threadIdx.x;
  for (int e = tid; e < D * D / 8; e += kMapThreads) {  // W's rows, 16-byte (bf16) chunks
    const int r = (8 * e) / D, i0 = (8 * e) % D;
    float v[8];
    load8f(w + 8 * e, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) wt[(i0 + j) * WS + r] = v[j];
  }
  __syncthreads();
  const int r = tid % D;
  const int part = __builtin_amdgcn_readfirstlane(tid / D);  // D >= 64: one value per wave
  for (int v0 = part * NQ; v0 < nv; v0 += TPR * NQ) {
    float acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
    for (int i0 = 0; i0 < D; i0 += 16) {
      float wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) wv[j] = wt[(i0 + j) * WS + r];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float *mq = means + (int64_t)min(v0 + q, nv - 1) * D + i0;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[q] += wv[j] * mq[j];
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (v0 + q >= nv) break;
      const int bl = (v0 + q) / hkv, g = (v0 + q) % hkv;
      const int64_t dst = ((b0 + bl) * jb.out_stride * hkv + g) * (int64_t)D + r;
      const uint16_t hi = f2bf_bits(acc[q]);
      if (jb.out_hi) jb.out_hi[dst] = hi;
      if (jb.out_lo) jb.out_lo[dst] = f2bf_bits(acc[q] - bfbits2f(hi));
      if (jb.out_h16) {
        const uint16_t h = f2h_bits(acc[q]);
        jb.out_h16[dst] = h;
        if (jb.packed) jb.packed[packed_at<D>(jb, b0 + bl, g, r)] = h;
        if (jb.status && h16_nonfinite(h)) atomicOr(jb.status, kStatusRange);
      }
      if (jb.out_f32) jb.out_f32[dst] = acc[q];
    }
  }
  // the last workgroup zeroes the packed rows past the last block
  if (jb.packed && b0 + kMapBlocks >= jb.n_blk) {
    const int64_t n_pad = (int64_t)jb.n_cch * kBlk - jb.n_blk;
    for (int64_t e = tid; e < n_pad * hkv * D; e += kMapThreads) {
      const int rr = (int)(e % D), g = (int)((e / D) % hkv);
      jb.packed[packed_at<D>(jb, jb.n_blk + e / ((int64_t)D * hkv), g, rr)] = 0;
    }
  }
}

// One new row per sequence into its cache, 16 bytes per thread.
__global__ __launch_bounds__(256) void append_rows_kernel(const uint16_t *__restrict__ k_new,
                                                          const uint16_t *__restrict__ v_new,
                                                          uint16_t *__restrict__ k_cache,
                                                          uint16_t *__restrict__ v_cache, int batch,
                                                          int n_cols, int64_t cap, int64_t row) {
  const int per = n_cols / 8;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * batch * per) return;
  const int kv = i / (batch * per), rest = i % (batch * per);
  const int b = rest / per, c = rest % per;
  const uint16_t *src = (kv ? v_new : k_new) + (int64_t)b * n_cols + 8 * c;
  uint16_t *dst = (kv ? v_cache : k_cache) + ((int64_t)b * cap + row) * n_cols + 8 * c;
  *reinterpret_cast<u16x8 *>(dst) = *reinterpret_cast<const u16x8 *>(src);
}

// fp32 inputs -> bf16 high part (and optionally the bf16 residual).
__global__ __launch_bounds__(256) void split_bf16_kernel(const float *__restrict__ x, int64_t n,
                                                         uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = x[i];
    const uint16_t h = f2bf_bits(v);
    hi[i] = h;
    if (lo) lo[i] = f2bf_bits(v - bfbits2f(h));
  }
}

// fp32 inputs -> fp16 (values past fp16's range flagged in *status).
__global__ __launch_bounds__(256) void to_f16_kernel(const float *__restrict__ x, int64_t n,
                                                     uint16_t *__restrict__ out, int32_t *status) {
  bool ovf = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint16_t h = f2h_bits(x[i]);
    out[i] = h;
    ovf |= h16_nonfinite(h);
  }
  if (ovf && status) atomicOr(status, kStatusRange);
}

}  // namespace

size_t pool_smem_bytes(int n_heads, int d) {
  const int C = n_heads * d, CH = C / 8;
  const int P = CH >= kPoolThreads ? 1 : kPoolThreads / CH;
  return sizeof(float) * (size_t)(P * C + C);
}

hipError_t launch_cmp_pool(const PoolJob &j0, const PoolJob *j1, int d, bool fp32, hipStream_t st) {
  const int64_t nb = j1 ? (j0.n_blk > j1->n_blk ? j0.n_blk : j1->n_blk) : j0.n_blk;
  if (nb <= 0) return hipSuccess;
  const int gx = (int)(nb < 1024 ? nb : 1024);
  dim3 grid(gx, j1 ? 2 : 1);
  const size_t smem = pool_smem_bytes(j0.n_heads, d);
  const PoolJob &jj = j1 ? *j1 : j0;
  if (fp32) {
    if (d == 64) hipLaunchKernelGGL((cmp_pool_kernel<float, 64>), grid, dim3(kPoolThreads), smem, st, j0, jj);
    else hipLaunchKernelGGL((cmp_pool_kernel<float, 128>), grid, dim3(kPoolThreads), smem, st, j0, jj);
  } else {
    if (d == 64) hipLaunchKernelGGL((cmp_pool_kernel<bf16, 64>), grid, dim3(kPoolThreads), smem, st, j0, jj);
    else hipLaunchKernelGGL((cmp_pool_kernel<bf16, 128>), grid, dim3(kPoolThreads), smem, st, j0, jj);
  }
  return hipGetLastError();
}

hipError_t launch_cmp_pool_split(const PoolJob &j0, const PoolJob &j1, int d, bool fp32, float *means,
                                 hipStream_t st) {
  const int64_t nb = j0.n_blk > j1.n_blk ? j0.n_blk : j1.n_blk;
  if (nb <= 0) return hipSuccess;
  const int64_t C = (int64_t)j0.n_heads * d;
  float *m0 = means, *m1 = means + j0.n_blk * C;
  const size_t smem = pool_smem_bytes(j0.n_heads, d);
  const dim3 g1((unsigned)nb, 2), g2((unsigned)((nb + kMapBlocks - 1) / kMapBlocks), 2);
  const size_t smem2 = sizeof(float) * (size_t)d * (d + 1);
#define NSA_POOL2(T, D)                                                                                  \
  hipLaunchKernelGGL((pool_mean_kernel<T, D>), g1, dim3(kPoolThreads), smem, st, j0, j1, m0, m1);       \
  hipLaunchKernelGGL((pool_map_kernel<T, D>), g2, dim3(kMapThreads), smem2, st, j0, j1, m0, m1);
  if (fp32) {
    if (d == 64) { NSA_POOL2(float, 64) } else { NSA_POOL2(float, 128) }
  } else {
    if (d == 64) { NSA_POOL2(bf16, 64) } else { NSA_POOL2(bf16, 128) }
  }
#undef NSA_POOL2
  return hipGetLastError();
}

hipError_t launch_cmp_map(const PoolJob &j0, const PoolJob &j1, int d, bool fp32, const float *means,
                          hipStream_t st) {
  const int64_t nb = j0.n_blk > j1.n_blk ? j0.n_blk : j1.n_blk;
  if (nb <= 0) return hipSuccess;
  const int64_t C = (int64_t)j0.n_heads * d;
  const float *m0 = means, *m1 = means + j0.n_blk * C;
  const dim3 g2((unsigned)((nb + kMapBlocks - 1) / kMapBlocks), 2);
  const size_t smem2 = sizeof(float) * (size_t)d * (d + 1);
#define NSA_MAP(T, D) hipLaunchKernelGGL((pool_map_kernel<T, D>), g2, dim3(kMapThreads), smem2, st, j0, j1, m0, m1);
  if (fp32) {
    if (d == 64) { NSA_MAP(float, 64) } else { NSA_MAP(float, 128) }
  } else {
    if (d == 64) { NSA_MAP(bf16, 64) } else { NSA_MAP(bf16, 128) }
  }
#undef NSA_MAP
  return hipGetLastError();
}

hipError_t launch_append_rows(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_cache,
                              uint16_t *v_cache, int batch, int n_cols, int64_t cap, int64_t row,
                              hipStream_t st) {
  const int n = 2 * batch * (n_cols / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, st, k_new, v_new,
                     k_cache, v_cache, batch, n_cols, cap, row);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, hi, lo);
  return hipGetLastError();
}

hipError_t launch_to_f16(const float *x, int64_t n, uint16_t *out, hipStream_t st, int32_t *status) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, out, status);
  return hipGetLastError();
}

}  // namespace nsa
