// Compression-branch pooling: every complete 64-token block of keys (values)
// is averaged per KV head and mapped through the learned d x d linear map
// (VideoNSA model card, "Model Architecture": frame KV blocks are averaged;
// paper summary page, "Method": a learned map turns each block into one
// block-level key/value). Reading: y = W * mean, no bias.
//
// HBM-bound: each workgroup streams one block (64 rows x Hkv x d, contiguous
// in the token-major layout, or gathered through a row map when the vision
// tokens lie in several runs) with 16-byte loads, reduces the rows in fp32,
// and applies W from the L1/L2-resident copy.
#include "nsa_kernels.h"

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

template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void cmp_pool_kernel(PoolJob j0, PoolJob j1) {
  const PoolJob &jb = blockIdx.y == 0 ? j0 : j1;
  const T *x = static_cast<const T *>(jb.x);
  const T *w = static_cast<const T *>(jb.w);
  const int hkv = jb.n_heads;
  const int C = hkv * D;     // columns of one token row
  const int CH = C / 8;      // 16-byte (bf16) column chunks
  const int P = CH >= kPoolThreads ? 1 : kPoolThreads / CH;  // row phases
  extern __shared__ float smem[];
  float *part = smem;             // [P][C]
  float *mean = smem + P * C;     // [C]
  const int tid = threadIdx.x;

  for (int64_t b = blockIdx.x; b < jb.n_blk; b += gridDim.x) {
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
    __syncthreads();
    for (int o = tid; o < C; o += kPoolThreads) {
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
      const int64_t dst = (b * jb.out_stride * hkv + g) * (int64_t)D + r;
      const uint16_t hi = f2bf_bits(acc);
      if (jb.out_hi) jb.out_hi[dst] = hi;
      if (jb.out_lo) jb.out_lo[dst] = f2bf_bits(acc - bfbits2f(hi));
      if (jb.out_h16) jb.out_h16[dst] = f2h_bits(acc);
      if (jb.out_f32) jb.out_f32[dst] = acc;
    }
    __syncthreads();
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

// fp32 inputs -> fp16.
__global__ __launch_bounds__(256) void to_f16_kernel(const float *__restrict__ x, int64_t n,
                                                     uint16_t *__restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = f2h_bits(x[i]);
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

hipError_t launch_to_f16(const float *x, int64_t n, uint16_t *out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, out);
  return hipGetLastError();
}

}  // namespace nsa
