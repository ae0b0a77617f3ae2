// Measurement aids (they compute nothing of the layer):
//   matrix-core peak probe: a loop of independent bf16 MFMAs per wave, enough
//     of them in flight (eight accumulators) that issue never waits on a
//     result; it measures the dense bf16 rate the kernels are priced against
//   block-stream probe: workgroups read pseudo-random 32 KB blocks of a
//     buffer, the access pattern of the selection kernel's copies, so its
//     rate at a buffer size far beyond the L2 is the fabric rate that kernel
//     can reach
#include "nsa.h"
#include "nsa_common.h"

namespace nsa {
namespace {

constexpr int kChains = 8;
constexpr int kUnroll = 16;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *__restrict__ out) {
  const int tid = threadIdx.x;
  u16x8 a, b[kChains];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // small finite bf16 values that differ per lane and chain (~0.0078..)
    a[i] = (uint16_t)(0x3c00u + ((tid * 8 + i) & 0xffu));
#pragma unroll
    for (int j = 0; j < kChains; ++j) b[j][i] = (uint16_t)(0x3c00u + ((tid * 5 + 3 * i + 17 * j) & 0xffu));
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // `iters` counts rounds of kUnroll; the back edge costs a few register
  // moves, paid once per kUnroll * kChains products
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < kChains; ++j) acc[j] = mfma_bf16(a, b[j], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * 256 + tid] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamWaves = 8, kStreamUnroll = 2;
constexpr int kBlockPieces = 32768 / 16;  // 16-byte pieces per 32 KB block

// Each workgroup reads `iters` blocks chosen by a linear congruential
// sequence seeded by its index (block = state mod n_blocks, always inside
// the buffer), every lane 16 bytes per load, two blocks in flight per wave,
// and folds them into one checksum word per thread.
__global__ __launch_bounds__(64 * kStreamWaves) void block_stream_kernel(const u32x4 *__restrict__ buf,
                                                                          int64_t n_blocks, int iters,
                                                                          uint32_t *__restrict__ out) {
  constexpr int PER = kBlockPieces / (64 * kStreamWaves);
  const int tid = threadIdx.x;
  uint32_t h = blockIdx.x * 2654435761u + 12345u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; it += kStreamUnroll) {
    u32x4 v[kStreamUnroll][PER];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      h = h * 1664525u + 1013904223u;
      const int64_t blk = (int64_t)((h >> 8) % (uint64_t)n_blocks);
      const u32x4 *src = buf + blk * kBlockPieces + tid;
#pragma unroll
      for (int q = 0; q < PER; ++q) v[u][q] = __builtin_nontemporal_load(src + q * 64 * kStreamWaves);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
#pragma unroll
      for (int q = 0; q < PER; ++q) acc ^= v[u][q];
  }
  out[(int64_t)blockIdx.x * 64 * kStreamWaves + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace
}  // namespace nsa

extern "C" nsa_status nsa_probe_block_stream(const void *buf, int64_t n_blocks, int32_t n_wg, int32_t iters,
                                             uint32_t *out, void *stream) {
  if (!buf || !out || n_blocks < 1 || n_wg < 1 || iters < 2 || iters % 2 != 0) return NSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return NSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(nsa::block_stream_kernel, dim3((unsigned)n_wg), dim3(64 * nsa::kStreamWaves), 0,
                     static_cast<hipStream_t>(stream), static_cast<const nsa::u32x4 *>(buf), n_blocks, iters, out);
  return hipGetLastError() == hipSuccess ? NSA_OK : NSA_ERR_HIP;
}

extern "C" nsa_status nsa_probe_mfma_bf16(int32_t n_wg, int32_t iters, float *out, void *stream) {
  if (n_wg < 1 || iters < 1 || out == nullptr) return NSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(nsa::mfma_loop_kernel, dim3((unsigned)n_wg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? NSA_OK : NSA_ERR_HIP;
}
