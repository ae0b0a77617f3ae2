// Matrix-core peak probe: a loop of independent bf16 MFMAs per wave, enough
// of them in flight (eight accumulators) that issue never waits on a result.
// It measures the dense bf16 rate the layer's kernels are priced against.
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

}  // namespace
}  // namespace nsa

extern "C" nsa_status nsa_probe_mfma_bf16(int32_t n_wg, int32_t iters, float *out, void *stream) {
  if (n_wg < 1 || iters < 1 || out == nullptr) return NSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(nsa::mfma_loop_kernel, dim3((unsigned)n_wg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? NSA_OK : NSA_ERR_HIP;
}
