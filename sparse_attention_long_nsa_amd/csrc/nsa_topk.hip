// Top-k block selection kernel: one wave per (vision query, KV group) row of
// the frame-packed group scores written by the compression kernel. The
// selection itself is select_topk_row.
#include "nsa_kernels.h"
#include "nsa_select.h"

namespace nsa {

namespace {

constexpr int kWavesPerWG = 1;  // one wave per workgroup: early exits need no barrier care

template <int NPL>
__global__ __launch_bounds__(64) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[256];
  const int lane = threadIdx.x;
  const int64_t wid = blockIdx.x;
  const int t = (int)(wid / p.hkv);
  const int g = (int)(wid % p.hkv);
  if (t >= p.n_vis) return;
  const int f = t / kBlk;  // own block == number of candidate blocks
  int32_t *out = p.sel + ((int64_t)t * p.hkv + g) * p.k;
  const float *row = p.gs + frame_off(f, p.hkv) + (int64_t)(g * kBlk + (t - f * kBlk)) * f;
  select_topk_row<NPL>(row, f, p.k, out, hist, lane);
}

template <int NPL>
hipError_t run(const TopkParams &p, hipStream_t st) {
  const int64_t n = (int64_t)p.n_vis * p.hkv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((topk_kernel<NPL>), dim3((unsigned)n), dim3(64 * kWavesPerWG), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, int n_blk_max, hipStream_t st) {
  if (n_blk_max <= 64 * 4) return run<4>(p, st);
  if (n_blk_max <= 64 * 16) return run<16>(p, st);
  if (n_blk_max <= 64 * 32) return run<32>(p, st);
  if (n_blk_max <= 64 * 64) return run<64>(p, st);
  if (n_blk_max <= 64 * 128) return run<128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace nsa
