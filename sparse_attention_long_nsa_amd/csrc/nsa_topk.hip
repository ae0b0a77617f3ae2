// Top-k block selection kernel over the frame-packed group scores written
// by the compression kernel (per frame f and KV group g a [64 tokens][f]
// block of scores). One wave per (token, group) row; a workgroup holds
// kWaves consecutive tokens of one (frame, group), heaviest frames first.
// The selection itself is select_topk_row.
#include "nsa_kernels.h"
#include "nsa_select.h"

namespace nsa {

namespace {

#ifndef NSA_TOPK_WAVES
#define NSA_TOPK_WAVES 1
#endif
constexpr int kWaves = NSA_TOPK_WAVES;  // rows (one per wave) per workgroup

template <int NPL>
__global__ __launch_bounds__(64 * kWaves) void topk_kernel(TopkParams p, int n_frames) {
  __shared__ uint32_t hist[kWaves][256];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar addressing
  constexpr int per_group = kBlk / kWaves;
  const int per_frame = p.hkv * per_group;
  const int f = n_frames - 1 - (int)(blockIdx.x / per_frame);  // own block == number of candidates
  const int rem = (int)(blockIdx.x % per_frame);
  const int g = rem / per_group;
  const int tl = (rem % per_group) * kWaves + wv;
  if (f * kBlk + tl >= p.n_vis) return;
  const float *row = p.gs + frame_off(f, p.hkv) + (int64_t)(g * kBlk + tl) * f;
  select_topk_row<NPL>(row, f, p.k, p.sel + ((int64_t)(f * kBlk + tl) * p.hkv + g) * p.k, hist[wv], lane);
}

template <int NPL>
hipError_t run(const TopkParams &p, int n_frames, hipStream_t st) {
  const int64_t n_wg = (int64_t)n_frames * p.hkv * (kBlk / kWaves);
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((topk_kernel<NPL>), dim3((unsigned)n_wg), dim3(64 * kWaves), 0, st, p, n_frames);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, int n_blk_max, hipStream_t st) {
  const int n_frames = (p.n_vis + kBlk - 1) / kBlk;
  if (n_blk_max <= 64 * 4) return run<4>(p, n_frames, st);
  if (n_blk_max <= 64 * 16) return run<16>(p, n_frames, st);
  if (n_blk_max <= 64 * 32) return run<32>(p, n_frames, st);
  if (n_blk_max <= 64 * 64) return run<64>(p, n_frames, st);
  if (n_blk_max <= 64 * 128) return run<128>(p, n_frames, st);
  return hipErrorInvalidValue;
}

}  // namespace nsa
