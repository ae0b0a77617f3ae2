// Top-k block selection kernel over the frame-packed group scores written
// by the compression kernel (per frame f and KV group g a [64 tokens][f]
// block of scores). One wave (one workgroup) per (token, group) row,
// heaviest frames first.
// The selection itself is select_topk_row.
#include "nsa_kernels.h"
#include "nsa_select.h"

namespace nsa {

namespace {

// The row's loads per lane (NPL) are chosen per frame from the sizes
// 1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128 (the smallest that covers the
// row), so a short row does not issue the loads of the longest.
constexpr int smaller_npl(int n) { return n <= 8 ? n / 2 : (n % 3 == 0 ? n / 3 * 2 : n / 4 * 3); }

template <int NPL>
__device__ __forceinline__ void select_sized(const float *row, int f, int k, int32_t *out, uint32_t *hist,
                                             int lane) {
  constexpr int P = smaller_npl(NPL);
  if constexpr (P >= 1) {
    if (f <= 64 * P) {  // wave-uniform
      select_sized<P>(row, f, k, out, hist, lane);
      return;
    }
  }
  select_topk_row<NPL>(row, f, k, out, hist, lane);
}

// Rows of up to 2,048 candidates run at six waves per SIMD (0.50 ms at
// 131,072 tokens against 0.52 ms at five); longer rows keep every candidate
// in registers at lower occupancy.
template <int NPL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NPL <= 32 ? 6 : 1)))
void topk_kernel(TopkParams p, int n_frames) {
  __shared__ uint32_t hist[256];
  const int lane = threadIdx.x & 63;
  const int per_frame = p.hkv * kBlk;
  const int f = n_frames - 1 - (int)(blockIdx.x / per_frame);  // own block == number of candidates
  const int rem = (int)(blockIdx.x % per_frame);
  const int g = rem / kBlk;
  const int tl = rem % kBlk;
  if (f * kBlk + tl >= p.n_vis) return;
  const float *row = p.gs + frame_off(f, p.hkv) + (int64_t)(g * kBlk + tl) * f;
  select_sized<NPL>(row, f, p.k, p.sel + ((int64_t)(f * kBlk + tl) * p.hkv + g) * p.k, hist, lane);
}

template <int NPL>
hipError_t run(const TopkParams &p, int n_frames, hipStream_t st) {
  const int64_t n_wg = (int64_t)n_frames * p.hkv * kBlk;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((topk_kernel<NPL>), dim3((unsigned)n_wg), dim3(64), 0, st, p, n_frames);
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
