// Row maps of a sequence whose vision tokens lie in several runs (paper
// summary page, "Method": the tokens are split into a vision set and a text
// set by position; the NSA branches run on the vision set in position
// order). The kernels address a vision row t or text row r through
//   vmap[t] = position of the t-th vision token,
//   tmap[r] = position of the r-th text token,
//   tnvb[r] = vision tokens before that text token (its visible vision keys
//             are the vision rows 0 .. tnvb[r] - 1).
// The mask itself travels as kernel arguments, one slice of 32 * kMaskWords
// positions per launch, so no host buffer has to outlive the call.
#include "nsa_kernels.h"

namespace nsa {

namespace {

__global__ __launch_bounds__(kMaskWords) void row_map_kernel(MaskSlice m, int32_t *__restrict__ vmap,
                                                             int32_t *__restrict__ tmap,
                                                             int32_t *__restrict__ tnvb) {
  __shared__ int scan[kMaskWords];
  const int i = threadIdx.x;
  const int nb = max(0, min(32, m.n - 32 * i));  // positions held by word i
  const uint32_t w = m.bits[i] & (nb >= 32 ? ~0u : (1u << nb) - 1u);
  const int c = __popc(w);
  // inclusive scan of the per-word vision counts
  scan[i] = c;
  __syncthreads();
  for (int off = 1; off < kMaskWords; off <<= 1) {
    const int x = i >= off ? scan[i - off] : 0;
    __syncthreads();
    scan[i] += x;
    __syncthreads();
  }
  const int64_t vis0 = m.vis_before + scan[i] - c;  // vision tokens before word i
  for (int j = 0; j < nb; ++j) {
    const int64_t pos = m.base + 32 * i + j;
    const int64_t vis = vis0 + __popc(w & ((1u << j) - 1u));
    if ((w >> j) & 1u) {
      vmap[vis] = (int32_t)pos;
    } else {
      const int64_t tr = pos - vis;  // text tokens before pos
      tmap[tr] = (int32_t)pos;
      tnvb[tr] = (int32_t)vis;
    }
  }
}

}  // namespace

__global__ void status_clear_kernel(int32_t *status) { *status = 0; }

hipError_t launch_status_clear(int32_t *status, hipStream_t st) {
  hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(1), 0, st, status);
  return hipGetLastError();
}

hipError_t launch_row_maps(const MaskSlice &m, int32_t *vmap, int32_t *tmap, int32_t *tnvb,
                           hipStream_t st) {
  if (m.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_map_kernel, dim3(1), dim3(kMaskWords), 0, st, m, vmap, tmap, tnvb);
  return hipGetLastError();
}

}  // namespace nsa
