// Decode step: one query per sequence at the last slot of its vision cache.
#include "../../include/nsa.h"
#include "nsa_kernels.h"

namespace nsa {
bool decode_supported(int d, int G) { return (d == 64 || d == 128) && G >= 1 && G <= 8; }
hipError_t launch_decode(const DecodeParams &, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace nsa

extern "C" {
nsa_status nsa_decode_workspace_size(const nsa_decode_desc *desc, size_t *bytes) {
  if (!desc || !bytes) return NSA_ERR_INVALID_ARG;
  return NSA_ERR_UNSUPPORTED;
}
nsa_status nsa_decode(const nsa_decode_desc *desc, const void *, const void *, const void *,
                      const void *, const void *, const float *, float *, int32_t *, float *,
                      void *, size_t, void *) {
  if (!desc) return NSA_ERR_INVALID_ARG;
  return NSA_ERR_UNSUPPORTED;
}
}
