// Scoped launch timer used by the host code (see nsa_timing.hip).
#pragma once
#include <hip/hip_runtime.h>

namespace nsa {
class Timed {
 public:
  Timed(const char *name, hipStream_t s);
  ~Timed();
  Timed(const Timed &) = delete;
  Timed &operator=(const Timed &) = delete;

 private:
  const char *name_;
  hipStream_t stream_;
  void *start_;
};
}  // namespace nsa
