// Opt-in per-launch timing for benchmarks: while enabled, every kernel the
// library launches is bracketed by a pair of HIP events recorded on the
// launch stream; nsa_timing_read() folds completed pairs into per-kernel
// totals (the caller synchronises its streams first).
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/nsa.h"
#include "nsa_timing.h"

namespace nsa {
namespace {

struct Pending {
  std::string name;
  hipEvent_t a, b;
};

struct Registry {
  std::mutex mu;
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<double, int>> acc;
  std::vector<std::string> names;  // stable storage for nsa_timing_read

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Registry &reg() {
  static Registry r;
  return r;
}

}  // namespace

Timed::Timed(const char *name, hipStream_t s) : name_(name), stream_(s), start_(nullptr) {
  Registry &r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  if (!r.on) return;
  start_ = r.get();
  if (start_) hipEventRecord(static_cast<hipEvent_t>(start_), s);
}

Timed::~Timed() {
  if (!start_) return;
  Registry &r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  hipEvent_t stop = r.get();
  if (!stop) return;
  hipEventRecord(stop, stream_);
  r.pending.push_back({name_, static_cast<hipEvent_t>(start_), stop});
}

}  // namespace nsa

using namespace nsa;

extern "C" {

nsa_status nsa_timing_enable(int enable) {
  Registry &r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  r.on = enable != 0;
  return NSA_OK;
}

nsa_status nsa_timing_reset(void) {
  Registry &r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  for (auto &p : r.pending) {
    hipEventSynchronize(p.b);
    r.pool.push_back(p.a);
    r.pool.push_back(p.b);
  }
  r.pending.clear();
  r.acc.clear();
  return NSA_OK;
}

int nsa_timing_read(int max_entries, const char **names, double *total_ms, int *counts) {
  Registry &r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  for (auto &p : r.pending) {
    float ms = 0.f;
    hipEventSynchronize(p.b);
    if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto &a = r.acc[p.name];
      a.first += ms;
      a.second += 1;
    }
    r.pool.push_back(p.a);
    r.pool.push_back(p.b);
  }
  r.pending.clear();
  r.names.clear();
  for (auto &kv : r.acc) r.names.push_back(kv.first);
  int i = 0;
  for (auto &kv : r.acc) {
    if (i >= max_entries) break;
    if (names) names[i] = r.names[i].c_str();
    if (total_ms) total_ms[i] = kv.second.first;
    if (counts) counts[i] = kv.second.second;
    ++i;
  }
  return (int)r.acc.size();
}

}  // extern "C"
