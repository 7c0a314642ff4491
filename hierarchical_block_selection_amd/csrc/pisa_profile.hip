// Opt-in per-launch timing: when enabled, every kernel launch of the library
// is bracketed by two HIP events recorded on the launch stream; a report
// waits for the events and aggregates elapsed time per kernel name.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pisa.h"
#include "pisa_launch.h"

namespace pisa {
namespace prof {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

Scope::Scope(const char* name, hipStream_t st) : name_(name), st_(st), start_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, st_) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

Scope::~Scope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (stop && hipEventRecord(stop, st_) == hipSuccess) {
    g_records.push_back({name_, start_, stop});
  } else {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
  }
}

}  // namespace prof
}  // namespace pisa

extern "C" {

int pisa_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(pisa::prof::g_mu);
  pisa::prof::g_on = enable != 0;
  return PISA_OK;
}

int pisa_profile_report(char* names, size_t names_len, float* total_ms, int32_t* counts,
                        int32_t max_kernels, int32_t* n_kernels) {
  if (!n_kernels || (max_kernels > 0 && (!total_ms || !counts))) return PISA_ERR_INVALID;
  std::vector<pisa::prof::Record> recs;
  {
    std::lock_guard<std::mutex> lk(pisa::prof::g_mu);
    recs.swap(pisa::prof::g_records);
  }
  std::vector<std::string> keys;
  std::vector<double> tot;
  std::vector<int> cnt;
  int status = PISA_OK;
  for (const auto& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = PISA_ERR_HIP;
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) ++i;
    if (i == keys.size()) {
      keys.emplace_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
  }
  {
    std::lock_guard<std::mutex> lk(pisa::prof::g_mu);
    for (const auto& r : recs) {
      pisa::prof::g_pool.push_back(r.start);
      pisa::prof::g_pool.push_back(r.stop);
    }
  }
  *n_kernels = (int32_t)keys.size();
  std::string joined;
  for (size_t i = 0; i < keys.size() && (int32_t)i < max_kernels; ++i) {
    total_ms[i] = (float)tot[i];
    counts[i] = cnt[i];
    joined += keys[i];
    joined += '\n';
  }
  if (names && names_len > 0) {
    const size_t n = joined.size() < names_len - 1 ? joined.size() : names_len - 1;
    memcpy(names, joined.data(), n);
    names[n] = '\0';
  }
  return status;
}

}  // extern "C"
