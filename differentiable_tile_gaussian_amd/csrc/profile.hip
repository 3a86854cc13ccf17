// Per-kernel timing records behind gs_profile_enable / gs_profile_query.
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

struct Rec {
  std::string name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::string g_only;               // record only this kernel name when non-empty
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;   // events to reuse

}  // namespace

bool profile_on() { return g_on; }

bool profile_wants(const char* name) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on && (g_only.empty() || g_only == name);
}

hipEvent_t profile_event() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void profile_record(const char* name, hipEvent_t a, hipEvent_t b) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{name, a, b});
}

hipError_t profile_enable(bool on, const char* only) {
  std::lock_guard<std::mutex> lk(g_mu);
  hipError_t first = hipSuccess;
  for (auto& r : g_recs) {
    const hipError_t e = hipEventSynchronize(r.b);
    if (first == hipSuccess) first = e;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_only = only ? only : "";
  g_on = on;
  return first;
}

hipError_t profile_query(int32_t max_names, char* names, int64_t* launches, double* total_ms, int32_t* written) {
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<std::string> keys;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  for (auto& r : g_recs) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return e;
    size_t k = 0;
    while (k < keys.size() && keys[k] != r.name) ++k;
    if (k == keys.size()) {
      keys.push_back(r.name);
      cnt.push_back(0);
      ms.push_back(0.0);
    }
    cnt[k] += 1;
    ms[k] += double(t);
  }
  const int32_t out = int32_t(keys.size()) < max_names ? int32_t(keys.size()) : max_names;
  for (int32_t k = 0; k < out; ++k) {
    snprintf(names + 64 * k, 64, "%s", keys[k].c_str());
    launches[k] = cnt[k];
    total_ms[k] = ms[k];
  }
  *written = out;
  return hipSuccess;
}

}  // namespace gsk
