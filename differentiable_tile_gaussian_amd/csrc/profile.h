// Optional per-kernel timing: when enabled (gs_profile_enable), each kernel launch
// that a library call makes (or only those of one kernel name) is bracketed by two
// HIP events recorded on the launch stream; gs_profile_query sums the elapsed times
// per kernel name.  Off by default, and then a launch costs one branch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gsk {

bool profile_on();
bool profile_wants(const char* name);
void profile_record(const char* name, hipEvent_t start, hipEvent_t stop);
hipEvent_t profile_event();
// Drops the held records (after waiting for them) and switches recording on or off.
hipError_t profile_enable(bool on, const char* only);
// Per kernel name in first-seen order: name (64-byte slots), launches, summed ms.
hipError_t profile_query(int32_t max_names, char* names, int64_t* launches, double* total_ms, int32_t* written);

struct ProfScope {
  const char* name;
  hipStream_t stream;
  hipEvent_t a = nullptr;
  ProfScope(const char* n, hipStream_t s) : name(n), stream(s) {
    if (profile_on() && profile_wants(name)) {
      a = profile_event();
      (void)hipEventRecord(a, stream);   // a failed record leaves the launch untimed
    }
  }
  ~ProfScope() {
    if (a) {
      hipEvent_t b = profile_event();
      (void)hipEventRecord(b, stream);
      profile_record(name, a, b);
    }
  }
};

}  // namespace gsk

#define GSK_PROF_CAT2(a, b) a##b
#define GSK_PROF_CAT(a, b) GSK_PROF_CAT2(a, b)
#define GSK_PROF(name, stream) ::gsk::ProfScope GSK_PROF_CAT(gsk_prof_scope_, __LINE__)(name, stream)
