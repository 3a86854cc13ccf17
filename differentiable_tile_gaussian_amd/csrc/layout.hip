// Conversion between the plane-major [P][n] parameter layout and the blocked layout
// the library works in (groups of 64 Gaussians, each group's P planes of 64 floats
// one after another).  One thread per float of the blocked array, so the blocked
// side is streamed contiguously and the planar side in 256-byte rows.
#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kThreads = 256;

template <bool TO_BLOCKED>
__global__ void __launch_bounds__(kThreads) convert_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                            int n, int P, uint32_t count) {
  const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= count) return;
  const uint32_t group = e / uint32_t(P * kGB), r = e % uint32_t(P * kGB);
  const int p = int(r / kGB);
  const int i = int(group) * kGB + int(r % kGB);
  const size_t planar = size_t(p) * n + i;
  if (TO_BLOCKED)
    dst[e] = i < n ? src[planar] : 0.0f;
  else if (i < n)
    dst[planar] = src[e];
}

}  // namespace

hipError_t launch_to_blocked(const float* planar, float* blocked, int n, int P, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t count = uint32_t(param_floats(n, P));
  GSK_PROF("to_blocked", s);
  convert_kernel<true><<<div_up(count, kThreads), kThreads, 0, s>>>(planar, blocked, n, P, count);
  return hipGetLastError();
}

hipError_t launch_from_blocked(const float* blocked, float* planar, int n, int P, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t count = uint32_t(param_floats(n, P));
  GSK_PROF("from_blocked", s);
  convert_kernel<false><<<div_up(count, kThreads), kThreads, 0, s>>>(blocked, planar, n, P, count);
  return hipGetLastError();
}

}  // namespace gsk
