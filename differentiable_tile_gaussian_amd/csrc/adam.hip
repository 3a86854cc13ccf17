// Fused Adam over every parameter plane ([GSG] Adam section of "How a computer
// rebuilds a real place out of soft colored dots called Gaussian Splats"; per-group
// learning rates, [DR] "From a pixel error back to a quaternion").
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// Streaming, HBM-bound: 16 bytes read and 12 written per parameter.  Each thread
// keeps four independent 16-byte accesses of each of the four streams in flight, and
// the accesses are non-temporal (every byte is touched once per step).
#include "adam_math.h"
#include "profile.h"

namespace gsk {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;


// Arrays in the blocked layout, streamed flat as float4 units: unit q covers
// Gaussians i0 .. i0 + 3 of one plane, with group b = q / (16 P), plane
// p = (q / 16) % P and i0 = 64 b + 4 (q % 16).  Slots of Gaussians i >= n (padding of
// the last group) are neither read nor written.
template <int P>
__global__ void __launch_bounds__(kThreads) adam_vec4_kernel(f4* __restrict__ params, const f4* __restrict__ grads,
                                                              f4* __restrict__ m, f4* __restrict__ v, int n,
                                                              uint32_t units, const AdamArgs h) {
  const uint32_t q0 = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  f4 th[kUnroll], gg[kUnroll], mm[kUnroll], vv[kUnroll];
  int valid[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t q = q0 + u * kThreads;
    const int i0 = int(q / (16u * P)) * kGB + int(q % 16u) * 4;
    valid[u] = q < units ? min(n - i0, 4) : 0;
    if (valid[u] > 0) {
      th[u] = __builtin_nontemporal_load(&params[q]);
      gg[u] = __builtin_nontemporal_load(&grads[q]);
      mm[u] = __builtin_nontemporal_load(&m[q]);
      vv[u] = __builtin_nontemporal_load(&v[q]);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t q = q0 + u * kThreads;
    if (valid[u] > 0) {
      const float lr = h.lr[adam_group(int((q / 16u) % P))];
      f4 t = th[u], mu = mm[u], vu = vv[u];
      float mx = mu.x, my = mu.y, mz = mu.z, mw = mu.w, vx = vu.x, vy = vu.y, vz = vu.z, vw = vu.w;
      t.x = adam_update(t.x, gg[u].x, mx, vx, lr, h);
      t.y = adam_update(t.y, gg[u].y, my, vy, lr, h);
      t.z = adam_update(t.z, gg[u].z, mz, vz, lr, h);
      t.w = adam_update(t.w, gg[u].w, mw, vw, lr, h);
      if (valid[u] == 4) {
        __builtin_nontemporal_store(t, &params[q]);
        __builtin_nontemporal_store(f4{mx, my, mz, mw}, &m[q]);
        __builtin_nontemporal_store(f4{vx, vy, vz, vw}, &v[q]);
      } else {
        // last group: only the first valid[u] lanes hold Gaussians
        float* pt = reinterpret_cast<float*>(&params[q]);
        float* pm = reinterpret_cast<float*>(&m[q]);
        float* pv = reinterpret_cast<float*>(&v[q]);
        const float ts[4] = {t.x, t.y, t.z, t.w}, ms[4] = {mx, my, mz, mw}, vs[4] = {vx, vy, vz, vw};
        for (int e = 0; e < valid[u]; ++e) {
          pt[e] = ts[e];
          pm[e] = ms[e];
          pv[e] = vs[e];
        }
      }
    }
  }
}

// Any alignment: one thread per float of the blocked arrays.
__global__ void __launch_bounds__(kThreads) adam_scalar_kernel(float* __restrict__ params,
                                                                const float* __restrict__ grads,
                                                                float* __restrict__ m, float* __restrict__ v, int n,
                                                                int P, uint32_t count, const AdamArgs h) {
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < count; e += gridDim.x * blockDim.x) {
    const uint32_t r = e % uint32_t(P * kGB);
    const int i = int(e / uint32_t(P * kGB)) * kGB + int(r % kGB);
    if (i >= n) continue;
    float mm = m[e], vv = v[e];
    params[e] = adam_update(params[e], grads[e], mm, vv, h.lr[adam_group(int(r / kGB))], h);
    m[e] = mm;
    v[e] = vv;
  }
}

template <int P>
void launch_vec4(float* params, const float* grads, float* m, float* v, int n, const AdamArgs& h, hipStream_t s) {
  const uint32_t units = uint32_t(param_floats(n, P) / 4);
  GSK_PROF("adam_vec4", s);
  adam_vec4_kernel<P><<<div_up(units, kThreads * kUnroll), kThreads, 0, s>>>(
      reinterpret_cast<f4*>(params), reinterpret_cast<const f4*>(grads), reinterpret_cast<f4*>(m),
      reinterpret_cast<f4*>(v), n, units, h);
}

}  // namespace

hipError_t launch_adam(float* params, const float* grads, float* m, float* v, int n, int deg, const float lr[5],
                       float b1, float b2, float omb1, float omb2, float eps, float inv_bc1, float inv_bc2,
                       hipStream_t s) {
  if (n == 0) return hipSuccess;
  AdamArgs h;
  for (int k = 0; k < 5; ++k) h.lr[k] = lr[k];
  h.b1 = b1; h.b2 = b2; h.omb1 = omb1; h.omb2 = omb2; h.eps = eps; h.inv_bc1 = inv_bc1; h.inv_bc2 = inv_bc2;
  const int P = num_planes(deg);
  const bool aligned = (reinterpret_cast<uintptr_t>(params) % 16) == 0 && (reinterpret_cast<uintptr_t>(grads) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(m) % 16) == 0 && (reinterpret_cast<uintptr_t>(v) % 16) == 0;
  if (aligned) {
    switch (deg) {
      case 0: launch_vec4<14>(params, grads, m, v, n, h, s); break;
      case 1: launch_vec4<23>(params, grads, m, v, n, h, s); break;
      case 2: launch_vec4<38>(params, grads, m, v, n, h, s); break;
      default: launch_vec4<59>(params, grads, m, v, n, h, s); break;
    }
  } else {
    const uint32_t count = uint32_t(param_floats(n, P));
    const unsigned blocks = div_up(count, kThreads) < 4096u ? div_up(count, kThreads) : 4096u;
    GSK_PROF("adam_scalar", s);
    adam_scalar_kernel<<<blocks, kThreads, 0, s>>>(params, grads, m, v, n, P, count, h);
  }
  return hipGetLastError();
}

}  // namespace gsk
