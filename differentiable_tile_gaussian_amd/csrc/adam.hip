// Fused Adam over every parameter plane ([GSG] Adam section of "How a computer
// rebuilds a real place out of soft colored dots called Gaussian Splats"; per-group
// learning rates, [DR] "From a pixel error back to a quaternion").
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// Streaming, HBM-bound: 16 bytes read and 12 written per parameter.  One block row
// per plane (the group's rate is uniform per block); each thread keeps four
// independent 16-byte accesses of each of the four streams in flight, and the
// accesses are non-temporal (every byte is touched once per step).
#include "adam_math.h"
#include "profile.h"

namespace gsk {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;


__global__ void __launch_bounds__(kThreads) adam_vec4_kernel(f4* __restrict__ params, const f4* __restrict__ grads,
                                                              f4* __restrict__ m, f4* __restrict__ v, int n4,
                                                              const AdamArgs h) {
  const int plane = blockIdx.y;
  const float lr = h.lr[adam_group(plane)];
  const size_t base = size_t(plane) * n4;
  const int i0 = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  f4 th[kUnroll], gg[kUnroll], mm[kUnroll], vv[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int i = i0 + u * kThreads;
    if (i < n4) {
      const size_t k = base + i;
      th[u] = __builtin_nontemporal_load(&params[k]);
      gg[u] = __builtin_nontemporal_load(&grads[k]);
      mm[u] = __builtin_nontemporal_load(&m[k]);
      vv[u] = __builtin_nontemporal_load(&v[k]);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int i = i0 + u * kThreads;
    if (i < n4) {
      const size_t k = base + i;
      f4 t = th[u], mu = mm[u], vu = vv[u];
      float mx = mu.x, my = mu.y, mz = mu.z, mw = mu.w, vx = vu.x, vy = vu.y, vz = vu.z, vw = vu.w;
      t.x = adam_update(t.x, gg[u].x, mx, vx, lr, h);
      t.y = adam_update(t.y, gg[u].y, my, vy, lr, h);
      t.z = adam_update(t.z, gg[u].z, mz, vz, lr, h);
      t.w = adam_update(t.w, gg[u].w, mw, vw, lr, h);
      mu = f4{mx, my, mz, mw};
      vu = f4{vx, vy, vz, vw};
      __builtin_nontemporal_store(t, &params[k]);
      __builtin_nontemporal_store(mu, &m[k]);
      __builtin_nontemporal_store(vu, &v[k]);
    }
  }
}

__global__ void __launch_bounds__(kThreads) adam_scalar_kernel(float* __restrict__ params,
                                                                const float* __restrict__ grads,
                                                                float* __restrict__ m, float* __restrict__ v, int n,
                                                                const AdamArgs h) {
  const int plane = blockIdx.y;
  const float lr = h.lr[adam_group(plane)];
  const size_t base = size_t(plane) * n;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const size_t k = base + i;
    float mm = m[k], vv = v[k];
    params[k] = adam_update(params[k], grads[k], mm, vv, lr, h);
    m[k] = mm;
    v[k] = vv;
  }
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
  const bool aligned = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(params) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(grads) % 16) == 0 && (reinterpret_cast<uintptr_t>(m) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(v) % 16) == 0;
  if (aligned) {
    const int n4 = n / 4;
    {
      GSK_PROF("adam_vec4", s);
      adam_vec4_kernel<<<dim3(div_up(n4, kThreads * kUnroll), P), kThreads, 0, s>>>(
          reinterpret_cast<f4*>(params), reinterpret_cast<const f4*>(grads), reinterpret_cast<f4*>(m),
          reinterpret_cast<f4*>(v), n4, h);
    }
  } else {
    const unsigned bx = div_up(n, 256) < 256u ? div_up(n, 256) : 256u;
    {
      GSK_PROF("adam_scalar", s);
      adam_scalar_kernel<<<dim3(bx, P), kThreads, 0, s>>>(params, grads, m, v, n, h);
    }
  }
  return hipGetLastError();
}

}  // namespace gsk
