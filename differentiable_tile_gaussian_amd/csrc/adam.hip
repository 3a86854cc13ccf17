// Fused Adam over every parameter plane ([GSG] Adam section of "How a computer
// rebuilds a real place out of soft colored dots called Gaussian Splats"; per-group
// learning rates, [DR] "From a pixel error back to a quaternion").
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// Streaming: 16 bytes read and 12 written per parameter; one block row per plane so the
// group's rate is uniform per block; float4 accesses when the plane length allows.
#include "gs_internal.h"

namespace gsk {
namespace {

struct Rates { float lr[5]; };

__device__ inline int plane_group(int plane) {
  return plane < 3 ? 0 : plane < 6 ? 1 : plane < 10 ? 2 : plane == 10 ? 3 : 4;
}

struct Hyper { float b1, b2, omb1, omb2, eps, inv_bc1, inv_bc2; };

__device__ inline float adam_one(float& th, float g, float& m, float& v, float lr, const Hyper& h) {
  m = h.b1 * m + h.omb1 * g;
  v = h.b2 * v + h.omb2 * g * g;
  const float inv_bc1 = h.inv_bc1, inv_bc2 = h.inv_bc2, eps = h.eps;
  const float mh = m * inv_bc1, vh = v * inv_bc2;
  th = th - lr * mh / (sqrtf(vh) + eps);
  return th;
}

__global__ void __launch_bounds__(256) adam_vec4_kernel(float4* __restrict__ params, const float4* __restrict__ grads,
                                                         float4* __restrict__ m, float4* __restrict__ v, int n4,
                                                         Rates rates, Hyper h) {
  const int plane = blockIdx.y;
  const float lr = rates.lr[plane_group(plane)];
  const size_t base = size_t(plane) * n4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    const size_t k = base + i;
    float4 th = params[k], gg = grads[k], mm = m[k], vv = v[k];
    adam_one(th.x, gg.x, mm.x, vv.x, lr, h);
    adam_one(th.y, gg.y, mm.y, vv.y, lr, h);
    adam_one(th.z, gg.z, mm.z, vv.z, lr, h);
    adam_one(th.w, gg.w, mm.w, vv.w, lr, h);
    params[k] = th;
    m[k] = mm;
    v[k] = vv;
  }
}

__global__ void __launch_bounds__(256) adam_scalar_kernel(float* __restrict__ params, const float* __restrict__ grads,
                                                           float* __restrict__ m, float* __restrict__ v, int n,
                                                           Rates rates, Hyper h) {
  const int plane = blockIdx.y;
  const float lr = rates.lr[plane_group(plane)];
  const size_t base = size_t(plane) * n;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const size_t k = base + i;
    float th = params[k], mm = m[k], vv = v[k];
    adam_one(th, grads[k], mm, vv, lr, h);
    params[k] = th;
    m[k] = mm;
    v[k] = vv;
  }
}

}  // namespace

hipError_t launch_adam(float* params, const float* grads, float* m, float* v, int n, int deg, const float lr[5],
                       float b1, float b2, float omb1, float omb2, float eps, float inv_bc1, float inv_bc2,
                       hipStream_t s) {
  if (n == 0) return hipSuccess;
  const Hyper h{b1, b2, omb1, omb2, eps, inv_bc1, inv_bc2};
  Rates r;
  for (int k = 0; k < 5; ++k) r.lr[k] = lr[k];
  const int P = num_planes(deg);
  const bool aligned = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(params) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(grads) % 16) == 0 && (reinterpret_cast<uintptr_t>(m) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(v) % 16) == 0;
  if (aligned) {
    const int n4 = n / 4;
    const unsigned bx = div_up(n4, 256) < 64u ? div_up(n4, 256) : 64u;
    adam_vec4_kernel<<<dim3(bx, P), 256, 0, s>>>(reinterpret_cast<float4*>(params),
                                                 reinterpret_cast<const float4*>(grads),
                                                 reinterpret_cast<float4*>(m), reinterpret_cast<float4*>(v), n4, r, h);
  } else {
    const unsigned bx = div_up(n, 256) < 256u ? div_up(n, 256) : 256u;
    adam_scalar_kernel<<<dim3(bx, P), 256, 0, s>>>(params, grads, m, v, n, r, h);
  }
  return hipGetLastError();
}

}  // namespace gsk
