// Adam update of one parameter, shared by the standalone Adam kernel (adam.hip)
// and the backward chain with Adam fused in (chain.hip).  [GSG] Adam section of
// "How a computer rebuilds a real place out of soft colored dots called Gaussian
// Splats"; per-group rates, [DR] "From a pixel error back to a quaternion".
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// 1 - beta and the bias corrections are formed in fp64 on the host.  The square root
// and the reciprocal are the hardware's (about one ulp each) rather than correctly
// rounded sequences: the update carries a relative error of a few ulp of the step,
// and the chain pass it runs in issues fewer VALU instructions (1.61 -> 1.59 ms).
#pragma once

#include "gs_internal.h"

namespace gsk {

struct AdamArgs {
  float lr[5];          // means, log-scales, quaternion, opacity, colour
  float b1, b2, omb1, omb2, eps, inv_bc1, inv_bc2;
};

__device__ inline int adam_group(int plane) {
  return plane < 3 ? 0 : plane < 6 ? 1 : plane < 10 ? 2 : plane == 10 ? 3 : 4;
}

__device__ inline float adam_update(float th, float g, float& m, float& v, float lr, const AdamArgs& a) {
  m = a.b1 * m + a.omb1 * g;
  v = a.b2 * v + a.omb2 * g * g;
  const float mh = m * a.inv_bc1, vh = v * a.inv_bc2;
  return th - lr * mh * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vh) + a.eps);
}

}  // namespace gsk
