// Per-Gaussian projection (forward).
//
// This translation unit is compiled with -ffp-contract=off: the key path
// (camera-space depth, screen centre, extent, tile rectangle) must be plain
// IEEE fp32 in the written order so that the pair list is reproducible
// bit for bit.  exp, log and the sigmoid on that path are evaluated in fp64
// and rounded once.  Division and square root are the correctly rounded fp32
// operations (the HIP default).
//
// One thread per Gaussian; each parameter plane of a group of 64 Gaussians is one
// contiguous 256-byte row of the blocked layout, read by one wave.
//
// Pages (titles as they appear on the pages):
//   [DR]  "Differentiable rasterisation";  [GST] Gaussian splatting training study deck;
//   [GSG] "How a computer rebuilds a real place out of soft colored dots called Gaussian Splats".
#include "projection.h"
#include "profile.h"

namespace gsk {
namespace {

using namespace proj;

template <int DEG>
__global__ void __launch_bounds__(256) preprocess_fwd_kernel(const float* __restrict__ params, int n,
                                                              gs_camera cam, int tx, int ty, float4* __restrict__ splat,
                                                              float* __restrict__ depth, uint2* __restrict__ rect,
                                                              uint32_t* __restrict__ tiles) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  constexpr int P = 11 + 3 * (K + 1);
  const float* g0 = gaussian_base(params, i, P);
  Proj g;
  bool vis = project_geometry(g0, cam, g);
  float rgb[3] = {0.f, 0.f, 0.f};
  uint32_t x0 = 0, y0 = 0, x1 = 0, y1 = 0, cnt = 0;
  if (vis) {
    float Y[16];
    if (K > 0) {
      float dir[3];
      view_dir(g0, cam, dir);
      sh_eval(dir[0], dir[1], dir[2], Y);
    }
    float raw[3];
    sh_colour(g0, K, Y, raw);
    bool finite = __builtin_isfinite(g.u) && __builtin_isfinite(g.v) && __builtin_isfinite(g.A) &&
                  __builtin_isfinite(g.B) && __builtin_isfinite(g.C) && __builtin_isfinite(g.o);
    for (int ch = 0; ch < 3; ++ch) {
      rgb[ch] = fmaxf(raw[ch], 0.0f);
      finite = finite && __builtin_isfinite(rgb[ch]);
    }
    vis = finite;
    if (vis) {
      // opacity-aware extent ([GSG] "Why tiling"): rad = sqrt(2 eMax) sqrt(lambda_max)
      const float mid = 0.5f * (g.a + g.c);
      const float disc = sqrtf(fmaxf(mid * mid - g.det, 0.0f));
      const float lmax = mid + disc;
      const float emax = float(fmin(4.5, log(fmax(double(g.o) * 255.0, 1.0001))));
      const float rad = sqrtf(2.0f * emax) * sqrtf(lmax);
      vis = __builtin_isfinite(rad);
      if (vis) {
        const float fx0 = floorf((g.u - rad) / 16.0f), fx1 = floorf((g.u + rad) / 16.0f);
        const float fy0 = floorf((g.v - rad) / 16.0f), fy1 = floorf((g.v + rad) / 16.0f);
        if (fx1 < 0.0f || fx0 > float(tx - 1) || fy1 < 0.0f || fy0 > float(ty - 1)) {
          vis = false;
        } else {
          x0 = uint32_t(fmaxf(fx0, 0.0f));
          y0 = uint32_t(fmaxf(fy0, 0.0f));
          x1 = uint32_t(fminf(fx1, float(tx - 1)));
          y1 = uint32_t(fminf(fy1, float(ty - 1)));
          cnt = (x1 - x0 + 1) * (y1 - y0 + 1);
        }
      }
    }
  }
  if (vis) {
    splat[3 * i + 0] = make_float4(g.u, g.v, g.A, g.B);
    splat[3 * i + 1] = make_float4(g.C, g.o, rgb[0], rgb[1]);
    splat[3 * i + 2] = make_float4(rgb[2], 0.f, 0.f, 0.f);
    depth[i] = g.p[2];
    rect[i] = make_uint2(x0 | (y0 << 16), x1 | (y1 << 16));
    tiles[i] = cnt;
  } else {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    splat[3 * i + 0] = z;
    splat[3 * i + 1] = z;
    splat[3 * i + 2] = z;
    depth[i] = 0.0f;
    rect[i] = make_uint2(0u, 0u);
    tiles[i] = 0u;
  }
}

}  // namespace

hipError_t launch_preprocess_fwd(const float* params, int n, int deg, const gs_camera& cam, const gs_proj& out,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(div_up(n, 256)), block(256);
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  float4* splat = reinterpret_cast<float4*>(out.splat);
  uint2* rect = reinterpret_cast<uint2*>(out.rect);
  GSK_PROF("preprocess_fwd", s);
  switch (deg) {
    case 0: preprocess_fwd_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    case 1: preprocess_fwd_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    case 2: preprocess_fwd_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    default: preprocess_fwd_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
  }
  return hipGetLastError();
}

}  // namespace gsk
