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

// Half-widths of a box around (u, v) outside which no pixel centre can get
// alpha >= 1/255 from this Gaussian, for the blend's per-quadrant skipping.  The
// blend tests o exp(-e) >= 1/255 with e from the fp32 conic (A, B, C), so the box
// bounds the ellipse e <= ln(255 o) of that conic: |dx| <= sqrt(2 t C / (A C - B^2)),
// |dy| <= sqrt(2 t A / (A C - B^2)), evaluated in fp64 from the fp32 conic and widened
// to cover the blend's fp32 evaluation of e: t by 1 % + 0.01 (the widened value is
// returned in tm, for the blend's finer per-quadrant test of e itself), the half-widths
// by 1 % + 0.05 px.  With A C / (A C - B^2) <= 1000 the rounding error of e stays below
// 0.2 % of e (about 0.01 at the box), inside the margin; more elongated conics get an
// unbounded box.  Negative when o < e^-0.001 / 255 (no pixel can reach 1/255);
// infinite (box and tm) when the fp32 conic is not positive definite.
__device__ inline void blend_box(const Proj& g, float& hx, float& hy, float& tm_out) {
  const double t = log(double(g.o) * 255.0);
  if (!(t > -1e-3)) {
    hx = hy = tm_out = -1.0f;
    return;
  }
  const double A = g.A, B = g.B, C = g.C;
  const double det = A * C - B * B;
  if (!(det > 0.0) || !(A > 0.0) || !(C > 0.0) || !(A * C <= 1000.0 * det)) {
    hx = hy = tm_out = __builtin_inff();
    return;
  }
  const double tm = t + 0.01 + 0.01 * fabs(t);
  hx = float(sqrt(2.0 * tm * C / det) * 1.01 + 0.05);
  hy = float(sqrt(2.0 * tm * A / det) * 1.01 + 0.05);
  tm_out = float(tm);
}

// One Gaussian: writes its projected record and returns its tile count.
template <int DEG>
__device__ inline uint32_t project_one(const float* __restrict__ params, int i, const gs_camera& cam, int tx, int ty,
                                       float4* __restrict__ splat, float* __restrict__ depth,
                                       uint2* __restrict__ rect, uint32_t* __restrict__ tiles) {
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
    float hx, hy, tm;
    blend_box(g, hx, hy, tm);
    splat[3 * i + 2] = make_float4(rgb[2], hx, hy, tm);
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
  return vis ? cnt : 0u;
}

template <int DEG>
__global__ void __launch_bounds__(256) preprocess_fwd_kernel(const float* __restrict__ params, int n,
                                                              gs_camera cam, int tx, int ty, float4* __restrict__ splat,
                                                              float* __restrict__ depth, uint2* __restrict__ rect,
                                                              uint32_t* __restrict__ tiles,
                                                              uint32_t* __restrict__ block_tiles,
                                                              uint64_t* __restrict__ total) {
  __shared__ uint32_t s_wave[4];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *total = 0u;   // sum_counts_kernel adds into it after this kernel
  const uint32_t cnt = i < n ? project_one<DEG>(params, i, cam, tx, ty, splat, depth, rect, tiles) : 0u;
  // the block's total of tile counts (the pair count is the sum over blocks)
  uint32_t v = cnt;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (__lane_id() == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) block_tiles[blockIdx.x] = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
}

// Sum of the per-block tile counts: each block adds up 1024 of them and adds its sum
// to *total (zeroed by the projection kernel).
__global__ void __launch_bounds__(1024) sum_counts_kernel(const uint32_t* __restrict__ block_tiles, int nb,
                                                           uint64_t* __restrict__ total) {
  __shared__ uint64_t s_wave[16];
  const int k = blockIdx.x * 1024 + threadIdx.x;
  uint64_t v = k < nb ? block_tiles[k] : 0u;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (__lane_id() == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < 16; ++w) t += s_wave[w];
    atomicAdd(reinterpret_cast<unsigned long long*>(total), static_cast<unsigned long long>(t));
  }
}

}  // namespace

hipError_t launch_preprocess_fwd(const float* params, int n, int deg, const gs_camera& cam, const gs_proj& out,
                                 uint32_t* block_tiles, uint64_t* total_pairs, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(div_up(n, 256)), block(256);
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  float4* splat = reinterpret_cast<float4*>(out.splat);
  uint2* rect = reinterpret_cast<uint2*>(out.rect);
  {
    GSK_PROF("preprocess_fwd", s);
    switch (deg) {
      case 0: preprocess_fwd_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs); break;
      case 1: preprocess_fwd_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs); break;
      case 2: preprocess_fwd_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs); break;
      default: preprocess_fwd_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs); break;
    }
  }
  GSK_PROF("sum_counts", s);
  sum_counts_kernel<<<div_up(grid.x, 1024), 1024, 0, s>>>(block_tiles, int(grid.x), total_pairs);
  return hipGetLastError();
}

}  // namespace gsk
