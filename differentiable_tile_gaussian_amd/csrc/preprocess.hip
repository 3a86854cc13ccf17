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

// One Gaussian: writes its projected record and returns its tile count.
template <int DEG>
__device__ inline uint32_t project_one(const float* __restrict__ params, int i, const gs_camera& cam, int tx, int ty,
                                       Shade shade, float4* __restrict__ splat, float* __restrict__ depth,
                                       uint2* __restrict__ rect, uint32_t* __restrict__ tiles) {
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  constexpr int P = 11 + 3 * (K + 1);
  const float* g0 = gaussian_base(params, i, P);
  Proj g;
  const bool geom = project_geometry(g0, cam, shade.mip, g);
  float raw[3] = {0.f, 0.f, 0.f};
  if (geom) {
    float Y[16];
    if (K > 0) {
      float dir[3];
      view_dir(g0, cam, dir);
      sh_eval(dir[0], dir[1], dir[2], Y);
    }
    sh_colour<K>(g0, shade.kact, Y, raw);
  }
  Record r;
  make_record(geom, g, raw, tx, ty, r);
  store_record(r, i, splat, depth, rect, tiles);
  return r.tiles;
}

template <int DEG>
__global__ void __launch_bounds__(256) preprocess_fwd_kernel(const float* __restrict__ params, int n,
                                                              gs_camera cam, int tx, int ty, float4* __restrict__ splat,
                                                              float* __restrict__ depth, uint2* __restrict__ rect,
                                                              uint32_t* __restrict__ tiles,
                                                              uint32_t* __restrict__ block_tiles,
                                                              uint64_t* __restrict__ total, Shade shade) {
  __shared__ uint32_t s_wave[4];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *total = 0u;   // sum_counts_kernel adds into it after this kernel
  const uint32_t cnt = i < n ? project_one<DEG>(params, i, cam, tx, ty, shade, splat, depth, rect, tiles) : 0u;
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
                                 uint32_t* block_tiles, uint64_t* total_pairs, Shade shade, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(div_up(n, 256)), block(256);
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  float4* splat = reinterpret_cast<float4*>(out.splat);
  uint2* rect = reinterpret_cast<uint2*>(out.rect);
  {
    GSK_PROF("preprocess_fwd", s);
    switch (deg) {
      case 0: preprocess_fwd_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs, shade); break;
      case 1: preprocess_fwd_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs, shade); break;
      case 2: preprocess_fwd_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs, shade); break;
      default: preprocess_fwd_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles, block_tiles, total_pairs, shade); break;
    }
  }
  return launch_tile_count_total(block_tiles, int(grid.x), total_pairs, s);
}

hipError_t launch_tile_count_total(const uint32_t* block_tiles, int nb, uint64_t* total, hipStream_t s) {
  GSK_PROF("sum_counts", s);
  sum_counts_kernel<<<div_up(nb, 1024), 1024, 0, s>>>(block_tiles, nb, total);
  return hipGetLastError();
}

}  // namespace gsk
