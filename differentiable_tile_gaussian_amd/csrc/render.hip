// Tile blend kernels: front-to-back forward and back-to-front backward.
//
// One 256-thread block per 16x16 tile, one thread per pixel.  The tile's sorted
// pair list is walked in batches of 256: the block gathers the batch's packed
// records (48 bytes each) into LDS once, then every pixel reads them as wave-wide
// broadcasts.
//
// Pages: [GSG] "The painting itself: front-to-back alpha compositing", "The clever
// bit: a single backward sweep through the blend", "From a pixel's blame to the
// oval's shape and place"; [DR] "The trick: recompute the blend state instead of
// storing it"; [GST] opacity slide (cap 0.99, skip below 1/255) and compositing-
// derivative slide.  ([GSG] is "How a computer rebuilds a real place out of soft
// colored dots called Gaussian Splats", [DR] "Differentiable rasterisation",
// [GST] the Gaussian splatting training study deck.)
#include "gs_internal.h"

namespace gsk {
namespace {

constexpr int kBatch = 256;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaCap = 0.99f;
constexpr float kTStop = 1e-4f;

__global__ void __launch_bounds__(256) render_fwd_kernel(const float4* __restrict__ splat,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ ranges, int num_tiles, int tx,
                                                          int W, int H, float bg0, float bg1, float bg2,
                                                          float* __restrict__ rgb, float* __restrict__ T_final,
                                                          uint32_t* __restrict__ n_contrib) {
  __shared__ float4 s_a[kBatch];   // u, v, A, B
  __shared__ float4 s_b[kBatch];   // C, opacity, r, g
  __shared__ float s_c[kBatch];    // b
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int px = (tile % tx) * kTile + (tid & (kTile - 1));
  const int py = (tile / tx) * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fx = float(px) + 0.5f, fy = float(py) + 0.5f;
  const uint32_t start = ranges[tile], end = ranges[num_tiles + tile];
  float T = 1.0f, c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
  uint32_t last = 0;
  bool done = !inside;
  for (uint32_t base = start; base < end; base += kBatch) {
    if (__syncthreads_count(done) == kBatch) break;
    const uint32_t idx = base + tid;
    if (idx < end) {
      const uint32_t g = vals[idx];
      s_a[tid] = splat[3 * g];
      s_b[tid] = splat[3 * g + 1];
      s_c[tid] = splat[3 * g + 2].x;
    }
    __syncthreads();
    const int cnt = int(min(uint32_t(kBatch), end - base));
    if (!done) {
      for (int j = 0; j < cnt; ++j) {
        const float4 a = s_a[j];
        const float4 b = s_b[j];
        const float dx = fx - a.x, dy = fy - a.y;
        const float e = 0.5f * (a.z * dx * dx + b.x * dy * dy) + a.w * dx * dy;
        const float alpha = fminf(kAlphaCap, b.y * __expf(-e));
        if (alpha < kAlphaMin) continue;
        const float w = alpha * T;
        c0 += w * b.z;
        c1 += w * b.w;
        c2 += w * s_c[j];
        T = T * (1.0f - alpha);
        last = base - start + uint32_t(j) + 1;
        if (T < kTStop) {
          done = true;
          break;
        }
      }
    }
  }
  if (inside) {
    const int p = py * W + px;
    const int HW = W * H;
    rgb[p] = c0 + T * bg0;
    rgb[HW + p] = c1 + T * bg1;
    rgb[2 * HW + p] = c2 + T * bg2;
    T_final[p] = T;
    n_contrib[p] = last;
  }
}

// Sum 9 per-lane values over the 64 lanes of a wave.  Values 0..7 use a transposed
// butterfly (each exchange halves the values a lane carries), value 8 a plain one.
// On return lane l holds the total of value (l >> 3) in v[0] and every lane holds
// the total of value 8 in v[8].
__device__ inline void wave_sum9(float* v) {
  const int lane = __lane_id();
  {
    const bool hi = lane & 32;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float send = hi ? v[k] : v[k + 4];
      const float keep = hi ? v[k + 4] : v[k];
      v[k] = keep + __shfl_xor(send, 32, 64);
    }
  }
  {
    const bool hi = lane & 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float send = hi ? v[k] : v[k + 2];
      const float keep = hi ? v[k + 2] : v[k];
      v[k] = keep + __shfl_xor(send, 16, 64);
    }
  }
  {
    const bool hi = lane & 8;
    const float send = hi ? v[0] : v[1];
    const float keep = hi ? v[1] : v[0];
    v[0] = keep + __shfl_xor(send, 8, 64);
  }
  v[0] += __shfl_xor(v[0], 4, 64);
  v[0] += __shfl_xor(v[0], 2, 64);
  v[0] += __shfl_xor(v[0], 1, 64);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v[8] += __shfl_xor(v[8], d, 64);
}

__global__ void __launch_bounds__(256) render_bwd_kernel(const float4* __restrict__ splat,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ ranges, int num_tiles, int tx,
                                                          int W, int H, float bg0, float bg1, float bg2,
                                                          const float* __restrict__ T_final,
                                                          const uint32_t* __restrict__ n_contrib,
                                                          const float* __restrict__ dL_dimg, int n,
                                                          float* __restrict__ gscreen) {
  __shared__ float4 s_a[kBatch];
  __shared__ float4 s_b[kBatch];
  __shared__ float s_c[kBatch];
  __shared__ uint32_t s_id[kBatch];
  __shared__ uint32_t s_max;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int px = (tile % tx) * kTile + (tid & (kTile - 1));
  const int py = (tile / tx) * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fx = float(px) + 0.5f, fy = float(py) + 0.5f;
  const uint32_t start = ranges[tile];
  const int HW = W * H;
  const int p = py * W + px;
  uint32_t nc = 0;
  float T = 0.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
  if (inside) {
    nc = n_contrib[p];
    T = T_final[p];
    g0 = dL_dimg[p];
    g1 = dL_dimg[HW + p];
    g2 = dL_dimg[2 * HW + p];
  }
  float S0 = bg0 * T, S1 = bg1 * T, S2 = bg2 * T;
  if (tid == 0) s_max = 0u;
  __syncthreads();
  if (nc > 0) atomicMax(&s_max, nc);
  __syncthreads();
  const uint32_t max_nc = s_max;
  for (int hi_end = int(max_nc); hi_end > 0; hi_end -= kBatch) {
    const int lo = hi_end > kBatch ? hi_end - kBatch : 0;
    const int cnt = hi_end - lo;
    __syncthreads();
    if (tid < cnt) {
      const uint32_t g = vals[start + uint32_t(lo + tid)];
      s_id[tid] = g;
      s_a[tid] = splat[3 * g];
      s_b[tid] = splat[3 * g + 1];
      s_c[tid] = splat[3 * g + 2].x;
    }
    __syncthreads();
    for (int j = cnt - 1; j >= 0; --j) {
      float v[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) v[k] = 0.0f;
      bool contributed = false;
      if (uint32_t(lo + j) < nc) {
        const float4 a = s_a[j];
        const float4 b = s_b[j];
        const float cb = s_c[j];
        const float dx = fx - a.x, dy = fy - a.y;
        const float e = 0.5f * (a.z * dx * dx + b.x * dy * dy) + a.w * dx * dy;
        const float G = __expf(-e);
        const float araw = b.y * G;
        const float alpha = fminf(kAlphaCap, araw);
        if (alpha >= kAlphaMin) {
          contributed = true;
          const float inv = __builtin_amdgcn_rcpf(1.0f - alpha);
          T = T * inv;                         // transmittance in front of this entry
          const float w = alpha * T;
          v[6] = g0 * w;
          v[7] = g1 * w;
          v[8] = g2 * w;
          const float galpha = g0 * (b.z * T - S0 * inv) + g1 * (b.w * T - S1 * inv) + g2 * (cb * T - S2 * inv);
          S0 += b.z * w;
          S1 += b.w * w;
          S2 += cb * w;
          if (araw <= kAlphaCap) {
            v[5] = galpha * G;
            const float ge = -galpha * araw;
            v[2] = ge * 0.5f * dx * dx;
            v[3] = ge * dx * dy;
            v[4] = ge * 0.5f * dy * dy;
            v[0] = -ge * (a.z * dx + a.w * dy);
            v[1] = -ge * (a.w * dx + b.x * dy);
          }
        }
      }
      if (__ballot(contributed) != 0) {
        wave_sum9(v);
        const uint32_t g = s_id[j];
        if ((lane & 7) == 0) atomicAdd(&gscreen[(lane >> 3) * n + g], v[0]);
        if (lane == 0) atomicAdd(&gscreen[8 * n + g], v[8]);
      }
    }
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t count) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_render_fwd(const gs_proj& proj, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, float* rgb, float* T_final, uint32_t* n_contrib, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  render_fwd_kernel<<<num_tiles, 256, 0, s>>>(reinterpret_cast<const float4*>(proj.splat), vals, ranges, num_tiles,
                                              tx, cam.width, cam.height, cam.bg[0], cam.bg[1], cam.bg[2], rgb,
                                              T_final, n_contrib);
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_proj& proj, int n, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, const float* T_final, const uint32_t* n_contrib,
                             const float* dL_dimg, float* gscreen, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  if (n > 0) zero_f32_kernel<<<div_up(9 * int64_t(n), 256), 256, 0, s>>>(gscreen, 9 * int64_t(n));
  render_bwd_kernel<<<num_tiles, 256, 0, s>>>(reinterpret_cast<const float4*>(proj.splat), vals, ranges, num_tiles,
                                              tx, cam.width, cam.height, cam.bg[0], cam.bg[1], cam.bg[2], T_final,
                                              n_contrib, dL_dimg, n, gscreen);
  return hipGetLastError();
}

}  // namespace gsk
