// Tile blend kernels: front-to-back forward and back-to-front backward.
//
// One 256-thread block per 16x16 tile, one thread per pixel; blocks take the
// tiles longest list first (a one-block bucket sort by log2 of the list length)
// so that the long lists start at once and the short ones fill in behind them.
// A tile's sorted pair list is walked in batches of 256: the block gathers the
// batch's records into LDS (double-buffered: the next batch's global gather is
// issued before the current batch is blended), then every pixel reads them as
// wave-wide broadcasts.
//
// The per-entry arithmetic is branch-free.  A pair that is skipped (alpha below
// 1/255) or that comes after the pixel stopped is blended with alpha = 0, which
// leaves T and the colour unchanged bit for bit, so the result is the one of the
// sequential walk with `continue` and `break`.  Waves leave the batch loop as soon
// as all their pixels have stopped.
//
// The conic is prescaled when staged: q = a' dx^2 + b' dx dy + c' dy^2 with
// (a', b', c') = -log2(e) (A/2, B, C/2), so the Gaussian factor exp(-e) is one exp2.
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
constexpr float kLog2e = 1.44269504088896341f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- tile order
// Tiles sorted by bucket 32 - clz(length), longest bucket first (order within a
// bucket is arbitrary).  One block; num_tiles may exceed the block size.
__global__ void __launch_bounds__(1024) tile_order_kernel(const uint32_t* __restrict__ ranges, int num_tiles,
                                                           uint32_t* __restrict__ order) {
  __shared__ uint32_t s_cnt[33];
  __shared__ uint32_t s_pos[33];
  if (threadIdx.x < 33) s_cnt[threadIdx.x] = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t < num_tiles; t += blockDim.x) {
    const uint32_t len = ranges[num_tiles + t] - ranges[t];
    const int b = len ? 32 - __clz(len) : 0;
    atomicAdd(&s_cnt[b], 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int b = 32; b >= 0; --b) {
      s_pos[b] = acc;
      acc += s_cnt[b];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < num_tiles; t += blockDim.x) {
    const uint32_t len = ranges[num_tiles + t] - ranges[t];
    const int b = len ? 32 - __clz(len) : 0;
    order[atomicAdd(&s_pos[b], 1u)] = uint32_t(t);
  }
}

// Record as staged in LDS for the forward: (u, v, a', b'), (c', opacity, r, g), b.
__device__ inline void stage_fwd(const float4* __restrict__ splat, uint32_t g, float4& a, float4& b, float& c) {
  const float4 r0 = splat[3 * g], r1 = splat[3 * g + 1];
  c = splat[3 * g + 2].x;
  a = make_float4(r0.x, r0.y, -0.5f * kLog2e * r0.z, -kLog2e * r0.w);
  b = make_float4(-0.5f * kLog2e * r1.x, r1.y, r1.z, r1.w);
}

__global__ void __launch_bounds__(256) render_fwd_kernel(const float4* __restrict__ splat,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ ranges,
                                                          const uint32_t* __restrict__ order, int num_tiles, int tx,
                                                          int W, int H, float bg0, float bg1, float bg2,
                                                          float* __restrict__ rgb, float* __restrict__ T_final,
                                                          uint32_t* __restrict__ n_contrib) {
  __shared__ float4 s_a[2][kBatch];
  __shared__ float4 s_b[2][kBatch];
  __shared__ float s_c[2][kBatch];
  const int tile = int(order[blockIdx.x]);
  const int tid = threadIdx.x;
  const int px = (tile % tx) * kTile + (tid & (kTile - 1));
  const int py = (tile / tx) * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fx = float(px) + 0.5f, fy = float(py) + 0.5f;
  const uint32_t start = ranges[tile];
  const int n = int(ranges[num_tiles + tile] - start);
  float T = 1.0f, c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
  uint32_t last = 0;
  bool done = !inside;
  if (n > 0) {
    {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      float c = 0.f;
      if (tid < n) stage_fwd(splat, vals[start + tid], a, b, c);
      s_a[0][tid] = a; s_b[0][tid] = b; s_c[0][tid] = c;
    }
    __syncthreads();
    int buf = 0;
    for (int base = 0; base < n; base += kBatch) {
      // gather the next batch while this one is blended (zero records pad the tail: opacity 0)
      const int nxt = base + kBatch + tid;
      float4 na = make_float4(0.f, 0.f, 0.f, 0.f), nb = na;
      float nc = 0.f;
      if (nxt < n) stage_fwd(splat, vals[start + nxt], na, nb, nc);
      const int cnt = min(kBatch, n - base);
      if (!__all(done)) {
        for (int j = 0; j < cnt; j += 4) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 a = s_a[buf][j + k];
            const float4 b = s_b[buf][j + k];
            const float cb = s_c[buf][j + k];
            const float dx = fx - a.x, dy = fy - a.y;
            const float q = a.z * dx * dx + a.w * dx * dy + b.x * dy * dy;
            float alpha = fminf(kAlphaCap, b.y * fast_exp2(q));
            const bool ok = !done && alpha >= kAlphaMin;
            alpha = ok ? alpha : 0.0f;
            const float w = alpha * T;
            c0 += w * b.z;
            c1 += w * b.w;
            c2 += w * cb;
            T = T * (1.0f - alpha);
            last = ok ? uint32_t(base + j + k + 1) : last;
            done = done || (T < kTStop);
          }
          if (__all(done)) break;
        }
      }
      if (base + kBatch < n) {
        s_a[buf ^ 1][tid] = na; s_b[buf ^ 1][tid] = nb; s_c[buf ^ 1][tid] = nc;
      }
      if (__syncthreads_count(done) == kBatch) break;
      buf ^= 1;
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

// Record as staged in LDS for the backward: (u, v, a', b'), (c', opacity, r, g), (b, A, B, C).
__device__ inline void stage_bwd(const float4* __restrict__ splat, uint32_t g, float4& a, float4& b, float4& c) {
  const float4 r0 = splat[3 * g], r1 = splat[3 * g + 1], r2 = splat[3 * g + 2];
  a = make_float4(r0.x, r0.y, -0.5f * kLog2e * r0.z, -kLog2e * r0.w);
  b = make_float4(-0.5f * kLog2e * r1.x, r1.y, r1.z, r1.w);
  c = make_float4(r2.x, r0.z, r0.w, r1.x);
}

__global__ void __launch_bounds__(256) render_bwd_kernel(const float4* __restrict__ splat,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ ranges,
                                                          const uint32_t* __restrict__ order, int num_tiles, int tx,
                                                          int W, int H, float bg0, float bg1, float bg2,
                                                          const float* __restrict__ T_final,
                                                          const uint32_t* __restrict__ n_contrib,
                                                          const float* __restrict__ dL_dimg, int n,
                                                          float* __restrict__ gscreen) {
  __shared__ float4 s_a[2][kBatch];
  __shared__ float4 s_b[2][kBatch];
  __shared__ float4 s_c[2][kBatch];
  __shared__ uint32_t s_id[2][kBatch];
  __shared__ float s_acc[9][kBatch];     // per-entry sums over the block's four waves
  __shared__ uint32_t s_max;
  const int tile = int(order[blockIdx.x]);
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
#pragma unroll
  for (int k = 0; k < 9; ++k) s_acc[k][tid] = 0.0f;
  __syncthreads();
  if (nc > 0) atomicMax(&s_max, nc);
  // largest n_contrib of this wave: entries at or beyond it need no work from this wave
  uint32_t wave_max = nc;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) wave_max = max(wave_max, uint32_t(__shfl_xor(int(wave_max), d, 64)));
  __syncthreads();
  const int max_nc = int(s_max);
  if (max_nc == 0) return;
  // batch k covers local entries [hi - 256, hi), walked from hi - 1 down
  int hi = max_nc;
  {
    const int lo = max(hi - kBatch, 0);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a, c = a;
    uint32_t g = 0;
    if (lo + tid < hi) {
      g = vals[start + uint32_t(lo + tid)];
      stage_bwd(splat, g, a, b, c);
    }
    s_a[0][tid] = a; s_b[0][tid] = b; s_c[0][tid] = c; s_id[0][tid] = g;
  }
  __syncthreads();
  int buf = 0;
  while (hi > 0) {
    const int lo = max(hi - kBatch, 0);
    // gather the next (earlier) batch
    const int nhi = lo, nlo = max(nhi - kBatch, 0);
    float4 na = make_float4(0.f, 0.f, 0.f, 0.f), nb = na, ncr = na;
    uint32_t ng = 0;
    if (nlo + tid < nhi) {
      ng = vals[start + uint32_t(nlo + tid)];
      stage_bwd(splat, ng, na, nb, ncr);
    }
    const int jtop = min(hi, int(wave_max)) - 1;
    for (int j = jtop; j >= lo; --j) {
      const int e = j - lo;
      const float4 a = s_a[buf][e];
      const float4 b = s_b[buf][e];
      const float4 c = s_c[buf][e];
      const float dx = fx - a.x, dy = fy - a.y;
      const float q = a.z * dx * dx + a.w * dx * dy + b.x * dy * dy;
      const float G = fast_exp2(q);
      const float araw = b.y * G;
      const float alpha = fminf(kAlphaCap, araw);
      const bool ok = uint32_t(j) < nc && alpha >= kAlphaMin;
      if (__ballot(ok) == 0) continue;
      float v[9];
      const float inv = __builtin_amdgcn_rcpf(1.0f - alpha);
      const float Tn = T * inv;           // transmittance in front of this entry
      const float w = alpha * Tn;
      const float galpha = g0 * (b.z * Tn - S0 * inv) + g1 * (b.w * Tn - S1 * inv) + g2 * (c.x * Tn - S2 * inv);
      const bool unc = ok && araw <= kAlphaCap;
      const float ge = unc ? -galpha * araw : 0.0f;
      v[0] = -ge * (c.y * dx + c.z * dy);
      v[1] = -ge * (c.z * dx + c.w * dy);
      v[2] = ge * 0.5f * dx * dx;
      v[3] = ge * dx * dy;
      v[4] = ge * 0.5f * dy * dy;
      v[5] = unc ? galpha * G : 0.0f;
      v[6] = ok ? g0 * w : 0.0f;
      v[7] = ok ? g1 * w : 0.0f;
      v[8] = ok ? g2 * w : 0.0f;
      if (ok) {
        S0 += b.z * w;
        S1 += b.w * w;
        S2 += c.x * w;
        T = Tn;
      }
      wave_sum9(v);
      if ((lane & 7) == 0) atomicAdd(&s_acc[lane >> 3][e], v[0]);
      if (lane == 0) atomicAdd(&s_acc[8][e], v[8]);
    }
    if (nlo < nhi) {
      s_a[buf ^ 1][tid] = na; s_b[buf ^ 1][tid] = nb; s_c[buf ^ 1][tid] = ncr; s_id[buf ^ 1][tid] = ng;
    }
    __syncthreads();
    // one set of global atomics per (tile, Gaussian)
    if (tid < hi - lo) {
      const uint32_t g = s_id[buf][tid];
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const float val = s_acc[k][tid];
        if (val != 0.0f) atomicAdd(&gscreen[k * n + g], val);
        s_acc[k][tid] = 0.0f;
      }
    }
    __syncthreads();
    hi = lo;
    buf ^= 1;
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t count) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

}  // namespace

size_t render_ws_bytes(int W, int H) { return size_t((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile) * 4 + 256; }

hipError_t launch_render_fwd(const gs_proj& proj, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, float* rgb, float* T_final, uint32_t* n_contrib, void* ws,
                             hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  uint32_t* order = static_cast<uint32_t*>(ws);
  tile_order_kernel<<<1, 1024, 0, s>>>(ranges, num_tiles, order);
  render_fwd_kernel<<<num_tiles, 256, 0, s>>>(reinterpret_cast<const float4*>(proj.splat), vals, ranges, order,
                                              num_tiles, tx, cam.width, cam.height, cam.bg[0], cam.bg[1], cam.bg[2],
                                              rgb, T_final, n_contrib);
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_proj& proj, int n, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, const float* T_final, const uint32_t* n_contrib,
                             const float* dL_dimg, float* gscreen, void* ws, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  uint32_t* order = static_cast<uint32_t*>(ws);
  if (n > 0) zero_f32_kernel<<<div_up(9 * int64_t(n), 256), 256, 0, s>>>(gscreen, 9 * int64_t(n));
  tile_order_kernel<<<1, 1024, 0, s>>>(ranges, num_tiles, order);
  render_bwd_kernel<<<num_tiles, 256, 0, s>>>(reinterpret_cast<const float4*>(proj.splat), vals, ranges, order,
                                              num_tiles, tx, cam.width, cam.height, cam.bg[0], cam.bg[1], cam.bg[2],
                                              T_final, n_contrib, dL_dimg, n, gscreen);
  return hipGetLastError();
}

}  // namespace gsk
