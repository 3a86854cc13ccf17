// Loss (1 - lambda) L1 + lambda (1 - SSIM) and its image gradient.
//
// [GST] loss slides (Gaussian splatting training study deck): L1 is the mean over
// 3HW with a zero subgradient at zero residual; SSIM uses an 11x11 Gaussian window
// of standard deviation 1.5 (normalised), C1 = 0.01^2, C2 = 0.03^2, zero padding,
// and is averaged over pixels and channels; D-SSIM carries no one-half.
//
// The 2-D window is the outer product of the normalised 1-D window, so the five
// local moments are computed with a horizontal then a vertical 11-tap pass through
// LDS (32x16 output pixels per block, 5-pixel halo).  Each thread makes four
// adjacent outputs of a row in the horizontal pass (14 inputs read once) and two
// adjacent rows of a column in the vertical pass, reusing the taps in registers.
//   ssim_fwd   moments -> SSIM per pixel, the three derivative maps
//                a = dS/dmu_x - 2 mu_x dS/dvar_x - mu_y dS/dcov,  b = dS/dvar_x,  c = dS/dcov,
//              and per-block partial sums of SSIM and |x - y|
//   ssim_bwd   dL/dx = (1-lambda)/N sign(x-y) - lambda/N (w*a + 2 x (w*b) + y (w*c))
//              (w* = the same zero-padded window; it is symmetric, so it is its own adjoint)
//   finalize   sums the partials (fp64) into total, L1, mean SSIM
#include <math.h>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kTW = 32, kTH = 16, kR = 5;
constexpr int kPW = kTW + 2 * kR;   // 42
constexpr int kPH = kTH + 2 * kR;   // 26

struct Window { float w[11]; };

__device__ inline void reduce_block_2(float& a, float& b, float* s_tmp) {
  const int lane = __lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    a += __shfl_xor(a, d, 64);
    b += __shfl_xor(b, d, 64);
  }
  if (lane == 0) {
    s_tmp[2 * wave] = a;
    s_tmp[2 * wave + 1] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = 0.f; b = 0.f;
    for (int w = 0; w < 4; ++w) { a += s_tmp[2 * w]; b += s_tmp[2 * w + 1]; }
  }
}

// Horizontal pass for row r: outputs 4g .. 4g+3 of the 32-wide tile from the 14 inputs
// 4g .. 4g+13 of the 42-wide row (each input read once into registers).
constexpr int kHG = 4;                  // outputs per thread, horizontal
constexpr int kHItems = kPH * (kTW / kHG);   // 208 (row, group) items
constexpr int kVG = 2;                  // outputs per thread, vertical
static_assert((kTW * kTH) / kVG == 256, "one vertical item per thread");

__global__ void __launch_bounds__(256) ssim_fwd_kernel(const float* __restrict__ img, const float* __restrict__ tgt,
                                                        int H, int W, Window win, float* __restrict__ amap,
                                                        float* __restrict__ bmap, float* __restrict__ cmap,
                                                        float* __restrict__ partial) {
  __shared__ float sx[kPH][kPW + 1];
  __shared__ float sy[kPH][kPW + 1];
  __shared__ float4 hs[5][kPH][kTW / 4];   // horizontal sums of x, y, xx, yy, xy
  __shared__ float s_tmp[8];
  const int ch = blockIdx.z;
  const int x0 = blockIdx.x * kTW, y0 = blockIdx.y * kTH;
  const size_t HW = size_t(H) * W;
  const float* X = img + ch * HW;
  const float* Y = tgt + ch * HW;
  for (int k = threadIdx.x; k < kPH * kPW; k += 256) {
    const int r = k / kPW, c = k % kPW;
    const int gy = y0 + r - kR, gx = x0 + c - kR;
    const bool in = gy >= 0 && gy < H && gx >= 0 && gx < W;
    sx[r][c] = in ? X[size_t(gy) * W + gx] : 0.0f;
    sy[r][c] = in ? Y[size_t(gy) * W + gx] : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x < kHItems) {
    const int r = threadIdx.x / (kTW / kHG), g = threadIdx.x % (kTW / kHG);
    float xv[kHG + 10], yv[kHG + 10];
#pragma unroll
    for (int j = 0; j < kHG + 10; ++j) {
      xv[j] = sx[r][kHG * g + j];
      yv[j] = sy[r][kHG * g + j];
    }
    float m[5][kHG];
#pragma unroll
    for (int o = 0; o < kHG; ++o) {
      m[0][o] = m[1][o] = m[2][o] = m[3][o] = m[4][o] = 0.f;
#pragma unroll
      for (int j = 0; j < 11; ++j) {
        const float wj = win.w[j], xj = xv[o + j], yj = yv[o + j];
        m[0][o] += wj * xj;
        m[1][o] += wj * yj;
        m[2][o] += wj * (xj * xj);
        m[3][o] += wj * (yj * yj);
        m[4][o] += wj * (xj * yj);
      }
    }
#pragma unroll
    for (int q = 0; q < 5; ++q) hs[q][r][g] = make_float4(m[q][0], m[q][1], m[q][2], m[q][3]);
  }
  __syncthreads();
  const float C1 = 0.01f * 0.01f, C2 = 0.03f * 0.03f;
  float ssim_acc = 0.f, l1_acc = 0.f;
  {
    // vertical pass: column c, output rows kVG h .. kVG h + 1
    const int c = threadIdx.x % kTW, h = threadIdx.x / kTW;
    const float* hsf = reinterpret_cast<const float*>(hs);
    float v[5][kVG];
#pragma unroll
    for (int o = 0; o < kVG; ++o) v[0][o] = v[1][o] = v[2][o] = v[3][o] = v[4][o] = 0.f;
#pragma unroll
    for (int i = 0; i < kVG + 10; ++i) {
      const int rr = kVG * h + i;
      float t[5];
#pragma unroll
      for (int q = 0; q < 5; ++q) t[q] = hsf[(q * kPH + rr) * kTW + c];
#pragma unroll
      for (int o = 0; o < kVG; ++o) {
        const int j = i - o;
        if (j >= 0 && j < 11) {
          const float wj = win.w[j];
#pragma unroll
          for (int q = 0; q < 5; ++q) v[q][o] += wj * t[q];
        }
      }
    }
#pragma unroll
    for (int o = 0; o < kVG; ++o) {
      const int r = kVG * h + o;
      const int gy = y0 + r, gx = x0 + c;
      if (gy >= H || gx >= W) continue;
      const float mx = v[0][o], my = v[1][o], exx = v[2][o], eyy = v[3][o], exy = v[4][o];
      const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
      const float A1 = 2.f * mx * my + C1, A2 = 2.f * sxy + C2;
      const float B1 = mx * mx + my * my + C1, B2 = sxx + syy + C2;
      const float inv = 1.0f / (B1 * B2);
      const float S = A1 * A2 * inv;
      const float dmu = 2.f * my * A2 * inv - 2.f * mx * S / B1;
      const float dvar = -S / B2;
      const float dcov = 2.f * A1 * inv;
      const size_t oo = ch * HW + size_t(gy) * W + gx;
      amap[oo] = dmu - 2.f * mx * dvar - my * dcov;
      bmap[oo] = dvar;
      cmap[oo] = dcov;
      ssim_acc += S;
      l1_acc += fabsf(sx[r + kR][c + kR] - sy[r + kR][c + kR]);
    }
  }
  reduce_block_2(ssim_acc, l1_acc, s_tmp);
  if (threadIdx.x == 0) {
    const int b = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    partial[2 * b] = ssim_acc;
    partial[2 * b + 1] = l1_acc;
  }
}

__global__ void __launch_bounds__(256) ssim_bwd_kernel(const float* __restrict__ img, const float* __restrict__ tgt,
                                                        int H, int W, Window win, float lambda,
                                                        const float* __restrict__ amap,
                                                        const float* __restrict__ bmap,
                                                        const float* __restrict__ cmap, float* __restrict__ grad) {
  __shared__ float sa[3][kPH][kPW + 1];
  __shared__ float4 hs[3][kPH][kTW / 4];
  const int ch = blockIdx.z;
  const int x0 = blockIdx.x * kTW, y0 = blockIdx.y * kTH;
  const size_t HW = size_t(H) * W;
  const float* maps[3] = {amap + ch * HW, bmap + ch * HW, cmap + ch * HW};
  for (int k = threadIdx.x; k < kPH * kPW; k += 256) {
    const int r = k / kPW, c = k % kPW;
    const int gy = y0 + r - kR, gx = x0 + c - kR;
    const bool in = gy >= 0 && gy < H && gx >= 0 && gx < W;
    const size_t o = size_t(gy) * W + gx;
#pragma unroll
    for (int m = 0; m < 3; ++m) sa[m][r][c] = in ? maps[m][o] : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x < kHItems) {
    const int r = threadIdx.x / (kTW / kHG), g = threadIdx.x % (kTW / kHG);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      float in[kHG + 10];
#pragma unroll
      for (int j = 0; j < kHG + 10; ++j) in[j] = sa[m][r][kHG * g + j];
      float out[kHG];
#pragma unroll
      for (int o = 0; o < kHG; ++o) {
        out[o] = 0.f;
#pragma unroll
        for (int j = 0; j < 11; ++j) out[o] += win.w[j] * in[o + j];
      }
      hs[m][r][g] = make_float4(out[0], out[1], out[2], out[3]);
    }
  }
  __syncthreads();
  const float invN = 1.0f / float(3 * HW);
  const float kl1 = (1.0f - lambda) * invN, kss = -lambda * invN;
  const int c = threadIdx.x % kTW, h = threadIdx.x / kTW;
  const float* hsf = reinterpret_cast<const float*>(hs);
  float v[3][kVG];
#pragma unroll
  for (int o = 0; o < kVG; ++o) v[0][o] = v[1][o] = v[2][o] = 0.f;
#pragma unroll
  for (int i = 0; i < kVG + 10; ++i) {
    const int rr = kVG * h + i;
    float t[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) t[q] = hsf[(q * kPH + rr) * kTW + c];
#pragma unroll
    for (int o = 0; o < kVG; ++o) {
      const int j = i - o;
      if (j >= 0 && j < 11) {
        const float wj = win.w[j];
#pragma unroll
        for (int q = 0; q < 3; ++q) v[q][o] += wj * t[q];
      }
    }
  }
#pragma unroll
  for (int o = 0; o < kVG; ++o) {
    const int gy = y0 + kVG * h + o, gx = x0 + c;
    if (gy >= H || gx >= W) continue;
    const size_t oo = ch * HW + size_t(gy) * W + gx;
    const float xv = img[oo], yv = tgt[oo];
    const float d = xv - yv;
    const float sgn = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
    grad[oo] = kl1 * sgn + kss * (v[0][o] + 2.f * xv * v[1][o] + yv * v[2][o]);
  }
}

__global__ void __launch_bounds__(256) loss_finalize_kernel(const float* __restrict__ partial, int nblocks,
                                                             double inv_n, float lambda, float* __restrict__ out) {
  __shared__ double s_a[256], s_b[256];
  double a = 0.0, b = 0.0;
  for (int k = threadIdx.x; k < nblocks; k += 256) {
    a += double(partial[2 * k]);
    b += double(partial[2 * k + 1]);
  }
  s_a[threadIdx.x] = a;
  s_b[threadIdx.x] = b;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      s_a[threadIdx.x] += s_a[threadIdx.x + s];
      s_b[threadIdx.x] += s_b[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double ssim = s_a[0] * inv_n, l1 = s_b[0] * inv_n;
    out[0] = float((1.0 - double(lambda)) * l1 + double(lambda) * (1.0 - ssim));
    out[1] = float(l1);
    out[2] = float(ssim);
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

size_t loss_ws_bytes(int H, int W) {
  const size_t NE = size_t(3) * H * W;
  const size_t nb = size_t(div_up(W, kTW)) * div_up(H, kTH) * 3;
  return 3 * align256(NE * 4) + align256(nb * 2 * 4);
}

hipError_t launch_loss(const float* img, const float* target, int H, int W, float lambda, float* loss_out,
                       float* grad, void* ws, hipStream_t s) {
  Window win;
  double wsum = 0.0, wd[11];
  for (int j = -kR; j <= kR; ++j) {
    wd[j + kR] = exp(-double(j * j) / (2.0 * 1.5 * 1.5));
    wsum += wd[j + kR];
  }
  for (int j = 0; j < 11; ++j) win.w[j] = float(wd[j] / wsum);
  const size_t NE = size_t(3) * H * W;
  char* p = static_cast<char*>(ws);
  float* amap = reinterpret_cast<float*>(p); p += align256(NE * 4);
  float* bmap = reinterpret_cast<float*>(p); p += align256(NE * 4);
  float* cmap = reinterpret_cast<float*>(p); p += align256(NE * 4);
  float* partial = reinterpret_cast<float*>(p);
  const dim3 grid(div_up(W, kTW), div_up(H, kTH), 3);
  {
    GSK_PROF("ssim_fwd", s);
    ssim_fwd_kernel<<<grid, 256, 0, s>>>(img, target, H, W, win, amap, bmap, cmap, partial);
  }
  {
    GSK_PROF("ssim_bwd", s);
    ssim_bwd_kernel<<<grid, 256, 0, s>>>(img, target, H, W, win, lambda, amap, bmap, cmap, grad);
  }
  const int nb = int(grid.x * grid.y * grid.z);
  {
    GSK_PROF("loss_finalize", s);
    loss_finalize_kernel<<<1, 256, 0, s>>>(partial, nb, 1.0 / double(NE), lambda, loss_out);
  }
  return hipGetLastError();
}

}  // namespace gsk
