// Loss (1 - lambda) L1 + lambda (1 - SSIM) and its image gradient.
//
// [GST] loss slides (Gaussian splatting training study deck): L1 is the mean over
// 3HW with a zero subgradient at zero residual; SSIM uses an 11x11 Gaussian window
// of standard deviation 1.5 (normalised), C1 = 0.01^2, C2 = 0.03^2, zero padding,
// and is averaged over pixels and channels; D-SSIM carries no one-half.
//
// The 2-D window is the outer product of the normalised 1-D window, so the five
// local moments are computed with a horizontal then a vertical 11-tap pass through
// LDS (32x16 output pixels per block, 5-pixel halo).
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

__global__ void __launch_bounds__(256) ssim_fwd_kernel(const float* __restrict__ img, const float* __restrict__ tgt,
                                                        int H, int W, Window win, float* __restrict__ amap,
                                                        float* __restrict__ bmap, float* __restrict__ cmap,
                                                        float* __restrict__ partial) {
  __shared__ float sx[kPH][kPW + 1];
  __shared__ float sy[kPH][kPW + 1];
  __shared__ float hs[5][kPH][kTW + 1];
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
  for (int k = threadIdx.x; k < kPH * kTW; k += 256) {
    const int r = k / kTW, c = k % kTW;
    float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f, m4 = 0.f;
#pragma unroll
    for (int j = 0; j < 11; ++j) {
      const float xv = sx[r][c + j], yv = sy[r][c + j], wj = win.w[j];
      m0 += wj * xv;
      m1 += wj * yv;
      m2 += wj * xv * xv;
      m3 += wj * yv * yv;
      m4 += wj * xv * yv;
    }
    hs[0][r][c] = m0; hs[1][r][c] = m1; hs[2][r][c] = m2; hs[3][r][c] = m3; hs[4][r][c] = m4;
  }
  __syncthreads();
  const float C1 = 0.01f * 0.01f, C2 = 0.03f * 0.03f;
  float ssim_acc = 0.f, l1_acc = 0.f;
  for (int k = threadIdx.x; k < kTH * kTW; k += 256) {
    const int r = k / kTW, c = k % kTW;
    const int gy = y0 + r, gx = x0 + c;
    if (gy >= H || gx >= W) continue;
    float mx = 0.f, my = 0.f, exx = 0.f, eyy = 0.f, exy = 0.f;
#pragma unroll
    for (int i = 0; i < 11; ++i) {
      const float wi = win.w[i];
      mx += wi * hs[0][r + i][c];
      my += wi * hs[1][r + i][c];
      exx += wi * hs[2][r + i][c];
      eyy += wi * hs[3][r + i][c];
      exy += wi * hs[4][r + i][c];
    }
    const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
    const float A1 = 2.f * mx * my + C1, A2 = 2.f * sxy + C2;
    const float B1 = mx * mx + my * my + C1, B2 = sxx + syy + C2;
    const float inv = 1.0f / (B1 * B2);
    const float S = A1 * A2 * inv;
    const float dmu = 2.f * my * A2 * inv - 2.f * mx * S / B1;
    const float dvar = -S / B2;
    const float dcov = 2.f * A1 * inv;
    const size_t o = ch * HW + size_t(gy) * W + gx;
    amap[o] = dmu - 2.f * mx * dvar - my * dcov;
    bmap[o] = dvar;
    cmap[o] = dcov;
    ssim_acc += S;
    l1_acc += fabsf(sx[r + kR][c + kR] - sy[r + kR][c + kR]);
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
  __shared__ float hs[3][kPH][kTW + 1];
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
  for (int k = threadIdx.x; k < kPH * kTW; k += 256) {
    const int r = k / kTW, c = k % kTW;
    float m0 = 0.f, m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int j = 0; j < 11; ++j) {
      const float wj = win.w[j];
      m0 += wj * sa[0][r][c + j];
      m1 += wj * sa[1][r][c + j];
      m2 += wj * sa[2][r][c + j];
    }
    hs[0][r][c] = m0; hs[1][r][c] = m1; hs[2][r][c] = m2;
  }
  __syncthreads();
  const float invN = 1.0f / float(3 * HW);
  const float kl1 = (1.0f - lambda) * invN, kss = -lambda * invN;
  for (int k = threadIdx.x; k < kTH * kTW; k += 256) {
    const int r = k / kTW, c = k % kTW;
    const int gy = y0 + r, gx = x0 + c;
    if (gy >= H || gx >= W) continue;
    float ba = 0.f, bb = 0.f, bc = 0.f;
#pragma unroll
    for (int i = 0; i < 11; ++i) {
      const float wi = win.w[i];
      ba += wi * hs[0][r + i][c];
      bb += wi * hs[1][r + i][c];
      bc += wi * hs[2][r + i][c];
    }
    const size_t o = ch * HW + size_t(gy) * W + gx;
    const float xv = img[o], yv = tgt[o];
    const float d = xv - yv;
    const float sgn = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
    grad[o] = kl1 * sgn + kss * (ba + 2.f * xv * bb + yv * bc);
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
