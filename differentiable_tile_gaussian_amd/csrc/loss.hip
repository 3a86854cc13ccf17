// Loss (1 - lambda) L1 + lambda (1 - SSIM) and its image gradient.
//
// [GST] loss slides (Gaussian splatting training study deck): L1 is the mean over
// 3HW with a zero subgradient at zero residual; SSIM uses an 11x11 Gaussian window
// of standard deviation 1.5 (normalised), C1 = 0.01^2, C2 = 0.03^2, zero padding,
// and is averaged over pixels and channels; D-SSIM carries no one-half.
//
// The 2-D window is the outer product of the normalised 1-D window w.  Per pixel the
// SSIM map needs the five local moments (w*x, w*y, w*xx, w*yy, w*xy); its gradient is
//   dL/dx = (1-lambda)/N sign(x-y) - lambda/N (w*a + 2 x (w*b) + y (w*c))
// with the derivative maps a = dS/dmu_x - 2 mu_x dS/dvar_x - mu_y dS/dcov,
// b = dS/dvar_x, c = dS/dcov (w* is the same zero-padded window; it is symmetric, so
// it is its own adjoint).
//
// One kernel does both passes over a strip of rows, sliding down the image one row
// per step.  A block of kSW threads owns kSW adjacent "moment" columns; the middle
// kSW - 10 of them are its output columns.  At step i the block stages input row i
// in LDS, each thread takes the horizontal moments of its column at row i and keeps
// the last eleven in registers (a ring, so the vertical sums need no LDS); with
// them it finishes the moments, SSIM and a, b, c of row i - 5, puts a, b, c in LDS,
// takes their horizontal sums at its column and keeps the last eleven of those; and
// with those finishes the gradient of row i - 10.  Inputs outside the image are
// zero, and so are a, b, c there.  The a, b, c maps never leave the chip.
//   loss_finalize   sums the per-block SSIM and |x - y| partials (fp64) into total,
//                   L1 and mean SSIM
#include <math.h>

#include <mutex>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kR = 5;                 // window radius
constexpr int kSW = 128;              // moment columns per block (threads)
constexpr int kSO = kSW - 2 * kR;     // output columns per block
constexpr int kSIn = kSW + 2 * kR;    // input columns staged per row
constexpr int kRing = 2 * kR + 1;     // 11
constexpr int kSR = 35;               // output rows per block: the kSR + 4 kR steps of a
constexpr int kSteps = kSR + 4 * kR;  // strip are a whole number of ring turns, so the
static_assert(kSteps % kRing == 0, "whole ring turns");   // step loop unrolls with static slots

struct Window { float w[11]; };

__device__ inline float load_or_zero(const float* __restrict__ p, int row, int col, int H, int W) {
  return (row >= 0 && row < H && col >= 0 && col < W) ? p[size_t(row) * W + col] : 0.0f;
}

__global__ void __launch_bounds__(kSW) ssim_fused_kernel(const float* __restrict__ img,
                                                         const float* __restrict__ tgt, int H, int W, Window win,
                                                         float kl1, float kss, float* __restrict__ grad,
                                                         float* __restrict__ partial) {
  // the last twelve input rows, row i in slot (i - first row) % 12: one more than the
  // eleven a step reads, so a row is rewritten only after a full step has passed its
  // last reader (the gradient of row i, read at step i + 10)
  __shared__ float s_x[kRing + 1][kSIn], s_y[kRing + 1][kSIn];
  __shared__ float s_abc[2][3][kSW];
  __shared__ float s_tmp[2 * (kSW / 64)];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
  const int ch = blockIdx.z;
  const int x0 = blockIdx.x * kSO, y0 = blockIdx.y * kSR;
  const int cf = x0 - kR + tid;                       // this thread's moment column
  const bool out_col = tid >= kR && tid < kSW - kR && cf < W;
  const size_t HW = size_t(H) * W;
  const float* __restrict__ X = img + ch * HW;
  const float* __restrict__ Y = tgt + ch * HW;
  const float C1 = 0.01f * 0.01f, C2 = 0.03f * 0.03f;
  // input column x0 - 2 kR + k for k in [0, kSIn): thread tid stages k = tid and,
  // for tid < 2 kR, k = kSW + tid
  const int cin0 = x0 - 2 * kR + tid, cin1 = x0 - 2 * kR + kSW + tid;
  const int ifirst = y0 - 2 * kR, ilast = y0 + kSR + 2 * kR - 1;
  float px0 = load_or_zero(X, ifirst, cin0, H, W), py0 = load_or_zero(Y, ifirst, cin0, H, W);
  float px1 = 0.0f, py1 = 0.0f;
  if (tid < 2 * kR) {
    px1 = load_or_zero(X, ifirst, cin1, H, W);
    py1 = load_or_zero(Y, ifirst, cin1, H, W);
  }
  float hm[kRing][5], ga[kRing][3];
#pragma unroll
  for (int u = 0; u < kRing; ++u) {
#pragma unroll
    for (int q = 0; q < 5; ++q) hm[u][q] = 0.0f;
#pragma unroll
    for (int q = 0; q < 3; ++q) ga[u][q] = 0.0f;
  }
  float ssim_acc = 0.0f, l1_acc = 0.0f;
  for (int turn = 0; turn < kSteps / kRing; ++turn) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int i = ifirst + turn * kRing + u;   // the register ring slot of step i is u
      const int b = i & 1;
      const int k = turn * kRing + u;
      const int row_i = k % (kRing + 1), row_r = (k + kRing + 1 - kR) % (kRing + 1),
                row_q = (k + kRing + 1 - 2 * kR) % (kRing + 1);   // LDS slots of rows i, i-5, i-10
      s_x[row_i][tid] = px0;
      s_y[row_i][tid] = py0;
      if (tid < 2 * kR) {
        s_x[row_i][kSW + tid] = px1;
        s_y[row_i][kSW + tid] = py1;
      }
      if (i < ilast) {   // the next row's loads are in flight during this step
        px0 = load_or_zero(X, i + 1, cin0, H, W);
        py0 = load_or_zero(Y, i + 1, cin0, H, W);
        if (tid < 2 * kR) {
          px1 = load_or_zero(X, i + 1, cin1, H, W);
          py1 = load_or_zero(Y, i + 1, cin1, H, W);
        }
      }
      __syncthreads();
      {
        float m[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const float wj = win.w[j], xv = s_x[row_i][tid + j], yv = s_y[row_i][tid + j];
          m[0] += wj * xv;
          m[1] += wj * yv;
          m[2] += wj * (xv * xv);
          m[3] += wj * (yv * yv);
          m[4] += wj * (xv * yv);
        }
#pragma unroll
        for (int q = 0; q < 5; ++q) hm[u][q] = m[q];
      }
      if (i >= y0) {
        // moments, SSIM and a, b, c of row r = i - 5 (ring slots of steps i-10 .. i)
        const int r = i - kR;
        float mv[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const float wj = win.w[j];
#pragma unroll
          for (int q = 0; q < 5; ++q) mv[q] += wj * hm[(u + 1 + j) % kRing][q];
        }
        float a = 0.f, bb = 0.f, c = 0.f;
        if (r >= 0 && r < H && cf >= 0 && cf < W) {
          const float mx = mv[0], my = mv[1], exx = mv[2], eyy = mv[3], exy = mv[4];
          const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
          const float A1 = 2.f * mx * my + C1, A2 = 2.f * sxy + C2;
          const float B1 = mx * mx + my * my + C1, B2 = sxx + syy + C2;
          const float inv = 1.0f / (B1 * B2);
          const float S = A1 * A2 * inv;
          const float dmu = 2.f * my * A2 * inv - 2.f * mx * S / B1;
          const float dvar = -S / B2;
          const float dcov = 2.f * A1 * inv;
          a = dmu - 2.f * mx * dvar - my * dcov;
          bb = dvar;
          c = dcov;
          if (out_col && r >= y0 && r < y0 + kSR) {
            ssim_acc += S;
            l1_acc += fabsf(s_x[row_r][tid + kR] - s_y[row_r][tid + kR]);
          }
        }
        s_abc[b][0][tid] = a;
        s_abc[b][1][tid] = bb;
        s_abc[b][2][tid] = c;
      }
      __syncthreads();
      if (i >= y0) {
        float g[3] = {0.f, 0.f, 0.f};
        if (tid >= kR && tid < kSW - kR) {
#pragma unroll
          for (int j = 0; j < kRing; ++j) {
            const float wj = win.w[j];
#pragma unroll
            for (int q = 0; q < 3; ++q) g[q] += wj * s_abc[b][q][tid - kR + j];
          }
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) ga[u][q] = g[q];
      }
      if (i >= y0 + 2 * kR) {
        // gradient of row q = i - 10: vertical sums of the horizontal sums of a, b, c
        // at rows q-5 .. q+5 (steps i-10 .. i); x, y of row q were staged at step i-10
        const int q = i - 2 * kR;
        float cv[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const float wj = win.w[j];
#pragma unroll
          for (int t = 0; t < 3; ++t) cv[t] += wj * ga[(u + 1 + j) % kRing][t];
        }
        if (out_col && q < H) {
          const float xv = s_x[row_q][tid + kR], yv = s_y[row_q][tid + kR];
          const float d = xv - yv;
          const float sgn = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
          grad[ch * HW + size_t(q) * W + cf] = kl1 * sgn + kss * (cv[0] + 2.f * xv * cv[1] + yv * cv[2]);
        }
      }
    }
  }
  // block sums of SSIM and |x - y|
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    ssim_acc += __shfl_xor(ssim_acc, d, 64);
    l1_acc += __shfl_xor(l1_acc, d, 64);
  }
  if (lane == 0) {
    s_tmp[2 * wave] = ssim_acc;
    s_tmp[2 * wave + 1] = l1_acc;
  }
  __syncthreads();
  if (tid == 0) {
    float sa = 0.f, sb = 0.f;
    for (int w = 0; w < kSW / 64; ++w) { sa += s_tmp[2 * w]; sb += s_tmp[2 * w + 1]; }
    const int blk = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    partial[2 * blk] = sa;
    partial[2 * blk + 1] = sb;
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

// ------------------------------------------------ Charbonnier loss with exposure
// [GSG] the trainer's loss (the code after "The painting itself") and "Forgiving the
// camera and the light": err = gain x + bias - y, root = sqrt(err^2 + delta^2); the loss is
// the mean of root - delta over the 3HW elements, dL/dx = gain (err / root) / 3HW, and the
// exposure gradients are the means of (err / root) x gain (log gain) and err / root (bias).
// One pass: 16 elements per thread (four 16-byte loads when the arrays allow), the
// block's three partial sums in fp32, then one block adds the partials in fp64 in a fixed
// order (so the result does not depend on scheduling).
constexpr int kCbThreads = 256;
constexpr int kCbItems = 16;
constexpr int kCbTile = kCbThreads * kCbItems;

__global__ void __launch_bounds__(kCbThreads) charbonnier_kernel(const float* __restrict__ img,
                                                                  const float* __restrict__ tgt, int64_t count,
                                                                  float delta, const float* __restrict__ exposure,
                                                                  float inv_count, bool vec, float* __restrict__ grad,
                                                                  float* __restrict__ partial) {
  __shared__ float s_part[3][kCbThreads / 64];
  const float gain = float(exp(double(exposure[0]))), bias = exposure[1];
  const int64_t base = int64_t(blockIdx.x) * kCbTile + int64_t(threadIdx.x) * 4;
  float sl = 0.0f, sg = 0.0f, sb = 0.0f;
#pragma unroll
  for (int r = 0; r < kCbItems / 4; ++r) {
    const int64_t i0 = base + int64_t(r) * kCbThreads * 4;
    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    const bool full = vec && i0 + 4 <= count;
    if (full) {
      const float4 a = *reinterpret_cast<const float4*>(img + i0), b = *reinterpret_cast<const float4*>(tgt + i0);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      y[0] = b.x; y[1] = b.y; y[2] = b.z; y[3] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < count) { x[k] = img[i0 + k]; y[k] = tgt[i0 + k]; }
    }
    float g[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = i0 + k < count;
      const float err = gain * x[k] + bias - y[k];
      const float root = sqrtf(err * err + delta * delta);
      const float eg = err / root;
      g[k] = gain * eg * inv_count;
      if (in) {
        sl += root - delta;
        sg += eg * x[k] * gain;
        sb += eg;
      }
    }
    if (full) {
      *reinterpret_cast<float4*>(grad + i0) = make_float4(g[0], g[1], g[2], g[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < count) grad[i0 + k] = g[k];
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    sl += __shfl_xor(sl, d, 64);
    sg += __shfl_xor(sg, d, 64);
    sb += __shfl_xor(sb, d, 64);
  }
  if (__lane_id() == 0) {
    s_part[0][threadIdx.x >> 6] = sl;
    s_part[1][threadIdx.x >> 6] = sg;
    s_part[2][threadIdx.x >> 6] = sb;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    float t = 0.0f;
    for (int w = 0; w < kCbThreads / 64; ++w) t += s_part[threadIdx.x][w];
    partial[3 * blockIdx.x + threadIdx.x] = t;
  }
}

__global__ void __launch_bounds__(256) charbonnier_finalize_kernel(const float* __restrict__ partial, int nblocks,
                                                                    double inv_n, float* __restrict__ loss_out,
                                                                    float* __restrict__ dexp) {
  __shared__ double s[3][256];
  double a[3] = {0.0, 0.0, 0.0};
  for (int k = threadIdx.x; k < nblocks; k += 256)
    for (int j = 0; j < 3; ++j) a[j] += double(partial[3 * k + j]);
  for (int j = 0; j < 3; ++j) s[j][threadIdx.x] = a[j];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h)
      for (int j = 0; j < 3; ++j) s[j][threadIdx.x] += s[j][threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    loss_out[0] = float(s[0][0] * inv_n);
    if (dexp) {
      dexp[0] = float(s[1][0] * inv_n);
      dexp[1] = float(s[2][0] * inv_n);
    }
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

size_t charbonnier_ws_bytes(int H, int W) {
  const int64_t count = int64_t(3) * H * W;
  return align256(size_t(div_up(count, kCbTile)) * 3 * 4);
}

hipError_t launch_charbonnier(const float* img, const float* target, int H, int W, float delta, const float* exposure,
                              float* loss_out, float* grad, float* dexp, void* ws, hipStream_t s) {
  const int64_t count = int64_t(3) * H * W;
  const int nb = int(div_up(count, kCbTile));
  float* partial = static_cast<float*>(ws);
  const bool vec = reinterpret_cast<uintptr_t>(img) % 16 == 0 && reinterpret_cast<uintptr_t>(target) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(grad) % 16 == 0;
  {
    GSK_PROF("charbonnier", s);
    charbonnier_kernel<<<nb, kCbThreads, 0, s>>>(img, target, count, delta, exposure, float(1.0 / double(count)),
                                                 vec, grad, partial);
  }
  {
    GSK_PROF("charbonnier_finalize", s);
    charbonnier_finalize_kernel<<<1, 256, 0, s>>>(partial, nb, 1.0 / double(count), loss_out, dexp);
  }
  return hipGetLastError();
}

// Scratch of the no-allocation entry point (gs_loss_l1_dssim_noalloc): the loss's
// per-block partial sums live in this array, one copy per GPU that the library runs on,
// held until the process ends.  Host code must not pass the array's name to a kernel (on
// the host it is a stand-in, not a device address): loss_scratch() looks its device
// address up once per device and keeps it.  Every partial is written by the loss kernel
// before the finalize kernel reads it, so nothing needs clearing between calls; calls
// that overlap on one GPU share the array and race.
constexpr size_t kLossScratchBytes = size_t(256) << 10;
static __device__ __align__(256) unsigned char scratch[kLossScratchBytes];

size_t loss_scratch_bytes() { return kLossScratchBytes; }

hipError_t loss_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

size_t loss_ws_bytes(int H, int W) {
  const size_t nb = size_t(div_up(W, kSO)) * div_up(H, kSR) * 3;
  return align256(nb * 2 * 4);
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
  float* partial = static_cast<float*>(ws);
  const dim3 grid(div_up(W, kSO), div_up(H, kSR), 3);
  const float invN = 1.0f / float(NE);
  {
    GSK_PROF("ssim", s);
    ssim_fused_kernel<<<grid, kSW, 0, s>>>(img, target, H, W, win, (1.0f - lambda) * invN, -lambda * invN, grad,
                                           partial);
  }
  const int nb = int(grid.x * grid.y * grid.z);
  {
    GSK_PROF("loss_finalize", s);
    loss_finalize_kernel<<<1, 256, 0, s>>>(partial, nb, 1.0 / double(NE), lambda, loss_out);
  }
  return hipGetLastError();
}

}  // namespace gsk
