// Per-Gaussian projection (forward) and parameter-gradient chain (backward).
//
// This translation unit is compiled with -ffp-contract=off: the key path
// (camera-space depth, screen centre, extent, tile rectangle) must be plain
// IEEE fp32 in the written order so that the pair list is reproducible
// bit for bit.  exp, log and the sigmoid on that path are evaluated in fp64
// and rounded once.  Division and square root are the correctly rounded fp32
// operations (the HIP default).
//
// One thread per Gaussian; params are read plane by plane (coalesced SoA).
//
// Pages (titles as they appear on the pages):
//   [DR]  "Differentiable rasterisation";  [GST] Gaussian splatting training study deck;
//   [GSG] "How a computer rebuilds a real place out of soft colored dots called Gaussian Splats".
#include "gs_internal.h"

namespace gsk {
namespace {

// Real spherical harmonics, Condon-Shortley phase (the sign convention of the
// degree-1 and degree-2 patterns printed in [GSG] "Spherical harmonics").
// Constants: sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) (x sqrt 2 for m != 0) times the
// leading factor of the associated Legendre polynomial written in x, y, z.
constexpr float kSH1 = 0.488602511902919920f;   // band 1
constexpr float kSH2xy = 1.09254843059207907f;  // 2xy, yz, xz terms of band 2
constexpr float kSH2z = 0.315391565252520050f;  // 2z^2 - x^2 - y^2
constexpr float kSH2xx = 0.546274215296039535f; // x^2 - y^2
constexpr float kSH3a = 0.590043589926643510f;  // y(3x^2-y^2), x(x^2-3y^2)
constexpr float kSH3b = 2.89061144264055405f;   // xyz
constexpr float kSH3c = 0.457045799464465737f;  // y(4z^2-x^2-y^2), x(4z^2-x^2-y^2)
constexpr float kSH3d = 0.373176332590115391f;  // z(2z^2-3x^2-3y^2)
constexpr float kSH3e = 1.44530572132027735f;   // z(x^2-y^2)

// Basis values Y[1..15] at unit direction (x, y, z); Y[0] is not used.
__device__ inline void sh_eval(float x, float y, float z, float* Y) {
  const float xx = x * x, yy = y * y, zz = z * z;
  Y[1] = -kSH1 * y;
  Y[2] = kSH1 * z;
  Y[3] = -kSH1 * x;
  Y[4] = kSH2xy * x * y;
  Y[5] = -kSH2xy * y * z;
  Y[6] = kSH2z * (2.0f * zz - xx - yy);
  Y[7] = -kSH2xy * x * z;
  Y[8] = kSH2xx * (xx - yy);
  Y[9] = -kSH3a * y * (3.0f * xx - yy);
  Y[10] = kSH3b * x * y * z;
  Y[11] = -kSH3c * y * (4.0f * zz - xx - yy);
  Y[12] = kSH3d * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
  Y[13] = -kSH3c * x * (4.0f * zz - xx - yy);
  Y[14] = kSH3e * z * (xx - yy);
  Y[15] = -kSH3a * x * (xx - 3.0f * yy);
}

// g . dY/d(x, y, z) for a per-basis weight vector w[1..K] (K = active bands), accumulated
// into out[3]: the derivative of sum_k w_k Y_k(x, y, z) as a polynomial in x, y, z.
__device__ inline void sh_grad_dot(float x, float y, float z, const float* w, int K, float* out) {
  const float xx = x * x, yy = y * y, zz = z * z;
  float gx = 0.f, gy = 0.f, gz = 0.f;
  if (K >= 3) {
    gy += -kSH1 * w[1];
    gz += kSH1 * w[2];
    gx += -kSH1 * w[3];
  }
  if (K >= 8) {
    gx += kSH2xy * y * w[4];          gy += kSH2xy * x * w[4];
    gy += -kSH2xy * z * w[5];         gz += -kSH2xy * y * w[5];
    gx += -2.0f * kSH2z * x * w[6];   gy += -2.0f * kSH2z * y * w[6];   gz += 4.0f * kSH2z * z * w[6];
    gx += -kSH2xy * z * w[7];         gz += -kSH2xy * x * w[7];
    gx += 2.0f * kSH2xx * x * w[8];   gy += -2.0f * kSH2xx * y * w[8];
  }
  if (K >= 15) {
    gx += -kSH3a * 6.0f * x * y * w[9];
    gy += -kSH3a * (3.0f * xx - 3.0f * yy) * w[9];
    gx += kSH3b * y * z * w[10];  gy += kSH3b * x * z * w[10];  gz += kSH3b * x * y * w[10];
    gx += -kSH3c * (-2.0f * x * y) * w[11];
    gy += -kSH3c * (4.0f * zz - xx - 3.0f * yy) * w[11];
    gz += -kSH3c * 8.0f * y * z * w[11];
    gx += kSH3d * (-6.0f * x * z) * w[12];
    gy += kSH3d * (-6.0f * y * z) * w[12];
    gz += kSH3d * (6.0f * zz - 3.0f * xx - 3.0f * yy) * w[12];
    gx += -kSH3c * (4.0f * zz - 3.0f * xx - yy) * w[13];
    gy += -kSH3c * (-2.0f * x * y) * w[13];
    gz += -kSH3c * 8.0f * x * z * w[13];
    gx += kSH3e * 2.0f * x * z * w[14];  gy += -kSH3e * 2.0f * y * z * w[14];  gz += kSH3e * (xx - yy) * w[14];
    gx += -kSH3a * (3.0f * xx - 3.0f * yy) * w[15];
    gy += -kSH3a * (-6.0f * x * y) * w[15];
  }
  out[0] += gx;
  out[1] += gy;
  out[2] += gz;
}

// Intermediate quantities of the projection of one Gaussian.
struct Proj {
  float p[3];            // camera-space centre
  float xz, yz, u, v;
  float s[3];            // scales
  float ql, q[4];        // |q| and the normalised quaternion
  float Rq[9];           // rotation, row-major
  float M[9];            // Rq diag(s)
  float Sig[6];          // 00 01 02 11 12 22
  float t0[3], t1[3];    // rows of T = J W
  float a, b, c, det;    // dilated screen covariance
  float A, B, C;         // conic
  float o;
};

// Geometry of one Gaussian ([GST] parameter and Jacobian slides; [DR] "Forward";
// [GSG] "Flattening a 3D blob into a 2D oval").  Returns false when culled (behind the
// near plane, zero quaternion, non-positive determinant).
__device__ inline bool project_geometry(const float* __restrict__ params, int n, int i, const gs_camera& cam,
                                        Proj& g) {
  const float mx = params[i], my = params[n + i], mz = params[2 * n + i];
  for (int r = 0; r < 3; ++r)
    g.p[r] = ((cam.R[3 * r] * mx + cam.R[3 * r + 1] * my) + cam.R[3 * r + 2] * mz) + cam.t[r];
  if (!(g.p[2] > cam.znear)) return false;
  g.xz = g.p[0] / g.p[2];
  g.yz = g.p[1] / g.p[2];
  g.u = cam.fx * g.xz + cam.cx;
  g.v = cam.fy * g.yz + cam.cy;
  for (int k = 0; k < 3; ++k) g.s[k] = float(exp(double(params[(3 + k) * n + i])));
  const float qw = params[6 * n + i], qx = params[7 * n + i], qy = params[8 * n + i], qz = params[9 * n + i];
  const float n2 = ((qw * qw + qx * qx) + qy * qy) + qz * qz;
  if (!(n2 > 0.0f)) return false;
  g.ql = sqrtf(n2);
  g.q[0] = qw / g.ql; g.q[1] = qx / g.ql; g.q[2] = qy / g.ql; g.q[3] = qz / g.ql;
  const float w = g.q[0], x = g.q[1], y = g.q[2], z = g.q[3];
  g.Rq[0] = 1.0f - 2.0f * (y * y + z * z);
  g.Rq[1] = 2.0f * (x * y - w * z);
  g.Rq[2] = 2.0f * (x * z + w * y);
  g.Rq[3] = 2.0f * (x * y + w * z);
  g.Rq[4] = 1.0f - 2.0f * (x * x + z * z);
  g.Rq[5] = 2.0f * (y * z - w * x);
  g.Rq[6] = 2.0f * (x * z - w * y);
  g.Rq[7] = 2.0f * (y * z + w * x);
  g.Rq[8] = 1.0f - 2.0f * (x * x + y * y);
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) g.M[3 * r + k] = g.Rq[3 * r + k] * g.s[k];
  const float* M = g.M;
  // Sigma = M M^T
  g.Sig[0] = (M[0] * M[0] + M[1] * M[1]) + M[2] * M[2];
  g.Sig[1] = (M[0] * M[3] + M[1] * M[4]) + M[2] * M[5];
  g.Sig[2] = (M[0] * M[6] + M[1] * M[7]) + M[2] * M[8];
  g.Sig[3] = (M[3] * M[3] + M[4] * M[4]) + M[5] * M[5];
  g.Sig[4] = (M[3] * M[6] + M[4] * M[7]) + M[5] * M[8];
  g.Sig[5] = (M[6] * M[6] + M[7] * M[7]) + M[8] * M[8];
  // T = J W with J = [fx/z, 0, -fx x/z^2; 0, fy/z, -fy y/z^2]
  const float J00 = cam.fx / g.p[2];
  const float J02 = -(cam.fx * g.xz) / g.p[2];
  const float J11 = cam.fy / g.p[2];
  const float J12 = -(cam.fy * g.yz) / g.p[2];
  for (int k = 0; k < 3; ++k) {
    g.t0[k] = J00 * cam.R[k] + J02 * cam.R[6 + k];
    g.t1[k] = J11 * cam.R[3 + k] + J12 * cam.R[6 + k];
  }
  const float* S = g.Sig;
  // rows of Sigma in full: (S0 S1 S2 / S1 S3 S4 / S2 S4 S5)
  const float w00 = (S[0] * g.t0[0] + S[1] * g.t0[1]) + S[2] * g.t0[2];
  const float w01 = (S[1] * g.t0[0] + S[3] * g.t0[1]) + S[4] * g.t0[2];
  const float w02 = (S[2] * g.t0[0] + S[4] * g.t0[1]) + S[5] * g.t0[2];
  const float w10 = (S[0] * g.t1[0] + S[1] * g.t1[1]) + S[2] * g.t1[2];
  const float w11 = (S[1] * g.t1[0] + S[3] * g.t1[1]) + S[4] * g.t1[2];
  const float w12 = (S[2] * g.t1[0] + S[4] * g.t1[1]) + S[5] * g.t1[2];
  const float V00 = (g.t0[0] * w00 + g.t0[1] * w01) + g.t0[2] * w02;
  const float V01 = (g.t1[0] * w00 + g.t1[1] * w01) + g.t1[2] * w02;
  const float V11 = (g.t1[0] * w10 + g.t1[1] * w11) + g.t1[2] * w12;
  g.a = V00 + 0.3f;   // 0.3 px^2 dilation ([GST] Jacobian slide)
  g.b = V01;
  g.c = V11 + 0.3f;
  g.det = g.a * g.c - g.b * g.b;
  if (!(g.det > 0.0f)) return false;
  g.A = g.c / g.det;
  g.B = -g.b / g.det;
  g.C = g.a / g.det;
  g.o = float(1.0 / (1.0 + exp(-double(params[10 * n + i]))));
  return true;
}

// View direction dir = normalize(mean - campos) and its length ([GSG] "Spherical harmonics").
__device__ inline float view_dir(const float* __restrict__ params, int n, int i, const gs_camera& cam,
                                 float* dir) {
  const float d0 = params[i] - cam.campos[0], d1 = params[n + i] - cam.campos[1],
              d2 = params[2 * n + i] - cam.campos[2];
  const float len = sqrtf((d0 * d0 + d1 * d1) + d2 * d2);
  dir[0] = d0 / len;
  dir[1] = d1 / len;
  dir[2] = d2 / len;
  return len;
}

// Colour before the clamp: DC + sum_k sh_k Y_k.
__device__ inline void sh_colour(const float* __restrict__ params, int n, int i, int K, const float* Y,
                                 float* raw) {
  for (int ch = 0; ch < 3; ++ch) {
    float col = params[(11 + ch) * n + i];
    for (int k = 1; k <= K; ++k) col = col + params[(14 + 3 * (k - 1) + ch) * n + i] * Y[k];
    raw[ch] = col;
  }
}

template <int DEG>
__global__ void __launch_bounds__(256) preprocess_fwd_kernel(const float* __restrict__ params, int n,
                                                              gs_camera cam, int tx, int ty, float4* __restrict__ splat,
                                                              float* __restrict__ depth, uint2* __restrict__ rect,
                                                              uint32_t* __restrict__ tiles) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  Proj g;
  bool vis = project_geometry(params, n, i, cam, g);
  float rgb[3] = {0.f, 0.f, 0.f};
  uint32_t x0 = 0, y0 = 0, x1 = 0, y1 = 0, cnt = 0;
  if (vis) {
    float Y[16];
    if (K > 0) {
      float dir[3];
      view_dir(params, n, i, cam, dir);
      sh_eval(dir[0], dir[1], dir[2], Y);
    }
    float raw[3];
    sh_colour(params, n, i, K, Y, raw);
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

// Backward chain, split in two kernels so each keeps few registers (and many waves
// in flight on a streaming, HBM-bound pass).  gscreen planes: 0 u, 1 v, 2 A, 3 B,
// 4 C, 5 opacity, 6-8 colour.
//
// Colour part ([GSG] "Spherical harmonics": dL/dsh_k = dRGB Y_k, and the
// view-direction term; the clamp at zero passes no gradient): writes the DC and
// band gradients and, at degree > 0, the direction term of the mean gradient.
template <int DEG>
__global__ void __launch_bounds__(256) chain_colour_kernel(const float* __restrict__ params, int n, gs_camera cam,
                                                            const uint32_t* __restrict__ tiles,
                                                            const float* __restrict__ gscreen,
                                                            float* __restrict__ gparams) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  constexpr int P = 11 + 3 * (K + 1);
  if (tiles[i] == 0u) {
    for (int pl = 11; pl < P; ++pl) gparams[pl * n + i] = 0.0f;
    if (K > 0)
      for (int c = 0; c < 3; ++c) gparams[c * n + i] = 0.0f;
    return;
  }
  float Y[16];
  float dir[3] = {0.f, 0.f, 0.f};
  float dlen = 1.0f;
  if (K > 0) {
    dlen = view_dir(params, n, i, cam, dir);
    sh_eval(dir[0], dir[1], dir[2], Y);
  }
  float raw[3];
  sh_colour(params, n, i, K, Y, raw);
  float gc[3];
  for (int ch = 0; ch < 3; ++ch) {
    gc[ch] = raw[ch] < 0.0f ? 0.0f : gscreen[(6 + ch) * n + i];
    gparams[(11 + ch) * n + i] = gc[ch];
  }
  if (K > 0) {
    float wk[16];
    for (int k = 1; k <= K; ++k) {
      float acc = 0.0f;
      for (int ch = 0; ch < 3; ++ch) {
        const int pl = 14 + 3 * (k - 1) + ch;
        gparams[pl * n + i] = gc[ch] * Y[k];
        acc += gc[ch] * params[pl * n + i];
      }
      wk[k] = acc;
    }
    float gdir[3] = {0.f, 0.f, 0.f};
    sh_grad_dot(dir[0], dir[1], dir[2], wk, K, gdir);
    const float dd = dir[0] * gdir[0] + dir[1] * gdir[1] + dir[2] * gdir[2];
    for (int a = 0; a < 3; ++a) gparams[a * n + i] = (gdir[a] - dir[a] * dd) / dlen;
  }
}

// Geometry part ([GSG] "From a pixel's blame to the oval's shape and place" (sigmoid),
// "The covariance chain" (dV = -K G K, dSigma = T^T H T, dT = 2 H T Sigma,
// dM = 2 dSigma M, scale and quaternion, projection off |q|), "Where the position
// gradient comes from"; [GST] Jacobian slide): writes the mean (adding the colour
// part's direction term at degree > 0), log-scale, quaternion and logit gradients.
template <int DEG>
__global__ void __launch_bounds__(256) chain_geometry_kernel(const float* __restrict__ params, int n, gs_camera cam,
                                                              const uint32_t* __restrict__ tiles,
                                                              const float* __restrict__ gscreen,
                                                              float* __restrict__ gparams) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  Proj g;
  if (tiles[i] == 0u || !project_geometry(params, n, i, cam, g)) {
    for (int pl = 0; pl < 11; ++pl) gparams[pl * n + i] = 0.0f;
    return;
  }
  const float gu = gscreen[i], gv = gscreen[n + i], gA = gscreen[2 * n + i], gB = gscreen[3 * n + i],
              gC = gscreen[4 * n + i], go = gscreen[5 * n + i];
  // opacity logit through the sigmoid
  gparams[10 * n + i] = go * g.o * (1.0f - g.o);
  float gm[3] = {0.f, 0.f, 0.f};
  if (DEG > 0)
    for (int a = 0; a < 3; ++a) gm[a] = gparams[a * n + i];
  // conic -> dilated covariance: dV' = -K Gk K with Gk = [[gA, gB/2], [gB/2, gC]]
  const float hB = 0.5f * gB;
  const float kg00 = g.A * gA + g.B * hB, kg01 = g.A * hB + g.B * gC;
  const float kg10 = g.B * gA + g.C * hB, kg11 = g.B * hB + g.C * gC;
  const float p00 = kg00 * g.A + kg01 * g.B, p01 = kg00 * g.B + kg01 * g.C;
  const float p10 = kg10 * g.A + kg11 * g.B, p11 = kg10 * g.B + kg11 * g.C;
  const float gV00 = -p00, gV01 = -(p01 + p10), gV11 = -p11;
  // V = T Sigma T^T: H = [[gV00, gV01/2], [gV01/2, gV11]]
  const float h00 = gV00, h01 = 0.5f * gV01, h11 = gV11;
  // U = H T (rows u0, u1)
  float u0[3], u1[3];
  for (int k = 0; k < 3; ++k) {
    u0[k] = h00 * g.t0[k] + h01 * g.t1[k];
    u1[k] = h01 * g.t0[k] + h11 * g.t1[k];
  }
  // dSigma = T^T H T = t0 u0^T + t1 u1^T (symmetric)
  float dS[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) dS[r][c] = g.t0[r] * u0[c] + g.t1[r] * u1[c];
  // dT = 2 H T Sigma = 2 U Sigma
  const float* S = g.Sig;
  const float Sf[3][3] = {{S[0], S[1], S[2]}, {S[1], S[3], S[4]}, {S[2], S[4], S[5]}};
  float dT0[3], dT1[3];
  for (int c = 0; c < 3; ++c) {
    dT0[c] = 2.0f * (u0[0] * Sf[0][c] + u0[1] * Sf[1][c] + u0[2] * Sf[2][c]);
    dT1[c] = 2.0f * (u1[0] * Sf[0][c] + u1[1] * Sf[1][c] + u1[2] * Sf[2][c]);
  }
  // T = J W: dJ = dT W^T; only J00, J02, J11, J12 depend on the position
  const float dJ00 = dT0[0] * cam.R[0] + dT0[1] * cam.R[1] + dT0[2] * cam.R[2];
  const float dJ02 = dT0[0] * cam.R[6] + dT0[1] * cam.R[7] + dT0[2] * cam.R[8];
  const float dJ11 = dT1[0] * cam.R[3] + dT1[1] * cam.R[4] + dT1[2] * cam.R[5];
  const float dJ12 = dT1[0] * cam.R[6] + dT1[1] * cam.R[7] + dT1[2] * cam.R[8];
  const float pz = g.p[2], pz2 = pz * pz, pz3 = pz2 * pz;
  const float fx = cam.fx, fy = cam.fy;
  const float dp0 = dJ02 * (-fx / pz2) + gu * fx / pz;
  const float dp1 = dJ12 * (-fy / pz2) + gv * fy / pz;
  const float dp2 = dJ00 * (-fx / pz2) + dJ02 * (2.0f * fx * g.p[0] / pz3) + dJ11 * (-fy / pz2) +
                    dJ12 * (2.0f * fy * g.p[1] / pz3) - gu * fx * g.p[0] / pz2 - gv * fy * g.p[1] / pz2;
  // p = W m + t: dm = W^T dp
  for (int c = 0; c < 3; ++c) gm[c] += cam.R[c] * dp0 + cam.R[3 + c] * dp1 + cam.R[6 + c] * dp2;
  for (int c = 0; c < 3; ++c) gparams[c * n + i] = gm[c];
  // Sigma = M M^T: dM = 2 dSigma M
  float dM[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c)
      dM[r][c] = 2.0f * (dS[r][0] * g.M[c] + dS[r][1] * g.M[3 + c] + dS[r][2] * g.M[6 + c]);
  // M = Rq diag(s): d log s_j = s_j sum_r dM_rj Rq_rj
  for (int j = 0; j < 3; ++j)
    gparams[(3 + j) * n + i] = (dM[0][j] * g.Rq[j] + dM[1][j] * g.Rq[3 + j] + dM[2][j] * g.Rq[6 + j]) * g.s[j];
  // dRq = dM diag(s), then the derivative of the unit-quaternion rotation matrix
  float dR[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) dR[r][c] = dM[r][c] * g.s[c];
  const float w = g.q[0], x = g.q[1], y = g.q[2], z = g.q[3];
  float gq[4];
  gq[0] = 2.0f * (-z * dR[0][1] + y * dR[0][2] + z * dR[1][0] - x * dR[1][2] - y * dR[2][0] + x * dR[2][1]);
  gq[1] = 2.0f * (y * dR[0][1] + z * dR[0][2] + y * dR[1][0] - 2.0f * x * dR[1][1] - w * dR[1][2] +
                  z * dR[2][0] + w * dR[2][1] - 2.0f * x * dR[2][2]);
  gq[2] = 2.0f * (-2.0f * y * dR[0][0] + x * dR[0][1] + w * dR[0][2] + x * dR[1][0] + z * dR[1][2] -
                  w * dR[2][0] + z * dR[2][1] - 2.0f * y * dR[2][2]);
  gq[3] = 2.0f * (-2.0f * z * dR[0][0] - w * dR[0][1] + x * dR[0][2] + w * dR[1][0] - 2.0f * z * dR[1][1] +
                  y * dR[1][2] + x * dR[2][0] + y * dR[2][1]);
  const float qd = (w * gq[0] + x * gq[1]) + (y * gq[2] + z * gq[3]);
  for (int k = 0; k < 4; ++k) gparams[(6 + k) * n + i] = (gq[k] - g.q[k] * qd) / g.ql;
}

}  // namespace

hipError_t launch_preprocess_fwd(const float* params, int n, int deg, const gs_camera& cam, const gs_proj& out,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(div_up(n, 256)), block(256);
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  float4* splat = reinterpret_cast<float4*>(out.splat);
  uint2* rect = reinterpret_cast<uint2*>(out.rect);
  switch (deg) {
    case 0: preprocess_fwd_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    case 1: preprocess_fwd_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    case 2: preprocess_fwd_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
    default: preprocess_fwd_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tx, ty, splat, out.depth, rect, out.tiles); break;
  }
  return hipGetLastError();
}

hipError_t launch_preprocess_bwd(const float* params, int n, int deg, const gs_camera& cam,
                                 const uint32_t* tiles, const float* gscreen, float* gparams, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(div_up(n, 256)), block(256);
  switch (deg) {
    case 0:
      chain_colour_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      chain_geometry_kernel<0><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      break;
    case 1:
      chain_colour_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      chain_geometry_kernel<1><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      break;
    case 2:
      chain_colour_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      chain_geometry_kernel<2><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      break;
    default:
      chain_colour_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      chain_geometry_kernel<3><<<grid, block, 0, s>>>(params, n, cam, tiles, gscreen, gparams);
      break;
  }
  return hipGetLastError();
}

}  // namespace gsk
