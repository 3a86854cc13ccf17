// Projection of one Gaussian and its spherical-harmonic colour: the device
// functions shared by the forward projection (preprocess.hip) and the backward
// chain (chain.hip).  Both translation units are compiled without floating-point
// contraction, so the chain recomputes exactly the values the forward produced.
//
// Pages (titles as they appear on the pages):
//   [DR]  "Differentiable rasterisation";  [GST] Gaussian splatting training study deck;
//   [GSG] "How a computer rebuilds a real place out of soft colored dots called Gaussian Splats".
#pragma once

#include "gs_internal.h"

namespace gsk {
namespace proj {


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
  float o;               // the record's opacity: ob comp with the Mip compensation, else ob
  float ob, comp;        // sigmoid of the logit; the compensation factor (1 when off)
  float v00, v11, detv;  // undilated screen covariance (its off-diagonal is b) and determinant
};

// Geometry of one Gaussian ([GST] parameter and Jacobian slides; [DR] "Forward";
// [GSG] "Flattening a 3D blob into a 2D oval").  Returns false when culled (behind the
// near plane, zero quaternion, non-positive determinant).
// th: the 11 geometry parameters (mean 0-2, log-scales 3-5, quaternion 6-9, logit 10).
// mip: the opacity is multiplied by comp = sqrt(det V / det(V + 0.3 I)) ([GSG] same section:
// the Mip-Splatting correction against the extra brightness the dilation gives very small
// Gaussians; this ratio gives the dilated footprint exactly the integral of the undilated
// one), 0 when det V <= 0.
__device__ inline bool project_geometry_from(const float* th, const gs_camera& cam, int mip, Proj& g) {
  const float mx = th[0], my = th[1], mz = th[2];
  for (int r = 0; r < 3; ++r)
    g.p[r] = ((cam.R[3 * r] * mx + cam.R[3 * r + 1] * my) + cam.R[3 * r + 2] * mz) + cam.t[r];
  if (!(g.p[2] > cam.znear)) return false;
  g.xz = g.p[0] / g.p[2];
  g.yz = g.p[1] / g.p[2];
  g.u = cam.fx * g.xz + cam.cx;
  g.v = cam.fy * g.yz + cam.cy;
  for (int k = 0; k < 3; ++k) g.s[k] = float(exp(double(th[3 + k])));
  const float qw = th[6], qx = th[7], qy = th[8], qz = th[9];
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
  g.ob = float(1.0 / (1.0 + exp(-double(th[10]))));
  g.v00 = V00;
  g.v11 = V11;
  g.detv = V00 * V11 - V01 * V01;
  g.comp = 1.0f;
  g.o = g.ob;
  if (mip) {
    g.comp = sqrtf(fmaxf(g.detv, 0.0f) / g.det);
    g.o = g.ob * g.comp;
  }
  return true;
}

// The same, reading the 11 geometry planes of one Gaussian; g0 = gaussian_base(params, i, P).
__device__ inline bool project_geometry(const float* __restrict__ g0, const gs_camera& cam, int mip, Proj& g) {
  float th[11];
#pragma unroll
  for (int k = 0; k < 11; ++k) th[k] = g0[k * kGB];
  return project_geometry_from(th, cam, mip, g);
}

// View direction dir = normalize(mean - campos) and its length ([GSG] "Spherical harmonics").
__device__ inline float view_dir_from(float mx, float my, float mz, const gs_camera& cam, float* dir) {
  const float d0 = mx - cam.campos[0], d1 = my - cam.campos[1], d2 = mz - cam.campos[2];
  const float len = sqrtf((d0 * d0 + d1 * d1) + d2 * d2);
  dir[0] = d0 / len;
  dir[1] = d1 / len;
  dir[2] = d2 / len;
  return len;
}

__device__ inline float view_dir(const float* __restrict__ g0, const gs_camera& cam, float* dir) {
  return view_dir_from(g0[0], g0[kGB], g0[2 * kGB], cam, dir);
}

// Colour before the clamp: DC + sum_k sh_k Y_k over the active bands k <= kact of the K
// stored ones.  The loop runs over the stored bands (unrolled, every load issued up
// front) and an inactive band's term is dropped by a select, so the sum is formed with
// the same roundings as a loop over the active bands alone.
template <int K>
__device__ inline void sh_colour(const float* __restrict__ g0, int kact, const float* Y, float* raw) {
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    float col = g0[(11 + ch) * kGB];
#pragma unroll
    for (int k = 1; k <= K; ++k) {
      const float t = g0[(14 + 3 * (k - 1) + ch) * kGB] * Y[k];
      col = k <= kact ? col + t : col;
    }
    raw[ch] = col;
  }
}

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

// A Gaussian's projected record (the gs_proj entries), zero when culled.
struct Record {
  float4 r0, r1, r2;   // u, v, A, B | C, o, r, g | b, hx, hy, tm
  float depth;
  uint2 rect;          // x0 | y0 << 16, x1 | y1 << 16
  uint32_t tiles;
};

// The record from the geometry (geom: project_geometry_from succeeded) and the colour
// before the clamp: clamped colour, culling of non-finite values, the opacity-aware
// extent and tile rectangle ([GSG] "Why tiling": rad = sqrt(2 eMax) sqrt(lambda_max)),
// and the blend box.
__device__ inline void make_record(bool geom, const Proj& g, const float* raw, int tx, int ty, Record& out) {
  bool vis = geom;
  float rgb[3] = {0.f, 0.f, 0.f};
  uint32_t x0 = 0, y0 = 0, x1 = 0, y1 = 0, cnt = 0;
  if (vis) {
    bool finite = __builtin_isfinite(g.u) && __builtin_isfinite(g.v) && __builtin_isfinite(g.A) &&
                  __builtin_isfinite(g.B) && __builtin_isfinite(g.C) && __builtin_isfinite(g.o);
    for (int ch = 0; ch < 3; ++ch) {
      rgb[ch] = fmaxf(raw[ch], 0.0f);
      finite = finite && __builtin_isfinite(rgb[ch]);
    }
    vis = finite;
    if (vis) {
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
    out.r0 = make_float4(g.u, g.v, g.A, g.B);
    out.r1 = make_float4(g.C, g.o, rgb[0], rgb[1]);
    float hx, hy, tm;
    blend_box(g, hx, hy, tm);
    out.r2 = make_float4(rgb[2], hx, hy, tm);
    out.depth = g.p[2];
    out.rect = make_uint2(x0 | (y0 << 16), x1 | (y1 << 16));
    out.tiles = cnt;
  } else {
    out.r0 = out.r1 = out.r2 = make_float4(0.f, 0.f, 0.f, 0.f);
    out.depth = 0.0f;
    out.rect = make_uint2(0u, 0u);
    out.tiles = 0u;
  }
}

__device__ inline void store_record(const Record& r, int i, float4* __restrict__ splat, float* __restrict__ depth,
                                    uint2* __restrict__ rect, uint32_t* __restrict__ tiles) {
  splat[3 * i + 0] = r.r0;
  splat[3 * i + 1] = r.r1;
  splat[3 * i + 2] = r.r2;
  depth[i] = r.depth;
  rect[i] = r.rect;
  tiles[i] = r.tiles;
}

}  // namespace proj
}  // namespace gsk
