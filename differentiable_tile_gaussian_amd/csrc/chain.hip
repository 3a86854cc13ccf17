// Backward chain per Gaussian: screen-space gradients -> parameter gradients, and
// optionally Adam applied on the spot (without writing the gradient to memory).
//
// One block per group of 64 Gaussians (one group of the blocked layout), four waves:
//   waves 0-2  one colour channel each: the DC and band gradients of that channel
//              ([GSG] "Spherical harmonics": dL/dsh_k = dRGB Y_k; the clamp at zero
//              passes no gradient) and its share of the view-direction term;
//   wave 3     one thread per Gaussian: mean (projected-mean path, J(z) covariance
//              path, plus the direction term the colour waves leave in LDS),
//              log-scales, quaternion and opacity logit ([GSG] "From a pixel's blame
//              to the oval's shape and place", "The covariance chain", "Where the
//              position gradient comes from"; [GST] Jacobian slide).
// Wave 3 loads the geometry planes and hands the means and tile counts to the colour
// waves through LDS; every parameter, moment and screen-gradient byte crosses HBM once.
// gscreen: [n][9] per Gaussian: 0 u, 1 v, 2 A, 3 B, 4 C, 5 opacity, 6-8 colour (read only).
//
// With PROJ the block then projects its 64 updated Gaussians for the next camera, from
// the values it has just written (so they are not read back): wave 3 the geometry and
// view direction, waves 0-2 the colour of one channel each, wave 3 the record, as the
// projection kernel does (the same device functions).
//
// Compiled without floating-point contraction, like the forward projection, so the
// recomputed projection is the forward's bit for bit.
#include "adam_math.h"
#include "projection.h"
#include "profile.h"

namespace gsk {
namespace {

using namespace proj;

// Plane of colour coefficient k (0 = DC, 1.. = bands) of channel ch.
__device__ inline int colour_plane(int k, int ch) { return k == 0 ? 11 + ch : 14 + 3 * (k - 1) + ch; }

// What the camera-pose gradient needs of one Gaussian's chain: the gradients of T = J W
// (rows dT0, dT1), of the camera-space centre p, and the view-direction part of the mean's
// gradient; zero, with geom false, when the Gaussian is not visible.
struct CamPart {
  float p[3], dT0[3], dT1[3], dp[3], gsh[3];
  bool geom;
};

// The eleven geometry gradients of one Gaussian (mean, log-scales, quaternion, opacity
// logit) from its screen partials gs6 and the colour waves' view-direction partials; with
// cp, also what the camera-pose gradient needs.
template <int K>
__device__ inline void geometry_grads(const float* th, const float* gs6, uint32_t ntile, int lane,
                                      const gs_camera& cam, int mip, const float (*s_gdir)[3][64], float* gp,
                                      CamPart* cp) {
#pragma unroll
  for (int k = 0; k < 11; ++k) gp[k] = 0.0f;
  if (cp) {
#pragma unroll
    for (int k = 0; k < 3; ++k) cp->p[k] = cp->dT0[k] = cp->dT1[k] = cp->dp[k] = cp->gsh[k] = 0.0f;
    cp->geom = false;
  }
  if (K > 0 && ntile != 0u) {
    // the colour's view-direction term, projected off the unit direction
    float dir[3];
    const float dlen = view_dir_from(th[0], th[1], th[2], cam, dir);
    float gt[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) gt[c] = s_gdir[0][c][lane] + s_gdir[1][c][lane] + s_gdir[2][c][lane];
    const float dd = dir[0] * gt[0] + dir[1] * gt[1] + dir[2] * gt[2];
#pragma unroll
    for (int c = 0; c < 3; ++c) gp[c] = (gt[c] - dir[c] * dd) / dlen;
    if (cp)
      for (int c = 0; c < 3; ++c) cp->gsh[c] = gp[c];
  }
  Proj g;
  if (ntile != 0u && project_geometry_from(th, cam, mip, g)) {
    const float gu = gs6[0], gv = gs6[1], gA = gs6[2], gB = gs6[3], gC = gs6[4], go = gs6[5];
    // opacity logit through the sigmoid (and the compensation factor when it is on)
    gp[10] = mip ? go * g.comp * g.ob * (1.0f - g.ob) : go * g.o * (1.0f - g.o);
    // conic -> dilated covariance: dV' = -K Gk K with Gk = [[gA, gB/2], [gB/2, gC]]
    const float hB = 0.5f * gB;
    const float kg00 = g.A * gA + g.B * hB, kg01 = g.A * hB + g.B * gC;
    const float kg10 = g.B * gA + g.C * hB, kg11 = g.B * hB + g.C * gC;
    const float p00 = kg00 * g.A + kg01 * g.B, p01 = kg00 * g.B + kg01 * g.C;
    const float p10 = kg10 * g.A + kg11 * g.B, p11 = kg10 * g.B + kg11 * g.C;
    float gV00 = -p00, gV01 = -(p01 + p10), gV11 = -p11;
    if (mip && g.detv > 0.0f) {
      // comp = sqrt(det V / det V'), V' = V + 0.3 I: d comp = comp / 2 (d det V / det V -
      // d det V' / det V'), d det V = (v11, -2 b, v00) . (d v00, d b, d v11), and for V' (c, -2 b, a)
      const float gcomp = go * g.ob;
      const float h = 0.5f * g.comp;
      gV00 += gcomp * h * (g.v11 / g.detv - g.c / g.det);
      gV11 += gcomp * h * (g.v00 / g.detv - g.a / g.det);
      gV01 += gcomp * h * (2.0f * g.b / g.det - 2.0f * g.b / g.detv);
    }
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
    for (int c = 0; c < 3; ++c) gp[c] += cam.R[c] * dp0 + cam.R[3 + c] * dp1 + cam.R[6 + c] * dp2;
    if (cp) {
      cp->geom = true;
      for (int c = 0; c < 3; ++c) {
        cp->p[c] = g.p[c];
        cp->dT0[c] = dT0[c];
        cp->dT1[c] = dT1[c];
      }
      cp->dp[0] = dp0;
      cp->dp[1] = dp1;
      cp->dp[2] = dp2;
    }
    // Sigma = M M^T: dM = 2 dSigma M
    float dM[3][3];
    for (int r = 0; r < 3; ++r)
      for (int c = 0; c < 3; ++c)
        dM[r][c] = 2.0f * (dS[r][0] * g.M[c] + dS[r][1] * g.M[3 + c] + dS[r][2] * g.M[6 + c]);
    // M = Rq diag(s): d log s_j = s_j sum_r dM_rj Rq_rj
    for (int j = 0; j < 3; ++j)
      gp[3 + j] = (dM[0][j] * g.Rq[j] + dM[1][j] * g.Rq[3 + j] + dM[2][j] * g.Rq[6 + j]) * g.s[j];
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
    for (int k = 0; k < 4; ++k) gp[6 + k] = (gq[k] - g.q[k] * qd) / g.ql;
  }
}

// A gradient written without Adam: gw g, or added to what is there (several views of one
// step summed into one gradient).  With gw = 1 and no accumulation the value itself.
__device__ inline void put_grad(float* __restrict__ gparams, size_t o, float g, float gw, int gacc) {
  gparams[o] = gacc ? gparams[o] + gw * g : gw * g;
}

// Wave 3's part after the colour waves: the geometry gradients and their Adam update
// (th returns the updated values).
template <int K, bool ADAM>
__device__ inline void geometry_tail(float* th, const float* gs6, float* mo, float* vo, uint32_t ntile, int lane,
                                     size_t gb, const gs_camera& cam, int mip, const float (*s_gdir)[3][64],
                                     float* __restrict__ params, float* __restrict__ gparams, float gw, int gacc,
                                     float* __restrict__ m, float* __restrict__ v, const AdamArgs& a) {
  float gp[11];
  geometry_grads<K>(th, gs6, ntile, lane, cam, mip, s_gdir, gp, nullptr);
#pragma unroll
  for (int pl = 0; pl < 11; ++pl) {
    const size_t o = gb + pl * kGB;
    if (ADAM) {
      th[pl] = adam_update(th[pl], gp[pl], mo[pl], vo[pl], a.lr[adam_group(pl)], a);
      __builtin_nontemporal_store(th[pl], params + o);
      __builtin_nontemporal_store(mo[pl], m + o);
      __builtin_nontemporal_store(vo[pl], v + o);
    } else {
      put_grad(gparams, o, gp[pl], gw, gacc);
    }
  }
}


template <int DEG, bool ADAM, bool PROJ>
__global__ void __launch_bounds__(256) chain_kernel(float* __restrict__ params, int n, gs_camera cam,
                                                     const uint32_t* tiles,   // may be np.tiles
                                                     const float* __restrict__ gscreen, float* __restrict__ gparams,
                                                     float gw, int gacc,
                                                     float* __restrict__ m, float* __restrict__ v, AdamArgs a,
                                                     NextProj np, float2* __restrict__ dstats, Shade shade) {
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  constexpr int P = 11 + 3 * (K + 1);
  __shared__ float s_gdir[3][3][64];   // view-direction partials of each colour channel
  __shared__ float s_mean[3][64];
  __shared__ uint32_t s_tile[64];
  __shared__ float s_ndir[PROJ ? 3 : 1][64];   // next camera: view direction, colour before the clamp
  __shared__ float s_nraw[PROJ ? 3 : 1][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  const bool valid = i < n;
  // This block's 64 Gaussians are one group of the blocked layout: each plane is a
  // contiguous 256-byte row.  Waves 0-2 take the colour planes of one channel each,
  // wave 3 the eleven geometry planes.  Every load of a lane is issued before any
  // arithmetic (the pass is a stream; a load that waited on another would add a
  // memory round trip).  (Separate code paths per wave kind, with the barriers
  // inside each, use fewer registers but ran slower.)
  const size_t gb = size_t(blockIdx.x) * P * kGB + lane;
  const int ch = wv;   // colour waves
  uint32_t ntile = 0;
  float th[11], gs6[6], mo[ADAM ? 11 : 1], vo[ADAM ? 11 : 1];
  float coef[K + 1], cmo[ADAM ? K + 1 : 1], cvo[ADAM ? K + 1 : 1];
  float gcol = 0.0f;
  if (wv == 3) {
    if (valid) {
      ntile = tiles[i];
#pragma unroll
      for (int k = 0; k < 11; ++k) th[k] = __builtin_nontemporal_load(params + gb + k * kGB);
#pragma unroll
      for (int k = 0; k < 6; ++k) gs6[k] = gscreen[size_t(i) * 9 + k];
      if (ADAM) {
#pragma unroll
        for (int k = 0; k < 11; ++k) {
          mo[k] = __builtin_nontemporal_load(m + gb + k * kGB);
          vo[k] = __builtin_nontemporal_load(v + gb + k * kGB);
        }
      }
    }
    s_tile[lane] = ntile;
#pragma unroll
    for (int c = 0; c < 3; ++c) s_mean[c][lane] = valid ? th[c] : 0.0f;
  } else if (valid) {
#pragma unroll
    for (int k = 0; k <= K; ++k) coef[k] = __builtin_nontemporal_load(params + gb + colour_plane(k, ch) * kGB);
    gcol = gscreen[size_t(i) * 9 + 6 + ch];
    if (ADAM) {
#pragma unroll
      for (int k = 0; k <= K; ++k) {
        const size_t o = gb + colour_plane(k, ch) * kGB;
        cmo[k] = __builtin_nontemporal_load(m + o);
        cvo[k] = __builtin_nontemporal_load(v + o);
      }
    }
  }
  __syncthreads();   // tile counts and means
  if (wv < 3) {
    const bool vis = valid && s_tile[lane] != 0u;
    float dir[3] = {0.f, 0.f, 0.f};
    float Y[16];
    if (K > 0 && vis) {
      view_dir_from(s_mean[0][lane], s_mean[1][lane], s_mean[2][lane], cam, dir);
      sh_eval(dir[0], dir[1], dir[2], Y);
    }
    float gc = 0.0f;
    if (vis) {
      float raw = coef[0];
#pragma unroll
      for (int k = 1; k <= K; ++k)
        if (k <= shade.kact) raw = raw + coef[k] * Y[k];
      gc = raw < 0.0f ? 0.0f : gcol;
    }
    if (K > 0) {
      float gd[3] = {0.f, 0.f, 0.f};
      if (vis) {
        float wk[16];
#pragma unroll
        for (int k = 1; k <= K; ++k) wk[k] = gc * coef[k];
        sh_grad_dot(dir[0], dir[1], dir[2], wk, shade.kact, gd);   // the active bands only
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) s_gdir[ch][c][lane] = gd[c];
    }
    if (valid) {
#pragma unroll
      for (int k = 0; k <= K; ++k) {
        const float g = k == 0 ? gc : (vis && k <= shade.kact ? gc * Y[k] : 0.0f);
        const size_t o = gb + colour_plane(k, ch) * kGB;
        if (ADAM) {
          coef[k] = adam_update(coef[k], g, cmo[k], cvo[k], a.lr[4], a);
          __builtin_nontemporal_store(coef[k], params + o);
          __builtin_nontemporal_store(cmo[k], m + o);
          __builtin_nontemporal_store(cvo[k], v + o);
        } else {
          put_grad(gparams, o, g, gw, gacc);
        }
      }
    }
  }
  __syncthreads();   // view-direction partials of the three channels
  if (wv == 3 && valid) {
    if (dstats && ntile != 0u) {   // density statistics: this observation's |(du, dv)| and 1
      float2 st = dstats[i];
      st.x += sqrtf(gs6[0] * gs6[0] + gs6[1] * gs6[1]);
      st.y += 1.0f;
      dstats[i] = st;
    }
    geometry_tail<K, ADAM>(th, gs6, mo, vo, ntile, lane, gb, cam, shade.mip, s_gdir, params, gparams, gw, gacc, m, v,
                           a);
  }
  if (!PROJ) return;
  // ---- projection of the updated Gaussians for the next camera
  Proj g;
  bool geom = false;
  if (wv == 3) {
    if (valid) {
      geom = project_geometry_from(th, np.cam, shade.mip, g);
      if (K > 0) {
        float dir[3];
        view_dir_from(th[0], th[1], th[2], np.cam, dir);
#pragma unroll
        for (int c = 0; c < 3; ++c) s_ndir[c][lane] = dir[c];
      }
    }
  }
  __syncthreads();   // next view directions
  if (wv < 3 && valid) {
    float Y[16];
    if (K > 0) sh_eval(s_ndir[0][lane], s_ndir[1][lane], s_ndir[2][lane], Y);
    float raw = coef[0];
#pragma unroll
    for (int k = 1; k <= K; ++k)
      if (k <= shade.kact) raw = raw + coef[k] * Y[k];
    s_nraw[ch][lane] = raw;
  }
  __syncthreads();   // next colours
  if (wv != 3) return;
  Record r;
  uint32_t cnt = 0u;
  if (valid) {
    const float raw[3] = {s_nraw[0][lane], s_nraw[1][lane], s_nraw[2][lane]};
    make_record(geom, g, raw, np.tx, np.ty, r);
    store_record(r, i, np.splat, np.depth, np.rect, np.tiles);
    cnt = r.tiles;
  }
  // this block's tile count (the pair count is the sum over blocks)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
  if (lane == 0) np.block_tiles[blockIdx.x] = cnt;
  if (blockIdx.x == 0 && lane == 0) *np.total = 0u;   // the per-block sums are added after this kernel
}

template <int DEG, bool ADAM, bool PROJ>
void launch_chain_deg(float* params, int n, const gs_camera& cam, const uint32_t* tiles, const float* gscreen,
                      float* gparams, float gw, int gacc, float* m, float* v, const AdamArgs& a, const NextProj& np,
                      float* dstats, Shade shade, hipStream_t s) {
  GSK_PROF("chain", s);
  chain_kernel<DEG, ADAM, PROJ><<<div_up(n, 64), 256, 0, s>>>(params, n, cam, tiles, gscreen, gparams, gw, gacc, m,
                                                              v, a, np, reinterpret_cast<float2*>(dstats), shade);
}

template <bool ADAM, bool PROJ>
void launch_chain_mode(float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles, const float* gscreen,
                       float* gparams, float gw, int gacc, float* m, float* v, const AdamArgs& a, const NextProj& np,
                       float* dstats, Shade shade, hipStream_t s) {
  switch (deg) {
#define GSK_CHAIN_CASE(D) \
    launch_chain_deg<D, ADAM, PROJ>(params, n, cam, tiles, gscreen, gparams, gw, gacc, m, v, a, np, dstats, shade, s)
    case 0: GSK_CHAIN_CASE(0); break;
    case 1: GSK_CHAIN_CASE(1); break;
    case 2: GSK_CHAIN_CASE(2); break;
    default: GSK_CHAIN_CASE(3); break;
#undef GSK_CHAIN_CASE
  }
}

// ---------------------------------------------------------------- camera-pose gradient
// [GSG] "Forgiving the camera and the light": the loss's gradient with respect to the
// camera pose, the rotation W perturbed on the left (W <- (I + [w]x) W) and the translation
// t.  Every Gaussian reaches the pose three ways: through T = J W of its covariance, through
// its camera-space centre p = W m + t, and through the view direction of its colour (the
// camera centre is -W^T t).  With G = J^T dT + dp m^T + t gsh^T (gsh: the view-direction
// part of the mean's gradient, so the centre's gradient is -gsh), dL/dW = G and
//   dL/dw = (M21 - M12, M02 - M20, M10 - M01) with M = G W^T,   dL/dt = dp + W gsh.
// For the position path alone the rotation term is (p - t) x dp, the pages' torque, and the
// translation's dp: the trainer's code accumulates exactly those (position_only).
// The per-Gaussian terms are formed in fp32 from the fp32 chain quantities (one fixed
// sequence of roundings: this file is compiled without contraction) and summed in double,
// per wave with a fixed butterfly and over blocks in a fixed order, so the result is
// reproducible; the terms' own rounding is below that of the chain quantities they are
// formed from.
__device__ inline void camera_terms(const CamPart& c, const float* mean, const gs_camera& cam, int position_only,
                                    double* out) {
  float G[3][3];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int k = 0; k < 3; ++k) G[r][k] = c.dp[r] * mean[k];
  float tr[3] = {c.dp[0], c.dp[1], c.dp[2]};
  if (!position_only) {
    const float iz = 1.0f / c.p[2];
    const float j00 = cam.fx * iz, j11 = cam.fy * iz;
    const float J[2][3] = {{j00, 0.0f, -(j00 * c.p[0]) * iz}, {0.0f, j11, -(j11 * c.p[1]) * iz}};
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k)
        G[r][k] = ((J[0][r] * c.dT0[k] + J[1][r] * c.dT1[k]) + G[r][k]) + cam.t[r] * c.gsh[k];
#pragma unroll
    for (int r = 0; r < 3; ++r)
      tr[r] = ((tr[r] + cam.R[3 * r] * c.gsh[0]) + cam.R[3 * r + 1] * c.gsh[1]) + cam.R[3 * r + 2] * c.gsh[2];
  }
  float M[3][3];
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      M[r][k] = (G[r][0] * cam.R[3 * k] + G[r][1] * cam.R[3 * k + 1]) + G[r][2] * cam.R[3 * k + 2];
  out[0] = double(M[2][1] - M[1][2]);
  out[1] = double(M[0][2] - M[2][0]);
  out[2] = double(M[1][0] - M[0][1]);
#pragma unroll
  for (int r = 0; r < 3; ++r) out[3 + r] = double(tr[r]);
}

// One block per group of 64 Gaussians, the chain kernel's split: waves 0-2 the view-direction
// partial of one colour channel each, wave 3 the geometry path and the six terms.  Writes
// the block's sums to part[k * nb + block].
template <int DEG>
__global__ void __launch_bounds__(256) camera_grad_kernel(const float* __restrict__ params, int n, gs_camera cam,
                                                           const uint32_t* __restrict__ tiles,
                                                           const float* __restrict__ gscreen,
                                                           double* __restrict__ part, Shade shade,
                                                           int position_only) {
  constexpr int K = (DEG + 1) * (DEG + 1) - 1;
  constexpr int P = 11 + 3 * (K + 1);
  __shared__ float s_gdir[3][3][64];
  __shared__ float s_mean[3][64];
  __shared__ uint32_t s_tile[64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  const bool valid = i < n;
  const size_t gb = size_t(blockIdx.x) * P * kGB + lane;
  float th[11], gs6[6];
  uint32_t ntile = 0;
  if (wv == 3) {
    if (valid) {
      ntile = tiles[i];
#pragma unroll
      for (int k = 0; k < 11; ++k) th[k] = params[gb + k * kGB];
#pragma unroll
      for (int k = 0; k < 6; ++k) gs6[k] = gscreen[size_t(i) * 9 + k];
    }
    s_tile[lane] = ntile;
#pragma unroll
    for (int c = 0; c < 3; ++c) s_mean[c][lane] = valid ? th[c] : 0.0f;
  }
  __syncthreads();
  if (K > 0 && wv < 3) {
    const int ch = wv;
    float gd[3] = {0.f, 0.f, 0.f};
    if (valid && s_tile[lane] != 0u) {
      float coef[K + 1];
#pragma unroll
      for (int k = 0; k <= K; ++k) coef[k] = params[gb + colour_plane(k, ch) * kGB];
      float dir[3], Y[16];
      view_dir_from(s_mean[0][lane], s_mean[1][lane], s_mean[2][lane], cam, dir);
      sh_eval(dir[0], dir[1], dir[2], Y);
      float raw = coef[0];
#pragma unroll
      for (int k = 1; k <= K; ++k)
        if (k <= shade.kact) raw = raw + coef[k] * Y[k];
      const float gc = raw < 0.0f ? 0.0f : gscreen[size_t(i) * 9 + 6 + ch];
      float wk[16];
#pragma unroll
      for (int k = 1; k <= K; ++k) wk[k] = gc * coef[k];
      sh_grad_dot(dir[0], dir[1], dir[2], wk, shade.kact, gd);
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) s_gdir[ch][c][lane] = gd[c];
  }
  __syncthreads();
  if (wv != 3) return;
  double t6[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (valid && ntile != 0u) {
    float gp[11];
    CamPart cp;
    geometry_grads<K>(th, gs6, ntile, lane, cam, shade.mip, s_gdir, gp, &cp);
    if (cp.geom) camera_terms(cp, th, cam, position_only, t6);
  }
#pragma unroll
  for (int k = 0; k < 6; ++k)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t6[k] += __shfl_xor(t6[k], d, 64);
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < 6; ++k) part[size_t(k) * gridDim.x + blockIdx.x] = t6[k];
}

// out[k] = sum over the nb block sums of component k, one block per component, each
// thread a fixed stride of them, then a fixed tree.
__global__ void __launch_bounds__(1024) camera_grad_finalize_kernel(const double* __restrict__ part, int nb,
                                                                    double* __restrict__ out) {
  __shared__ double s[1024];
  const int k = blockIdx.x, t = threadIdx.x;
  double acc = 0.0;
#pragma unroll 8
  for (int b = t; b < nb; b += 1024) acc += part[size_t(k) * nb + b];   // loads issued eight ahead
  s[t] = acc;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if (t < w) s[t] += s[t + w];
    __syncthreads();
  }
  if (t == 0) out[k] = s[0];
}

}  // namespace

size_t camera_grad_ws_bytes(int64_t n) { return size_t(div_up(n, 64)) * 6 * sizeof(double); }

hipError_t launch_camera_grad(const float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                              const float* gscreen, int position_only, double* out, void* ws, Shade shade,
                              hipStream_t s) {
  double* part = static_cast<double*>(ws);
  if (n == 0) {
    camera_grad_finalize_kernel<<<6, 1024, 0, s>>>(part, 0, out);
    return hipGetLastError();
  }
  const int nb = int(div_up(n, 64));
  {
    GSK_PROF("camera_grad", s);
    switch (deg) {
      case 0: camera_grad_kernel<0><<<nb, 256, 0, s>>>(params, n, cam, tiles, gscreen, part, shade, position_only); break;
      case 1: camera_grad_kernel<1><<<nb, 256, 0, s>>>(params, n, cam, tiles, gscreen, part, shade, position_only); break;
      case 2: camera_grad_kernel<2><<<nb, 256, 0, s>>>(params, n, cam, tiles, gscreen, part, shade, position_only); break;
      default: camera_grad_kernel<3><<<nb, 256, 0, s>>>(params, n, cam, tiles, gscreen, part, shade, position_only); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  camera_grad_finalize_kernel<<<6, 1024, 0, s>>>(part, nb, out);
  return hipGetLastError();
}

hipError_t launch_preprocess_bwd(const float* params, int n, int deg, const gs_camera& cam,
                                 const uint32_t* tiles, const float* gscreen, float* gparams, Shade shade,
                                 hipStream_t s, float weight, int accumulate) {
  if (n == 0) return hipSuccess;
  launch_chain_mode<false, false>(const_cast<float*>(params), n, deg, cam, tiles, gscreen, gparams, weight,
                                  accumulate, nullptr, nullptr, AdamArgs{}, NextProj{}, nullptr, shade, s);
  return hipGetLastError();
}

hipError_t launch_chain_adam(float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                             const float* gscreen, float* m, float* v, const AdamArgs& a, Shade shade, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_chain_mode<true, false>(params, n, deg, cam, tiles, gscreen, nullptr, 1.0f, 0, m, v, a, NextProj{}, nullptr,
                                 shade, s);
  return hipGetLastError();
}

hipError_t launch_chain_adam_project(float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                                     const float* gscreen, float* m, float* v, const AdamArgs& a,
                                     const NextProj& np, float* dstats, Shade shade, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_chain_mode<true, true>(params, n, deg, cam, tiles, gscreen, nullptr, 1.0f, 0, m, v, a, np, dstats, shade,
                                s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_tile_count_total(np.block_tiles, int(div_up(n, 64)), np.total, s);
}

}  // namespace gsk
