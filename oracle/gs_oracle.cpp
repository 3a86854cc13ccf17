// CPU oracle for the tile-based differentiable Gaussian rasteriser.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
// load this file; only the tests, the smoke check and the CPU-baseline leg of
// the benchmark do.  It shares no code, header, table or constant generator
// with the HIP library.
//
// It is deliberately plain: single-threaded loops, one Gaussian or one pixel at
// a time, in the order the pages describe.  Every routine is a template on the
// floating-point type R:
//   * R = float  is the parity instantiation.  The pages' trainer computes in
//     32-bit floats, and every threshold decision (cull, tile rectangle, alpha
//     skip, early stop, alpha cap) is taken in that precision.  exp, log and the
//     sigmoid are evaluated in double and rounded once to float, so that the
//     tile keys are a function of IEEE arithmetic alone.
//   * R = double is used for finite-difference checks of the gradients.
//
// Pages cited (titles as they appear on the pages):
//   [DR]   "Differentiable rasterisation" (splat-report knowledge base)
//   [TBDR] "Tile-based differentiable rasterization in 3DGS" (learn-ml-visualized)
//   [GST]  Gaussian splatting training study deck (bailiping.com)
//   [GSG]  "How a computer rebuilds a real place out of soft colored dots called
//          Gaussian Splats" (taosengine guide)
//   [LAB]  Gaussian splatting training live lab (bailiping.com)
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -shared -fPIC.

#include <algorithm>
#include <utility>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// ---------------------------------------------------------------- constants
constexpr int kTile = 16;                 // [GSG] "Why tiling, and the five stages"; [DR] "The trick"
constexpr double kDilation = 0.3;         // [GST] slide "J is the 2 x 3 Jacobian of perspective projection"
constexpr double kExtentCut = 4.5;        // [GSG] "Why tiling" (E_CUT)
constexpr double kExtentLogFloor = 1.0001;// [GSG] "Why tiling" (floor inside the extent log)
constexpr double kTStop = 1e-4;           // [GSG] "The painting itself: front-to-back alpha compositing"
constexpr double kAlphaCap = 0.99;        // [GST] opacity slide; [GSG] "The painting itself"
constexpr double kAlphaMinInv = 255.0;    // [GST] opacity slide: skip below 1/255

template <class R> inline R alpha_min() { return R(1) / R(kAlphaMinInv); }

struct Camera {          // same field order as the ctypes structure in oracle.py
  float R[9];            // world -> camera rotation, row-major
  float t[3];
  float campos[3];       // camera centre in world coordinates
  float fx, fy, cx, cy;
  int32_t width, height;
  float znear;
  float bg[3];
};

inline int tiles_x(const Camera& c) { return (c.width + kTile - 1) / kTile; }
inline int tiles_y(const Camera& c) { return (c.height + kTile - 1) / kTile; }

// exp and the sigmoid, evaluated in double and rounded once to R.
template <class R> inline R exp_r(R x) { return R(std::exp(double(x))); }
template <class R> inline R sigmoid_r(R x) { return R(1.0 / (1.0 + std::exp(-double(x)))); }

// ------------------------------------------------------ spherical harmonics
// Real spherical harmonics with the Condon-Shortley sign convention, which is
// the convention of the degree-1 and degree-2 bands printed in [GSG]
// "Spherical harmonics: color that changes with viewing angle".
//   N(l, m) = sqrt((2l+1)/(4 pi) * (l-m)!/(l+m)!) * (m > 0 ? sqrt(2) : 1)
// times the associated-Legendre polynomial written in (x, y, z) of a unit vector.
double sh_norm(int l, int m) {
  double r = 1.0;
  for (int k = l - m + 1; k <= l + m; ++k) r /= double(k);
  double v = std::sqrt((2.0 * l + 1.0) / (4.0 * M_PI) * r);
  return m == 0 ? v : v * std::sqrt(2.0);
}

// Y[k] for k = 1..15 (Y[0] unused: the DC term is a colour, not multiplied by a basis
// function) and the gradient of each polynomial with respect to (x, y, z).
// Order: band 1 = (y, z, x), band 2 = (xy, yz, 2z^2-x^2-y^2, xz, x^2-y^2), band 3 = m -3..3.
template <class R>
void sh_basis(const R d[3], R Y[16], R dY[16][3]) {
  const R x = d[0], y = d[1], z = d[2];
  for (int k = 0; k < 16; ++k) { Y[k] = R(0); dY[k][0] = dY[k][1] = dY[k][2] = R(0); }
  // band 1: P_1^0 = z, P_1^1 = -sin(theta)
  const R n10 = R(sh_norm(1, 0)), n11 = R(-sh_norm(1, 1));
  Y[1] = n11 * y;  dY[1][1] = n11;
  Y[2] = n10 * z;  dY[2][2] = n10;
  Y[3] = n11 * x;  dY[3][0] = n11;
  // band 2: P_2^0 = (3z^2-1)/2, P_2^1 = -3 z sin, P_2^2 = 3 sin^2
  const R k4 = R(sh_norm(2, 2) * 6.0);   // 2xy from sin(2 phi) sin^2
  const R k5 = R(-sh_norm(2, 1) * 3.0);
  const R k6 = R(sh_norm(2, 0) * 0.5);
  const R k8 = R(sh_norm(2, 2) * 3.0);
  Y[4] = k4 * x * y;   dY[4][0] = k4 * y;  dY[4][1] = k4 * x;
  Y[5] = k5 * y * z;   dY[5][1] = k5 * z;  dY[5][2] = k5 * y;
  Y[6] = k6 * (R(2) * z * z - x * x - y * y);
  dY[6][0] = k6 * R(-2) * x; dY[6][1] = k6 * R(-2) * y; dY[6][2] = k6 * R(4) * z;
  Y[7] = k5 * x * z;   dY[7][0] = k5 * z;  dY[7][2] = k5 * x;
  Y[8] = k8 * (x * x - y * y);  dY[8][0] = k8 * R(2) * x;  dY[8][1] = k8 * R(-2) * y;
  // band 3: P_3^0 = z(5z^2-3)/2, P_3^1 = -(3/2)(5z^2-1) sin, P_3^2 = 15 z sin^2, P_3^3 = -15 sin^3
  const R k9 = R(-sh_norm(3, 3) * 15.0);
  const R k10 = R(sh_norm(3, 2) * 30.0);
  const R k11 = R(-sh_norm(3, 1) * 1.5);
  const R k12 = R(sh_norm(3, 0) * 0.5);
  const R k14 = R(sh_norm(3, 2) * 15.0);
  // m = -3: y(3x^2 - y^2)
  Y[9] = k9 * y * (R(3) * x * x - y * y);
  dY[9][0] = k9 * R(6) * x * y; dY[9][1] = k9 * (R(3) * x * x - R(3) * y * y);
  // m = -2: xyz
  Y[10] = k10 * x * y * z;
  dY[10][0] = k10 * y * z; dY[10][1] = k10 * x * z; dY[10][2] = k10 * x * y;
  // m = -1: y(4z^2 - x^2 - y^2)
  Y[11] = k11 * y * (R(4) * z * z - x * x - y * y);
  dY[11][0] = k11 * R(-2) * x * y;
  dY[11][1] = k11 * (R(4) * z * z - x * x - R(3) * y * y);
  dY[11][2] = k11 * R(8) * y * z;
  // m = 0: z(2z^2 - 3x^2 - 3y^2)
  Y[12] = k12 * z * (R(2) * z * z - R(3) * x * x - R(3) * y * y);
  dY[12][0] = k12 * R(-6) * x * z; dY[12][1] = k12 * R(-6) * y * z;
  dY[12][2] = k12 * (R(6) * z * z - R(3) * x * x - R(3) * y * y);
  // m = 1: x(4z^2 - x^2 - y^2)
  Y[13] = k11 * x * (R(4) * z * z - x * x - y * y);
  dY[13][0] = k11 * (R(4) * z * z - R(3) * x * x - y * y);
  dY[13][1] = k11 * R(-2) * x * y;
  dY[13][2] = k11 * R(8) * x * z;
  // m = 2: z(x^2 - y^2)
  Y[14] = k14 * z * (x * x - y * y);
  dY[14][0] = k14 * R(2) * x * z; dY[14][1] = k14 * R(-2) * y * z; dY[14][2] = k14 * (x * x - y * y);
  // m = 3: x(x^2 - 3y^2)
  Y[15] = k9 * x * (x * x - R(3) * y * y);
  dY[15][0] = k9 * (R(3) * x * x - R(3) * y * y); dY[15][1] = k9 * R(-6) * x * y;
}

inline int num_planes(int deg) { return 11 + 3 * (deg + 1) * (deg + 1); }

// SH degree ramp ([GSG] "Spherical harmonics": only the first activeK = (activeDeg + 1)^2 - 1
// band weights are summed, and the inactive ones receive no gradient until their band
// switches on).  -1: every stored band.  Set by or_set_active_sh_degree.
int g_active_deg = -1;
// Mip-Splatting opacity compensation ([GSG] "Flattening a 3D blob into a 2D oval": a
// correction from Mip-Splatting so that the dilation does not make very small Gaussians
// brighter overall; the code there multiplies the opacity by comp in the extent and in
// alpha).  Off (0) by default; set by
// or_set_mip_compensation.  The factor is not printed on the pages; the reading taken is
// the one that removes exactly the energy the 0.3 px^2 dilation adds: the footprint
// o exp(-d^T V^-1 d / 2) integrates to o 2 pi sqrt(det V), so the dilated footprint keeps
// that integral with comp = sqrt(det V / det(V + 0.3 I)) (0 when det V <= 0).
int g_mip = 0;

inline int active_bands(int deg) {
  const int d = (g_active_deg < 0 || g_active_deg > deg) ? deg : g_active_deg;
  return (d + 1) * (d + 1) - 1;
}

// --------------------------------------------------------------- preprocess
// Everything the forward projection computes for one Gaussian, kept so the
// backward chain can reuse it.  Sources:
//   [GST] parameter slide: log-scales -> exp, opacity logit -> sigmoid, normalised quaternion;
//   [DR]  "From a pixel error back to a quaternion": Sigma = R S S^T R^T;
//   [GST] Jacobian slide: J = [fx/Z, 0, -fx X/Z^2; 0, fy/Z, -fy Y/Z^2], +0.3 px^2 dilation;
//   [DR]  "Forward": Sigma' = J W Sigma W^T J^T;
//   [GSG] "Flattening a 3D blob into a 2D oval": rows of T = J W, V = T Sigma T^T, conic;
//   [GSG] "Why tiling": extent and tile rectangle;
//   [GSG] "Spherical harmonics": view-dependent colour, clamped at zero.
template <class R>
struct Fwd {
  bool visible = false;
  R m[3], p[3];          // world and camera-space centre
  R xz, yz, u, v;        // normalised image coordinates and pixel position
  R s[3];                // scales
  R ql, q[4];            // |q| and normalised quaternion (w, x, y, z)
  R Rq[3][3];            // rotation from the quaternion
  R M[3][3];             // Rq * diag(s)
  R Sig[3][3];           // 3D covariance
  R J00, J02, J11, J12;  // projection Jacobian entries
  R t0[3], t1[3];        // rows of T = J W
  R a, b, c, det;        // dilated screen covariance [[a, b], [b, c]] and its determinant
  R A, B, C;             // conic
  R o;                   // opacity of the record (ob comp with the Mip compensation, else ob)
  R ob, comp;            // sigmoid of the logit; the compensation factor (1 when off)
  R va, vb, vc, detv;    // undilated screen covariance and its determinant
  R dvec[3], dlen, dir[3];
  R Y[16], dY[16][3];
  R raw[3], rgb[3];      // colour before / after the clamp at zero
  R lmax, emax, rad;
  int rect[4];           // tile rectangle x0, y0, x1, y1 (inclusive)
  uint32_t tiles = 0;
};

template <class R>
R cam_R(const Camera& c, int i, int j) { return R(c.R[3 * i + j]); }

// Returns the projected record of Gaussian i.  smooth = true drops the
// thresholds (near plane reduced to z > 0, no colour clamp, no tile rectangle),
// the smooth function of [GST] opacity slide, used only for finite differences.
template <class R>
Fwd<R> project(const R* params, int64_t n, int64_t i, int deg, const Camera& cam, bool smooth) {
  Fwd<R> f;
  auto P = [&](int plane) { return params[int64_t(plane) * n + i]; };
  for (int k = 0; k < 3; ++k) f.m[k] = P(k);
  // camera-space centre p = W m + t
  for (int r = 0; r < 3; ++r)
    f.p[r] = ((cam_R<R>(cam, r, 0) * f.m[0] + cam_R<R>(cam, r, 1) * f.m[1]) + cam_R<R>(cam, r, 2) * f.m[2]) +
             R(cam.t[r]);
  const R znear = smooth ? R(0) : R(cam.znear);
  if (!(f.p[2] > znear)) return f;
  const R fx = R(cam.fx), fy = R(cam.fy);
  f.xz = f.p[0] / f.p[2];
  f.yz = f.p[1] / f.p[2];
  f.u = fx * f.xz + R(cam.cx);
  f.v = fy * f.yz + R(cam.cy);
  // scales and rotation
  for (int k = 0; k < 3; ++k) f.s[k] = exp_r(P(3 + k));
  R qr[4];
  for (int k = 0; k < 4; ++k) qr[k] = P(6 + k);
  R n2 = ((qr[0] * qr[0] + qr[1] * qr[1]) + qr[2] * qr[2]) + qr[3] * qr[3];
  if (!(n2 > R(0))) return f;
  f.ql = std::sqrt(n2);
  for (int k = 0; k < 4; ++k) f.q[k] = qr[k] / f.ql;
  const R w = f.q[0], x = f.q[1], y = f.q[2], z = f.q[3];
  f.Rq[0][0] = R(1) - R(2) * (y * y + z * z);
  f.Rq[0][1] = R(2) * (x * y - w * z);
  f.Rq[0][2] = R(2) * (x * z + w * y);
  f.Rq[1][0] = R(2) * (x * y + w * z);
  f.Rq[1][1] = R(1) - R(2) * (x * x + z * z);
  f.Rq[1][2] = R(2) * (y * z - w * x);
  f.Rq[2][0] = R(2) * (x * z - w * y);
  f.Rq[2][1] = R(2) * (y * z + w * x);
  f.Rq[2][2] = R(1) - R(2) * (x * x + y * y);
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) f.M[r][k] = f.Rq[r][k] * f.s[k];
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k)
      f.Sig[r][k] = (f.M[r][0] * f.M[k][0] + f.M[r][1] * f.M[k][1]) + f.M[r][2] * f.M[k][2];
  // Jacobian and T = J W
  f.J00 = fx / f.p[2];
  f.J02 = -(fx * f.xz) / f.p[2];
  f.J11 = fy / f.p[2];
  f.J12 = -(fy * f.yz) / f.p[2];
  for (int k = 0; k < 3; ++k) {
    f.t0[k] = f.J00 * cam_R<R>(cam, 0, k) + f.J02 * cam_R<R>(cam, 2, k);
    f.t1[k] = f.J11 * cam_R<R>(cam, 1, k) + f.J12 * cam_R<R>(cam, 2, k);
  }
  R w0[3], w1[3];  // Sigma t0, Sigma t1
  for (int r = 0; r < 3; ++r) {
    w0[r] = (f.Sig[r][0] * f.t0[0] + f.Sig[r][1] * f.t0[1]) + f.Sig[r][2] * f.t0[2];
    w1[r] = (f.Sig[r][0] * f.t1[0] + f.Sig[r][1] * f.t1[1]) + f.Sig[r][2] * f.t1[2];
  }
  const R V00 = (f.t0[0] * w0[0] + f.t0[1] * w0[1]) + f.t0[2] * w0[2];
  const R V01 = (f.t1[0] * w0[0] + f.t1[1] * w0[1]) + f.t1[2] * w0[2];
  const R V11 = (f.t1[0] * w1[0] + f.t1[1] * w1[1]) + f.t1[2] * w1[2];
  f.a = V00 + R(kDilation);
  f.b = V01;
  f.c = V11 + R(kDilation);
  f.det = f.a * f.c - f.b * f.b;
  if (!(f.det > R(0))) return f;
  f.A = f.c / f.det;
  f.B = -f.b / f.det;
  f.C = f.a / f.det;
  f.ob = sigmoid_r(P(10));
  f.va = V00;
  f.vb = V01;
  f.vc = V11;
  f.detv = V00 * V11 - V01 * V01;
  f.comp = R(1);
  f.o = f.ob;
  if (g_mip) {
    f.comp = std::sqrt(std::max(f.detv, R(0)) / f.det);
    f.o = f.ob * f.comp;
  }
  // colour: DC plus the (active) higher bands along dir = normalize(m - campos)
  const int K = active_bands(deg);
  for (int k = 0; k < 3; ++k) f.dvec[k] = f.m[k] - R(cam.campos[k]);
  f.dlen = std::sqrt((f.dvec[0] * f.dvec[0] + f.dvec[1] * f.dvec[1]) + f.dvec[2] * f.dvec[2]);
  for (int k = 0; k < 3; ++k) f.dir[k] = f.dvec[k] / f.dlen;
  sh_basis<R>(f.dir, f.Y, f.dY);
  for (int ch = 0; ch < 3; ++ch) {
    R col = P(11 + ch);
    for (int k = 1; k <= K; ++k) col = col + P(14 + 3 * (k - 1) + ch) * f.Y[k];
    f.raw[ch] = col;
    f.rgb[ch] = smooth ? col : std::max(col, R(0));
  }
  bool finite = std::isfinite(f.u) && std::isfinite(f.v) && std::isfinite(f.A) && std::isfinite(f.B) &&
                std::isfinite(f.C) && std::isfinite(f.o);
  for (int ch = 0; ch < 3; ++ch) finite = finite && std::isfinite(f.rgb[ch]);
  if (!finite) return f;
  if (smooth) { f.visible = true; return f; }
  // screen extent: eigenvalue of the dilated covariance and the opacity-aware falloff cut
  const R mid = R(0.5) * (f.a + f.c);
  const R disc = std::sqrt(std::max(mid * mid - f.det, R(0)));
  f.lmax = mid + disc;
  f.emax = R(std::min(kExtentCut, std::log(std::max(double(f.o) * kAlphaMinInv, kExtentLogFloor))));
  f.rad = std::sqrt(R(2) * f.emax) * std::sqrt(f.lmax);
  if (!std::isfinite(f.rad)) return f;
  // tile rectangle: every tile whose square meets [centre - rad, centre + rad]
  const R fx0 = std::floor((f.u - f.rad) / R(kTile)), fx1 = std::floor((f.u + f.rad) / R(kTile));
  const R fy0 = std::floor((f.v - f.rad) / R(kTile)), fy1 = std::floor((f.v + f.rad) / R(kTile));
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  if (fx1 < R(0) || fx0 > R(tx - 1) || fy1 < R(0) || fy0 > R(ty - 1)) return f;
  f.rect[0] = int(std::max(fx0, R(0)));
  f.rect[1] = int(std::max(fy0, R(0)));
  f.rect[2] = int(std::min(fx1, R(tx - 1)));
  f.rect[3] = int(std::min(fy1, R(ty - 1)));
  f.tiles = uint32_t(f.rect[2] - f.rect[0] + 1) * uint32_t(f.rect[3] - f.rect[1] + 1);
  f.visible = true;
  return f;
}

// -------------------------------------------------------------- blending
struct PixelTrace {        // per-pixel bookkeeping of the forward decisions
  uint32_t n_contrib;      // 1 + local index of the last blended entry (0 if none)
  uint32_t n_examined;     // entries examined, including the one that stopped the walk
  double margin;           // smallest conditioned distance of a skip/stop decision to its threshold
};

// Decision margins.  A 32-bit evaluation of alpha = o exp(-e), e the conic's
// quadratic form at (dx, dy), carries a relative error of a few units of
// rounding times 1 + S, with S the sum of the magnitudes of the form's terms:
// S exceeds e wherever the cross term cancels the squares (thin, tilted
// footprints far from their centre), and then the rounding of each term is
// amplified by S / e.  The transmittance after a run of blends inherits, per
// blended entry, that error times alpha / (1 - alpha) plus one rounding.  A
// decision's margin is its relative distance to the threshold divided by this
// scale, so that a margin of m means the decision survives any evaluation whose
// per-unit error is below m (about 1e-6 covers two differently ordered fp32
// evaluations with one-ulp exp).
inline double exponent_scale(double A, double B, double C, double dx, double dy) {
  return 1.0 + 0.5 * (std::fabs(A) * dx * dx + std::fabs(C) * dy * dy) + std::fabs(B * dx * dy);
}

// One thresholded decision of a pixel's walk: entry k of the walked list, and
// which test (alpha below 1/255, transmittance below the stop value after the
// entry, alpha above the cap).  Used to log the decisions close to their
// threshold and to take one of them the other way.
enum DecisionKind : int { kDecSkip = 0, kDecStop = 1, kDecCap = 2 };
struct Decision {
  int64_t k;
  int kind;
};

// FNV-1a step over the eight bytes of v: folds a pixel's decision outcomes into one
// signature, so that two renders can be compared decision for decision.
inline uint64_t sig_mix(uint64_t h, uint64_t v) {
  for (int b = 0; b < 8; ++b) {
    h ^= (v >> (8 * b)) & 0xffu;
    h *= 0x100000001b3ull;
  }
  return h;
}
constexpr uint64_t kSigSeed = 0xcbf29ce484222325ull;

// Front-to-back compositing of one pixel over an ordered list, [GSG] "The
// painting itself: front-to-back alpha compositing"; weights as in [GST]
// opacity slide and [TBDR] worked examples.  In smooth mode nothing is capped,
// skipped or stopped.
//
// flip (optional) takes one decision the other way; close (optional) receives
// every decision whose margin is below close_below (the cap decision included,
// which changes no forward value but the backward's dependence on the entry).
template <class R>
void blend_pixel(R px, R py, const uint32_t* list, int64_t len, const R* uv, const R* conic, const R* opac,
                 const R* rgb, int64_t n, const R bg[3], bool smooth, R out[3], R* T_out, PixelTrace* tr,
                 int64_t* evals, const Decision* flip = nullptr, std::vector<Decision>* close = nullptr,
                 double close_below = 0.0, uint64_t* sig = nullptr) {
  R T = R(1);
  R C[3] = {R(0), R(0), R(0)};
  PixelTrace t{0, 0, std::numeric_limits<double>::infinity()};
  double tscale = 1.0;     // conditioning of T (see exponent_scale)
  for (int64_t k = 0; k < len; ++k) {
    const uint32_t g = list[k];
    t.n_examined = uint32_t(k + 1);
    if (evals) ++*evals;
    const R dx = px - uv[g], dy = py - uv[n + g];
    const R A = conic[g], B = conic[n + g], Cc = conic[2 * n + g];
    const R e = R(0.5) * (A * dx * dx + Cc * dy * dy) + B * dx * dy;
    const R G = exp_r(-e);
    const R araw = opac[g] * G;
    R alpha = araw;
    if (!smooth) {
      const bool capped = araw >= R(kAlphaCap);
      alpha = std::min(R(kAlphaCap), araw);
      const double ascale = exponent_scale(double(A), double(B), double(Cc), double(dx), double(dy));
      const double mskip = std::fabs(double(alpha) - double(alpha_min<R>())) / double(alpha_min<R>()) / ascale;
      t.margin = std::min(t.margin, mskip);
      if (close) {
        if (mskip < close_below) close->push_back({k, kDecSkip});
        if (std::fabs(double(araw) - kAlphaCap) / kAlphaCap / ascale < close_below) close->push_back({k, kDecCap});
      }
      bool skip = alpha < alpha_min<R>();
      if (flip && flip->k == k && flip->kind == kDecSkip) skip = !skip;
      // the outcome of each decision: entry k skipped, or blended with alpha capped (the
      // backward's test, o G > 0.99, which decides whether the entry passes gradient on)
      if (sig) *sig = sig_mix(sig_mix(*sig, uint64_t(k)), skip ? 1u : (araw > R(kAlphaCap) ? 2u : 3u));
      if (skip) continue;
      // a capped alpha is exact; closeness to the cap is the backward's concern
      tscale += 1.0 + (capped ? 0.0 : ascale * double(alpha) / (1.0 - double(alpha)));
    }
    for (int ch = 0; ch < 3; ++ch) C[ch] = C[ch] + T * alpha * rgb[ch * n + g];
    T = T * (R(1) - alpha);
    t.n_contrib = uint32_t(k + 1);
    if (!smooth) {
      const double mstop = std::fabs(double(T) - kTStop) / kTStop / tscale;
      t.margin = std::min(t.margin, mstop);
      if (close && mstop < close_below) close->push_back({k, kDecStop});
      bool stop = T < R(kTStop);
      if (flip && flip->k == k && flip->kind == kDecStop) stop = !stop;
      if (stop) break;
    }
  }
  for (int ch = 0; ch < 3; ++ch) out[ch] = C[ch] + T * bg[ch];
  *T_out = T;
  if (tr) *tr = t;
  if (sig) *sig = sig_mix(*sig, uint64_t(t.n_contrib) | (uint64_t(t.n_examined) << 32));
}

// Back-to-front walk of one pixel, recovering the transmittance by division
// ([DR] "The trick: recompute the blend state instead of storing it"; [GSG]
// "The clever bit: a single backward sweep through the blend"), with the
// per-entry derivatives of [GST] compositing slide (dI/dalpha_i = T_i (c_i - C_tail),
// dI/dc_i = T_i alpha_i) and of [GSG] "From a pixel's blame to the oval's shape and place".
// gscreen planes: 0 u, 1 v, 2 A, 3 B, 4 C, 5 opacity, 6-8 colour.
// flip (optional) takes one skip or cap decision the other way, as the forward
// walk that produced T_final and n_walk did.
//
// mass (optional, [2][9][n] doubles, and count [n]) records how large the terms are
// that each partial sums, so that a reordered or differently rounded evaluation can be
// bounded: mass[0] adds |term| and mass[1] adds |term| (2 n_walk + 16) (the terms'
// own rounding grows with the walk that recovers T and S), count the pixels that
// contribute.  Terms are counted by the magnitudes of their factors (the colour
// difference inside dL/dalpha and the conic products inside du, dv unexpanded), so
// that cancellation inside one pixel's term is covered too.
template <class R>
void blend_pixel_bwd(R px, R py, const uint32_t* list, int64_t n_walk, const R* uv, const R* conic,
                     const R* opac, const R* rgb, int64_t n, const R bg[3], bool smooth, R T_final,
                     const R gI[3], R* gscreen, const Decision* flip = nullptr, double* mass = nullptr,
                     uint32_t* count = nullptr) {
  const double wdepth = 2.0 * double(n_walk) + 16.0;
  auto add_mass = [&](int plane, uint32_t g, double m) {
    mass[int64_t(plane) * n + g] += m;
    mass[int64_t(9 + plane) * n + g] += m * wdepth;
  };
  R T = T_final;
  R S[3];
  for (int ch = 0; ch < 3; ++ch) S[ch] = bg[ch] * T_final;
  for (int64_t k = n_walk - 1; k >= 0; --k) {
    const uint32_t g = list[k];
    const R dx = px - uv[g], dy = py - uv[n + g];
    const R A = conic[g], B = conic[n + g], Cc = conic[2 * n + g];
    const R e = R(0.5) * (A * dx * dx + Cc * dy * dy) + B * dx * dy;
    const R G = exp_r(-e);
    const R araw = opac[g] * G;
    R alpha = araw;
    bool capped = false;
    if (!smooth) {
      capped = araw > R(kAlphaCap);
      alpha = std::min(R(kAlphaCap), araw);
      bool skip = alpha < alpha_min<R>();
      if (flip && flip->k == k && flip->kind == kDecSkip) skip = !skip;
      if (flip && flip->k == k && flip->kind == kDecCap) capped = !capped;
      if (skip) continue;
    }
    T = T / (R(1) - alpha);              // transmittance in front of this entry
    const R wgt = alpha * T;
    R galpha = R(0);
    double gam = 0.0;                    // magnitude of the terms of dL/dalpha
    for (int ch = 0; ch < 3; ++ch) {
      gscreen[(6 + ch) * n + g] += gI[ch] * wgt;
      galpha += gI[ch] * (rgb[ch * n + g] * T - S[ch] / (R(1) - alpha));
      if (mass) {
        gam += std::fabs(double(gI[ch])) * (std::fabs(double(rgb[ch * n + g])) * double(T) +
                                             std::fabs(double(S[ch])) / (1.0 - double(alpha)));
        add_mass(6 + ch, g, std::fabs(double(gI[ch]) * double(wgt)));
      }
      S[ch] += rgb[ch * n + g] * wgt;
    }
    if (count) ++count[g];
    if (capped) continue;                // alpha = 0.99 does not depend on opacity or position
    gscreen[5 * n + g] += galpha * G;    // d alpha / d opacity = G
    const R ge = -galpha * araw;         // d alpha / d e = -alpha
    gscreen[2 * n + g] += ge * R(0.5) * dx * dx;
    gscreen[3 * n + g] += ge * dx * dy;
    gscreen[4 * n + g] += ge * R(0.5) * dy * dy;
    gscreen[0 * n + g] += -ge * (A * dx + B * dy);   // d e / d u = -(A dx + B dy)
    gscreen[1 * n + g] += -ge * (B * dx + Cc * dy);
    if (mass) {
      const double me = gam * double(araw), ax = std::fabs(double(dx)), ay = std::fabs(double(dy));
      add_mass(5, g, gam * double(G));
      add_mass(2, g, me * 0.5 * ax * ax);
      add_mass(3, g, me * ax * ay);
      add_mass(4, g, me * 0.5 * ay * ay);
      add_mass(0, g, me * (std::fabs(double(A)) * ax + std::fabs(double(B)) * ay));
      add_mass(1, g, me * (std::fabs(double(B)) * ax + std::fabs(double(Cc)) * ay));
    }
  }
}

// [GSG] "Forgiving the camera and the light": the render depends on the camera pose, so
// backpropagation yields its gradient.  Pose W, t (p = W m + t; the camera centre is
// -W^T t), rotation perturbed on the left, W <- (I + [w]x) W.  One Gaussian's terms of
// dL/dW: the covariance path J^T dT (T = J W), the position path dp m^T, and the view
// direction's path through the centre, t gm_sh^T (dL/dcentre = -gm_sh); of dL/dt: dp and
// W gm_sh.  With G = dL/dW and M = G W^T the rotation gradient is (M21 - M12, M02 - M20,
// M10 - M01); for the position path alone that is (p - t) x dp, the pages' torque, and
// the translation's is dp alone: the trainer's code accumulates exactly those two
// (position_only), the exact derivative adds the other paths.
// out[0..2] += rotation gradient, out[3..5] += translation gradient.
template <class R>
void camera_grad_terms(const Fwd<R>& f, const Camera& cam, const R dT[2][3], const R dp[3], const R gm_sh[3],
                       bool position_only, double* out) {
  const double fx = cam.fx, fy = cam.fy, pz = f.p[2];
  const double J[2][3] = {{fx / pz, 0.0, -fx * double(f.p[0]) / (pz * pz)},
                          {0.0, fy / pz, -fy * double(f.p[1]) / (pz * pz)}};
  double W[3][3], G[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) W[r][c] = cam.R[3 * r + c];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c)
      G[r][c] = position_only ? double(dp[r]) * double(f.m[c])
                              : J[0][r] * double(dT[0][c]) + J[1][r] * double(dT[1][c]) +
                                    double(dp[r]) * double(f.m[c]) + double(cam.t[r]) * double(gm_sh[c]);
  double M[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) M[r][c] = G[r][0] * W[c][0] + G[r][1] * W[c][1] + G[r][2] * W[c][2];
  out[0] += M[2][1] - M[1][2];
  out[1] += M[0][2] - M[2][0];
  out[2] += M[1][0] - M[0][1];
  for (int r = 0; r < 3; ++r)
    out[3 + r] += position_only ? double(dp[r])
                                : double(dp[r]) + W[r][0] * double(gm_sh[0]) + W[r][1] * double(gm_sh[1]) +
                                      W[r][2] * double(gm_sh[2]);
}

// --------------------------------------------------------- backward chain
// Per Gaussian: screen gradients -> parameter gradients.  Sources:
//   [GSG] "From a pixel's blame to the oval's shape and place": opacity logit factor;
//   [GSG] "The covariance chain": conic -> V (dV = -K G K), V -> Sigma (T^T H T, dT = 2 H T Sigma),
//         Sigma -> M (dM = 2 dSigma M), scale and quaternion, projection off |q|;
//   [GSG] "Where the position gradient comes from" and [GST] Jacobian slide: both position paths;
//   [GSG] "Spherical harmonics": dL/dsh_k = dRGB Y_k and the view-direction term.
// With camg, the Gaussian's part of the camera-pose gradient is added to it (double[6]):
// see camera_grad_terms.
template <class R>
void chain_one(const R* params, int64_t n, int64_t i, int deg, const Camera& cam, bool smooth,
               const R* gscreen, R* gparams, double* camg = nullptr, bool cam_position_only = false) {
  const int P = num_planes(deg);
  for (int pl = 0; pl < P; ++pl) gparams[int64_t(pl) * n + i] = R(0);
  Fwd<R> f = project<R>(params, n, i, deg, cam, smooth);
  if (!f.visible) return;
  auto GS = [&](int k) { return gscreen[int64_t(k) * n + i]; };
  auto GP = [&](int plane) -> R& { return gparams[int64_t(plane) * n + i]; };
  const R gu = GS(0), gv = GS(1), gA = GS(2), gB = GS(3), gC = GS(4), go = GS(5);
  // opacity logit (through the compensation factor when it is on)
  GP(10) = g_mip ? go * f.comp * f.ob * (R(1) - f.ob) : go * f.o * (R(1) - f.o);
  // colour -> DC, the active higher bands (the others get none), view direction
  const int K = active_bands(deg);
  R gc[3];
  for (int ch = 0; ch < 3; ++ch) gc[ch] = (!smooth && f.raw[ch] < R(0)) ? R(0) : GS(6 + ch);
  R gdir[3] = {R(0), R(0), R(0)};
  for (int ch = 0; ch < 3; ++ch) {
    GP(11 + ch) = gc[ch];
    for (int k = 1; k <= K; ++k) {
      GP(14 + 3 * (k - 1) + ch) = gc[ch] * f.Y[k];
      const R coef = params[int64_t(14 + 3 * (k - 1) + ch) * n + i];
      for (int a = 0; a < 3; ++a) gdir[a] += gc[ch] * coef * f.dY[k][a];
    }
  }
  R gm[3] = {R(0), R(0), R(0)};
  if (K > 0) {
    const R dd = f.dir[0] * gdir[0] + f.dir[1] * gdir[1] + f.dir[2] * gdir[2];
    for (int a = 0; a < 3; ++a) gm[a] += (gdir[a] - f.dir[a] * dd) / f.dlen;
  }
  const R gm_sh[3] = {gm[0], gm[1], gm[2]};   // the view-direction part (dL/dcampos = -gm_sh)
  // conic -> dilated covariance: dL/dV' = -K G K, with G the symmetric conic gradient
  const R Km[2][2] = {{f.A, f.B}, {f.B, f.C}};
  const R Gm[2][2] = {{gA, R(0.5) * gB}, {R(0.5) * gB, gC}};
  R KG[2][2], KGK[2][2];
  for (int r = 0; r < 2; ++r)
    for (int c = 0; c < 2; ++c) KG[r][c] = Km[r][0] * Gm[0][c] + Km[r][1] * Gm[1][c];
  for (int r = 0; r < 2; ++r)
    for (int c = 0; c < 2; ++c) KGK[r][c] = KG[r][0] * Km[0][c] + KG[r][1] * Km[1][c];
  R gV00 = -KGK[0][0], gV01 = -(KGK[0][1] + KGK[1][0]), gV11 = -KGK[1][1];
  // the compensation factor comp = sqrt(det V / det V') with V' = V + 0.3 I:
  //   d comp = comp / 2 (d det V / det V - d det V' / det V'),
  //   d det V = (vc, -2 vb, va) . (d va, d vb, d vc), and the same for V' with (c, b, a)
  if (g_mip && f.detv > R(0)) {
    const R gcomp = go * f.ob;
    const R h = R(0.5) * f.comp;
    gV00 += gcomp * h * (f.vc / f.detv - f.c / f.det);
    gV11 += gcomp * h * (f.va / f.detv - f.a / f.det);
    gV01 += gcomp * h * (R(2) * f.b / f.det - R(2) * f.vb / f.detv);
  }
  // V = T Sigma T^T:  dSigma = T^T H T,  dT = 2 H T Sigma
  const R H[2][2] = {{gV00, R(0.5) * gV01}, {R(0.5) * gV01, gV11}};
  const R* Tr[2] = {f.t0, f.t1};
  R dSig[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) {
      R acc = R(0);
      for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b) acc += Tr[a][r] * H[a][b] * Tr[b][c];
      dSig[r][c] = acc;
    }
  R dT[2][3];
  for (int a = 0; a < 2; ++a)
    for (int c = 0; c < 3; ++c) {
      R acc = R(0);
      for (int b = 0; b < 2; ++b)
        for (int k = 0; k < 3; ++k) acc += H[a][b] * Tr[b][k] * f.Sig[k][c];
      dT[a][c] = R(2) * acc;
    }
  // T = J W  ->  dJ = dT W^T (only the four non-constant entries of J matter)
  R dJ[2][3];
  for (int a = 0; a < 2; ++a)
    for (int r = 0; r < 3; ++r) {
      R acc = R(0);
      for (int c = 0; c < 3; ++c) acc += dT[a][c] * cam_R<R>(cam, r, c);
      dJ[a][r] = acc;
    }
  const R fx = R(cam.fx), fy = R(cam.fy);
  const R pz = f.p[2], pz2 = pz * pz, pz3 = pz2 * pz;
  R dp[3] = {R(0), R(0), R(0)};
  // covariance path through J(p)
  dp[0] += dJ[0][2] * (-fx / pz2);
  dp[1] += dJ[1][2] * (-fy / pz2);
  dp[2] += dJ[0][0] * (-fx / pz2) + dJ[0][2] * (R(2) * fx * f.p[0] / pz3) + dJ[1][1] * (-fy / pz2) +
           dJ[1][2] * (R(2) * fy * f.p[1] / pz3);
  // projected-mean path: u = fx px/pz + cx, v = fy py/pz + cy
  dp[0] += gu * fx / pz;
  dp[1] += gv * fy / pz;
  dp[2] += -gu * fx * f.p[0] / pz2 - gv * fy * f.p[1] / pz2;
  // p = W m + t  ->  dm = W^T dp
  for (int c = 0; c < 3; ++c)
    for (int r = 0; r < 3; ++r) gm[c] += cam_R<R>(cam, r, c) * dp[r];
  for (int c = 0; c < 3; ++c) GP(c) = gm[c];
  if (camg) camera_grad_terms<R>(f, cam, dT, dp, gm_sh, cam_position_only, camg);
  // Sigma = M M^T -> dM = 2 dSigma M
  R dM[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c)
      dM[r][c] = R(2) * (dSig[r][0] * f.M[0][c] + dSig[r][1] * f.M[1][c] + dSig[r][2] * f.M[2][c]);
  // M = Rq diag(s): ds_j = sum_i dM_ij Rq_ij, log-scale gradient = ds * s
  for (int j = 0; j < 3; ++j) {
    const R ds = dM[0][j] * f.Rq[0][j] + dM[1][j] * f.Rq[1][j] + dM[2][j] * f.Rq[2][j];
    GP(3 + j) = ds * f.s[j];
  }
  // dRq = dM diag(s); derivative of the unit-quaternion rotation matrix, then off the norm
  R dR[3][3];
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c) dR[r][c] = dM[r][c] * f.s[c];
  const R w = f.q[0], x = f.q[1], y = f.q[2], z = f.q[3];
  R gq[4];
  gq[0] = R(2) * (-z * dR[0][1] + y * dR[0][2] + z * dR[1][0] - x * dR[1][2] - y * dR[2][0] + x * dR[2][1]);
  gq[1] = R(2) * (y * dR[0][1] + z * dR[0][2] + y * dR[1][0] - R(2) * x * dR[1][1] - w * dR[1][2] +
                  z * dR[2][0] + w * dR[2][1] - R(2) * x * dR[2][2]);
  gq[2] = R(2) * (-R(2) * y * dR[0][0] + x * dR[0][1] + w * dR[0][2] + x * dR[1][0] + z * dR[1][2] -
                  w * dR[2][0] + z * dR[2][1] - R(2) * y * dR[2][2]);
  gq[3] = R(2) * (-R(2) * z * dR[0][0] - w * dR[0][1] + x * dR[0][2] + w * dR[1][0] - R(2) * z * dR[1][1] +
                  y * dR[1][2] + x * dR[2][0] + y * dR[2][1]);
  const R qd = (w * gq[0] + x * gq[1]) + (y * gq[2] + z * gq[3]);
  for (int k = 0; k < 4; ++k) GP(6 + k) = (gq[k] - f.q[k] * qd) / f.ql;
}

// ------------------------------------------------------------------- loss
// 0.8 L1 + 0.2 (1 - SSIM): [GST] loss slides ("(1-lambda) L1 + lambda (1-SSIM)", no
// one-half, lambda = 0.2; L1 over 3HW with zero subgradient at zero residual; 11x11
// Gaussian window of standard deviation 1.5, C1 = 0.01^2, C2 = 0.03^2, zero padding,
// SSIM averaged over windows and channels); [LAB] combined objective.
// Written as the direct 2-D windowed sums (no separable pass) and their adjoint.
// mag (optional, [3][H][W]): per element, the sum of the magnitudes of the SSIM terms its
// gradient adds up (each window's three derivative terms, factor by factor), the scale of
// what a reordered or differently rounded evaluation of that gradient can change.
template <class R>
void loss_l1_dssim(const R* img, const R* tgt, int H, int W, R lambda, R out[3], R* grad, double* mag = nullptr) {
  const int rad = 5;
  const double sigma = 1.5;
  double wsum = 0.0;
  double w2[11][11];
  for (int i = -rad; i <= rad; ++i)
    for (int j = -rad; j <= rad; ++j) {
      w2[i + rad][j + rad] = std::exp(-double(i * i + j * j) / (2.0 * sigma * sigma));
      wsum += w2[i + rad][j + rad];
    }
  R w[11][11];
  for (int i = 0; i < 11; ++i)
    for (int j = 0; j < 11; ++j) w[i][j] = R(w2[i][j] / wsum);
  const R C1 = R(0.01 * 0.01), C2 = R(0.03 * 0.03);
  const int64_t HW = int64_t(H) * W, NE = 3 * HW;
  const R inv = R(1) / R(NE);
  R l1 = R(0), ssim_sum = R(0);
  std::vector<R> dmu(NE), dsx(NE), dsxy(NE), mux(NE), muy(NE);
  for (int ch = 0; ch < 3; ++ch) {
    const R* X = img + ch * HW;
    const R* Y = tgt + ch * HW;
    for (int yy = 0; yy < H; ++yy)
      for (int xx = 0; xx < W; ++xx) {
        R mx = 0, my = 0, exx = 0, eyy = 0, exy = 0;
        for (int i = -rad; i <= rad; ++i)
          for (int j = -rad; j <= rad; ++j) {
            const int y2 = yy + i, x2 = xx + j;
            if (y2 < 0 || y2 >= H || x2 < 0 || x2 >= W) continue;   // zero padding
            const R wt = w[i + rad][j + rad];
            const R xv = X[int64_t(y2) * W + x2], yv = Y[int64_t(y2) * W + x2];
            mx += wt * xv; my += wt * yv; exx += wt * xv * xv; eyy += wt * yv * yv; exy += wt * xv * yv;
          }
        const R sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
        const R A1 = R(2) * mx * my + C1, A2 = R(2) * sxy + C2;
        const R B1 = mx * mx + my * my + C1, B2 = sxx + syy + C2;
        const R S = (A1 * A2) / (B1 * B2);
        ssim_sum += S;
        const int64_t idx = ch * HW + int64_t(yy) * W + xx;
        // partials of S with respect to mu_x, sigma_x^2, sigma_xy (mu_y, sigma_y^2 held fixed)
        dmu[idx] = (R(2) * my * A2) / (B1 * B2) - (R(2) * mx * A1 * A2) / (B1 * B1 * B2);
        dsx[idx] = -(A1 * A2) / (B1 * B2 * B2);
        dsxy[idx] = (R(2) * A1) / (B1 * B2);
        mux[idx] = mx; muy[idx] = my;
        const R r = X[int64_t(yy) * W + xx] - Y[int64_t(yy) * W + xx];
        l1 += std::fabs(r);
      }
  }
  const R L1 = l1 * inv, SS = ssim_sum * inv;
  out[0] = (R(1) - lambda) * L1 + lambda * (R(1) - SS);
  out[1] = L1;
  out[2] = SS;
  if (!grad) return;
  for (int64_t k = 0; k < NE; ++k) {
    const R r = img[k] - tgt[k];
    grad[k] = (R(1) - lambda) * inv * (r > R(0) ? R(1) : (r < R(0) ? R(-1) : R(0)));
    if (mag) mag[k] = 0.0;
  }
  // adjoint of the windowed sums: pixel q receives from every window centre p within reach
  for (int ch = 0; ch < 3; ++ch) {
    const R* X = img + ch * HW;
    const R* Y = tgt + ch * HW;
    for (int yy = 0; yy < H; ++yy)
      for (int xx = 0; xx < W; ++xx) {
        const int64_t p = ch * HW + int64_t(yy) * W + xx;
        for (int i = -rad; i <= rad; ++i)
          for (int j = -rad; j <= rad; ++j) {
            const int y2 = yy + i, x2 = xx + j;
            if (y2 < 0 || y2 >= H || x2 < 0 || x2 >= W) continue;
            const R wt = w[i + rad][j + rad];
            const int64_t q = int64_t(y2) * W + x2;
            const R dS = dmu[p] * wt + dsx[p] * (R(2) * X[q] * wt - R(2) * mux[p] * wt) +
                         dsxy[p] * (Y[q] * wt - muy[p] * wt);
            grad[ch * HW + q] += -lambda * inv * dS;
            if (mag) {
              const double a = std::fabs(double(dmu[p])) + std::fabs(double(dsx[p])) * 2.0 *
                               (std::fabs(double(X[q])) + std::fabs(double(mux[p]))) +
                               std::fabs(double(dsxy[p])) * (std::fabs(double(Y[q])) + std::fabs(double(muy[p])));
              mag[ch * HW + q] += std::fabs(double(lambda) * double(inv)) * double(wt) * a;
            }
          }
      }
  }
}

// ------------------------------------------------------------------- Adam
// [GSG] Adam section: m, v running moments, bias correction, theta -= lr m^/(sqrt(v^) + eps);
// [DR] "From a pixel error back to a quaternion" and [GST] loop slide: per-group rates.
// Groups: planes 0-2 means, 3-5 log-scales, 6-9 quaternion, 10 opacity, 11.. colour.
template <class R>
void adam(R* params, const R* grads, R* m, R* v, int64_t n, int deg, const double lr[5], double b1, double b2,
          double eps, int step) {
  const int P = num_planes(deg);
  const double bc1 = 1.0 - std::pow(b1, step), bc2 = 1.0 - std::pow(b2, step);
  for (int pl = 0; pl < P; ++pl) {
    const int grp = pl < 3 ? 0 : pl < 6 ? 1 : pl < 10 ? 2 : pl == 10 ? 3 : 4;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t k = int64_t(pl) * n + i;
      const R g = grads[k];
      m[k] = R(b1) * m[k] + R(1.0 - b1) * g;
      v[k] = R(b2) * v[k] + R(1.0 - b2) * g * g;
      const R mh = m[k] / R(bc1), vh = v[k] / R(bc2);
      params[k] = params[k] - R(lr[grp]) * mh / (std::sqrt(vh) + R(eps));
    }
  }
}

// ------------------------------------------------------------ tile binning
// Count, scan, scatter and per-tile depth sort of [GSG] "Why tiling, and the five
// stages": every visible Gaussian, in ascending id, emits one (key, id) pair per
// covered tile in row-major tile order; key = tile << 32 | bits(depth), and a
// stable sort by key gives tile order, then depth, then id (the bitonic sort's
// tie-break in the same section).  ranges[t] = [first, last + 1) or (0, 0).
void bin_sort(int64_t n, const float* depth, const int32_t* rect, const uint32_t* tiles, int tx, int ty,
              uint64_t* keys, uint32_t* vals, uint32_t* ranges) {
  int64_t pos = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (tiles[i] == 0) continue;
    uint32_t dbits;
    std::memcpy(&dbits, &depth[i], 4);
    for (int y = rect[n + i]; y <= rect[3 * n + i]; ++y)
      for (int x = rect[i]; x <= rect[2 * n + i]; ++x) {
        keys[pos] = (uint64_t(uint32_t(y * tx + x)) << 32) | dbits;
        vals[pos] = uint32_t(i);
        ++pos;
      }
  }
  std::vector<int64_t> order(pos);
  for (int64_t k = 0; k < pos; ++k) order[k] = k;
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return keys[a] < keys[b]; });
  std::vector<uint64_t> k2(pos);
  std::vector<uint32_t> v2(pos);
  for (int64_t k = 0; k < pos; ++k) { k2[k] = keys[order[k]]; v2[k] = vals[order[k]]; }
  std::copy(k2.begin(), k2.end(), keys);
  std::copy(v2.begin(), v2.end(), vals);
  const int64_t nt = int64_t(tx) * ty;
  for (int64_t t = 0; t < 2 * nt; ++t) ranges[t] = 0;
  for (int64_t k = 0; k < pos; ++k) {
    const uint32_t t = uint32_t(keys[k] >> 32);
    if (k == 0 || uint32_t(keys[k - 1] >> 32) != t) ranges[t] = uint32_t(k);
    if (k == pos - 1 || uint32_t(keys[k + 1] >> 32) != t) ranges[nt + t] = uint32_t(k + 1);
  }
}

template <class R>
void smooth_order(int64_t n, const R* depth, const uint8_t* visible, std::vector<uint32_t>& list) {
  list.clear();
  for (int64_t i = 0; i < n; ++i)
    if (visible[i]) list.push_back(uint32_t(i));
  std::stable_sort(list.begin(), list.end(), [&](uint32_t a, uint32_t b) { return depth[a] < depth[b]; });
}

// Tiled forward render of all pixels.  Outputs planar rgb [3][H][W], T_final and
// n_contrib [H][W]; optional n_examined, margin and sig (the decision signature of
// blend_pixel) [H][W]; returns evals.
template <class R>
int64_t render_tiled(int64_t n, const R* uv, const R* conic, const R* opac, const R* rgb, const uint32_t* vals,
                     const uint32_t* ranges, const Camera* cam, R* out_rgb, R* T_final, uint32_t* n_contrib,
                     uint32_t* n_examined, double* margin, uint64_t* sig) {
  const int W = cam->width, H = cam->height, tx = tiles_x(*cam), ty = tiles_y(*cam);
  const int64_t nt = int64_t(tx) * ty, HW = int64_t(W) * H;
  const R bg[3] = {R(cam->bg[0]), R(cam->bg[1]), R(cam->bg[2])};
  int64_t evals = 0;
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      const int64_t t = int64_t(y / kTile) * tx + x / kTile;
      const uint32_t s = ranges[t], e = ranges[nt + t];
      const int64_t p = int64_t(y) * W + x;
      R out[3], T;
      PixelTrace tr;
      uint64_t h = kSigSeed;
      blend_pixel<R>(R(x) + R(0.5), R(y) + R(0.5), vals + s, int64_t(e) - s, uv, conic, opac, rgb, n, bg, false,
                     out, &T, &tr, &evals, nullptr, nullptr, 0.0, sig ? &h : nullptr);
      for (int ch = 0; ch < 3; ++ch) out_rgb[ch * HW + p] = out[ch];
      T_final[p] = T;
      n_contrib[p] = tr.n_contrib;
      if (n_examined) n_examined[p] = tr.n_examined;
      if (margin) margin[p] = tr.margin;
      if (sig) sig[p] = h;
    }
  return evals;
}

}  // namespace

// ===================================================================== C ABI
// Plain entry points for ctypes.  Arrays are planar ([plane][n] or [ch][H][W]).

// ------------------------------------------------ Charbonnier loss with exposure
// [GSG] the trainer's loss (the code after "The painting itself"): per element
// err = gain C + bias - target, root = sqrt(err^2 + delta^2), loss term root - delta, slope
// gain err / root; "Forgiving the camera and the light": one gain (stored as its log) and
// one bias per image, d/d(log gain) = sum (err / root) C gain, d/d bias = sum err / root.
// Reading: the loss is the mean over the 3HW elements (as the L1 term is).
template <class R>
void loss_charbonnier(const R* img, const R* tgt, int64_t count, R delta, R log_gain, R bias, R* out3, R* grad) {
  const R gain = R(std::exp(double(log_gain)));
  double sl = 0.0, sg = 0.0, sb = 0.0;
  const R inv = R(1.0 / double(count));
  for (int64_t i = 0; i < count; ++i) {
    const R err = gain * img[i] + bias - tgt[i];
    const R root = std::sqrt(err * err + delta * delta);
    const R eg = err / root;
    sl += double(root - delta);
    sg += double(eg * img[i] * gain);
    sb += double(eg);
    grad[i] = gain * eg * inv;
  }
  out3[0] = R(sl / double(count));
  out3[1] = R(sg / double(count));
  out3[2] = R(sb / double(count));
}

// ---------------------------------------------------------- density control
// [GST] density-control slide ("Original 3DGS periodically changes the number of
// primitives"): the screen-space centre gradient magnitude of every visible
// observation is accumulated and averaged over the observations; small Gaussians with a
// large average are cloned (an exact copy), large ones split into two children
// sampled around the parent with smaller scales, very transparent or oversized ones
// pruned; an opacity reset clamps opacity to at most a cap.  [GSG] "Densification":
// split halves shrink by 1.6 and a reshaped Gaussian starts with zero Adam moments.
// Thresholds the pages leave open are arguments; decisions are taken on the stored
// logit and log-scales against thresholds rounded once from double (reading R34).

// One step's observations: a Gaussian with tiles > 0 adds |(du, dv)| and 1.
void densify_accumulate(int64_t n, const uint32_t* tiles, const float* gscreen, float* stats) {
  for (int64_t i = 0; i < n; ++i) {
    if (tiles[i] == 0u) continue;
    const float du = gscreen[i], dv = gscreen[n + i];
    stats[2 * i] += std::sqrt(du * du + dv * dv);
    stats[2 * i + 1] += 1.0f;
  }
}

enum DensAct { kPrune = 0, kKeep = 1, kClone = 2, kSplit = 3 };

int densify_action(const float* params, int64_t n, int64_t i, const float* stats, float grad_thr, float logit_prune,
                   float lscale_prune, float lscale_split) {
  auto P = [&](int k) { return params[k * n + i]; };
  const float lsmax = std::max(std::max(P(3), P(4)), P(5));
  if (P(10) < logit_prune || lsmax > lscale_prune) return kPrune;
  const float cnt = stats[2 * i + 1];
  const float avg = cnt > 0.0f ? stats[2 * i] / cnt : 0.0f;
  if (!(avg >= grad_thr)) return kKeep;
  return lsmax > lscale_split ? kSplit : kClone;
}

// Mean of split child c of Gaussian i: mean + Rq (s * eps), eps = rand[i][c][0..2] standard
// normals drawn by the caller, Rq from the normalised quaternion (identity for a zero one).
void split_child_mean(const float* params, int64_t n, int64_t i, const float* eps, float* out) {
  auto P = [&](int k) { return params[k * n + i]; };
  float s[3];
  for (int k = 0; k < 3; ++k) s[k] = exp_r(P(3 + k));
  float Rq[3][3] = {{1.f, 0.f, 0.f}, {0.f, 1.f, 0.f}, {0.f, 0.f, 1.f}};
  const float n2 = ((P(6) * P(6) + P(7) * P(7)) + P(8) * P(8)) + P(9) * P(9);
  if (n2 > 0.0f) {
    const float ql = std::sqrt(n2);
    const float w = P(6) / ql, x = P(7) / ql, y = P(8) / ql, z = P(9) / ql;
    Rq[0][0] = 1.0f - 2.0f * (y * y + z * z);
    Rq[0][1] = 2.0f * (x * y - w * z);
    Rq[0][2] = 2.0f * (x * z + w * y);
    Rq[1][0] = 2.0f * (x * y + w * z);
    Rq[1][1] = 1.0f - 2.0f * (x * x + z * z);
    Rq[1][2] = 2.0f * (y * z - w * x);
    Rq[2][0] = 2.0f * (x * z - w * y);
    Rq[2][1] = 2.0f * (y * z + w * x);
    Rq[2][2] = 1.0f - 2.0f * (x * x + y * y);
  }
  const float d[3] = {s[0] * eps[0], s[1] * eps[1], s[2] * eps[2]};
  for (int r = 0; r < 3; ++r) out[r] = P(r) + ((Rq[r][0] * d[0] + Rq[r][1] * d[1]) + Rq[r][2] * d[2]);
}

// The new population, in the order: kept Gaussians, clones, first split children, second
// split children (each group in the order of its parents).  Returns its size; the
// outputs ([P][cap] planar; stats_out [cap][2], zeroed) are written only if it fits.
int64_t densify(int64_t n, int deg, const float* params, const float* m, const float* v, const float* stats,
                const float* rand, float grad_thr, float logit_prune, float lscale_prune, float lscale_split,
                float lscale_shrink, int reset, float logit_cap, int64_t cap, float* params_out, float* m_out,
                float* v_out, float* stats_out, int64_t* counts) {
  const int P = num_planes(deg);
  std::vector<int> act(static_cast<size_t>(n), 0);
  int64_t kept = 0, clones = 0, splits = 0;
  for (int64_t i = 0; i < n; ++i) {
    act[size_t(i)] = densify_action(params, n, i, stats, grad_thr, logit_prune, lscale_prune, lscale_split);
    kept += act[size_t(i)] == kKeep || act[size_t(i)] == kClone;
    clones += act[size_t(i)] == kClone;
    splits += act[size_t(i)] == kSplit;
  }
  counts[0] = kept;
  counts[1] = clones;
  counts[2] = splits;
  const int64_t total = kept + clones + 2 * splits;
  if (total > cap) return total;
  // writes Gaussian i as output d; fresh: zero moments; mean / lscale_delta: child changes
  auto put = [&](int64_t i, int64_t d, bool fresh, const float* mean, bool shrink) {
    for (int k = 0; k < P; ++k) {
      float th = params[k * n + i];
      if (mean && k < 3) th = mean[k];
      if (shrink && k >= 3 && k < 6) th = th - lscale_shrink;
      float mo = fresh ? 0.0f : m[k * n + i], vo = fresh ? 0.0f : v[k * n + i];
      if (reset && k == 10) {
        th = std::min(th, logit_cap);
        mo = vo = 0.0f;
      }
      params_out[k * cap + d] = th;
      m_out[k * cap + d] = mo;
      v_out[k * cap + d] = vo;
    }
    stats_out[2 * d] = stats_out[2 * d + 1] = 0.0f;
  };
  int64_t dk = 0, dc = kept, ds = kept + clones;
  for (int64_t i = 0; i < n; ++i) {
    const int a = act[size_t(i)];
    if (a == kKeep || a == kClone) put(i, dk++, false, nullptr, false);
    if (a == kClone) put(i, dc++, true, nullptr, false);
    if (a == kSplit) {
      for (int c = 0; c < 2; ++c) {
        float mean[3];
        split_child_mean(params, n, i, rand + (2 * i + c) * 3, mean);
        put(i, ds + c * splits, true, mean, true);
      }
      ++ds;
    }
  }
  return total;
}

// Relocation of the dead ([GSG] "Densification", the MCMC-style pass): a Gaussian whose
// opacity is below the dead threshold is dead, one above the donor threshold a donor
// (decisions on the stored logit against the thresholds' logit, rounded once to float;
// a donor's largest log-scale must not be NaN).  The donors are ranked by their largest
// log-scale, largest first, equal sizes in index order; the k-th dead Gaussian in index
// order moves to the k-th ranked donor, for k below the smaller count and max_moves.  A
// moved Gaussian takes the donor's parameters with its mean placed at mean + Rq (s eps)
// (eps: its own three caller-drawn normals, as a split child's) and the log-scales
// lowered by the shrink; the donor's log-scales are lowered too; both restart with zero
// moments.  Everything else is unchanged, and so is the count.  In place; returns the
// number of moves.
int64_t relocate(int64_t n, int deg, float* params, float* m, float* v, const float* rand, float logit_dead,
                 float logit_donor, float lscale_shrink, int64_t max_moves) {
  const int P = num_planes(deg);
  std::vector<int64_t> dead;
  std::vector<std::pair<float, int64_t>> donors;
  for (int64_t i = 0; i < n; ++i) {
    const float logit = params[10 * n + i];
    const float lsmax = std::max(std::max(params[3 * n + i], params[4 * n + i]), params[5 * n + i]);
    if (logit < logit_dead) dead.push_back(i);
    else if (logit > logit_donor && !std::isnan(lsmax)) donors.push_back({lsmax, i});
  }
  std::stable_sort(donors.begin(), donors.end(),
                   [](const std::pair<float, int64_t>& a, const std::pair<float, int64_t>& b) {
                     return a.first > b.first;
                   });
  int64_t moves = std::min<int64_t>(int64_t(dead.size()), int64_t(donors.size()));
  if (max_moves >= 0) moves = std::min(moves, max_moves);
  for (int64_t k = 0; k < moves; ++k) {
    const int64_t bi = dead[size_t(k)], bd = donors[size_t(k)].second;
    float mean[3];
    split_child_mean(params, n, bd, rand + 3 * bi, mean);
    for (int pl = 0; pl < P; ++pl) {
      float th = params[pl * n + bd];
      if (pl < 3) th = mean[pl];
      if (pl >= 3 && pl < 6) th = th - lscale_shrink;
      params[pl * n + bi] = th;
      m[pl * n + bi] = v[pl * n + bi] = 0.0f;
      m[pl * n + bd] = v[pl * n + bd] = 0.0f;
    }
    for (int pl = 3; pl < 6; ++pl) params[pl * n + bd] = params[pl * n + bd] - lscale_shrink;
  }
  return moves;
}

extern "C" {

int or_num_planes(int deg) { return num_planes(deg); }
void or_set_active_sh_degree(int d) { g_active_deg = d; }
void or_set_mip_compensation(int on) { g_mip = on ? 1 : 0; }

// Scalar helpers for the SH pins.
double or_sh_norm(int l, int m) { return sh_norm(l, m); }
void or_sh_basis_f64(const double* d, double* Y, double* dY) {
  double Yl[16], dYl[16][3];
  sh_basis<double>(d, Yl, dYl);
  for (int k = 0; k < 16; ++k) {
    Y[k] = Yl[k];
    for (int a = 0; a < 3; ++a) dY[3 * k + a] = dYl[k][a];
  }
}

#define OR_PREPROCESS(R, SUF)                                                                              \
  void or_preprocess_##SUF(int64_t n, int deg, const R* params, const Camera* cam, int smooth, R* uv,     \
                           R* conic, R* opac, R* rgb, R* depth, int32_t* rect, uint32_t* tiles,           \
                           uint8_t* visible, R* cov2d, R* extent) {                                        \
    for (int64_t i = 0; i < n; ++i) {                                                                      \
      Fwd<R> f = project<R>(params, n, i, deg, *cam, smooth != 0);                                         \
      visible[i] = f.visible ? 1 : 0;                                                                      \
      tiles[i] = f.visible ? f.tiles : 0;                                                                  \
      depth[i] = f.visible ? f.p[2] : R(0);                                                                \
      uv[i] = f.visible ? f.u : R(0);                                                                      \
      uv[n + i] = f.visible ? f.v : R(0);                                                                  \
      conic[i] = f.visible ? f.A : R(0);                                                                   \
      conic[n + i] = f.visible ? f.B : R(0);                                                               \
      conic[2 * n + i] = f.visible ? f.C : R(0);                                                           \
      opac[i] = f.visible ? f.o : R(0);                                                                    \
      for (int ch = 0; ch < 3; ++ch) rgb[ch * n + i] = f.visible ? f.rgb[ch] : R(0);                       \
      for (int k = 0; k < 4; ++k) rect[k * n + i] = (f.visible && !smooth) ? f.rect[k] : 0;                \
      if (extent) extent[i] = (f.visible && !smooth) ? f.rad : R(0);                                       \
      if (cov2d) {                                                                                         \
        cov2d[i] = f.visible ? f.a : R(0);                                                                 \
        cov2d[n + i] = f.visible ? f.b : R(0);                                                             \
        cov2d[2 * n + i] = f.visible ? f.c : R(0);                                                         \
      }                                                                                                    \
    }                                                                                                      \
  }
OR_PREPROCESS(float, f32)
OR_PREPROCESS(double, f64)

void or_bin_sort(int64_t n, const float* depth, const int32_t* rect, const uint32_t* tiles, int tx, int ty,
                 uint64_t* keys, uint32_t* vals, uint32_t* ranges) {
  bin_sort(n, depth, rect, tiles, tx, ty, keys, vals, ranges);
}

int64_t or_render_fwd_f32(int64_t n, const float* uv, const float* conic, const float* opac, const float* rgb,
                          const uint32_t* vals, const uint32_t* ranges, const Camera* cam, float* out_rgb,
                          float* T_final, uint32_t* n_contrib, uint32_t* n_examined, double* margin) {
  return render_tiled<float>(n, uv, conic, opac, rgb, vals, ranges, cam, out_rgb, T_final, n_contrib, n_examined,
                             margin, nullptr);
}

// The thresholded tiled forward in double, with every pixel's decision signature (for
// finite differences that keep only steps which change no decision).
int64_t or_render_fwd_f64(int64_t n, const double* uv, const double* conic, const double* opac, const double* rgb,
                          const uint32_t* vals, const uint32_t* ranges, const Camera* cam, double* out_rgb,
                          double* T_final, uint32_t* n_contrib, uint64_t* sig) {
  return render_tiled<double>(n, uv, conic, opac, rgb, vals, ranges, cam, out_rgb, T_final, n_contrib, nullptr,
                              nullptr, sig);
}

// Thresholded forward render without tiles: every pixel walks every visible
// Gaussian in (depth, id) order.  Equal to the tiled render whenever no
// Gaussian reaches alpha >= 1/255 outside its tile rectangle.
void or_render_untiled_f32(int64_t n, const float* uv, const float* conic, const float* opac, const float* rgb,
                           const float* depth, const uint8_t* visible, const Camera* cam, float* out_rgb,
                           float* T_final) {
  const int W = cam->width, H = cam->height;
  const int64_t HW = int64_t(W) * H;
  const float bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
  std::vector<uint32_t> list;
  smooth_order<float>(n, depth, visible, list);
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      float out[3], T;
      blend_pixel<float>(float(x) + 0.5f, float(y) + 0.5f, list.data(), int64_t(list.size()), uv, conic, opac,
                         rgb, n, bg, false, out, &T, nullptr, nullptr);
      const int64_t p = int64_t(y) * W + x;
      for (int ch = 0; ch < 3; ++ch) out_rgb[ch * HW + p] = out[ch];
      T_final[p] = T;
    }
}

// Forward render of a subset of pixels (for sampled checks at full size).
void or_render_pixels_f32(int64_t n, const float* uv, const float* conic, const float* opac, const float* rgb,
                          const uint32_t* vals, const uint32_t* ranges, const Camera* cam, int64_t npix,
                          const int32_t* px, const int32_t* py, float* out_rgb, float* T_final,
                          uint32_t* n_contrib, double* margin) {
  const int tx = tiles_x(*cam), ty = tiles_y(*cam);
  const int64_t nt = int64_t(tx) * ty;
  const float bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
  for (int64_t k = 0; k < npix; ++k) {
    const int x = px[k], y = py[k];
    const int64_t t = int64_t(y / kTile) * tx + x / kTile;
    const uint32_t s = ranges[t], e = ranges[nt + t];
    float out[3], T;
    PixelTrace tr;
    blend_pixel<float>(float(x) + 0.5f, float(y) + 0.5f, vals + s, int64_t(e) - s, uv, conic, opac, rgb, n, bg,
                       false, out, &T, &tr, nullptr);
    for (int ch = 0; ch < 3; ++ch) out_rgb[3 * k + ch] = out[ch];
    T_final[k] = T;
    n_contrib[k] = tr.n_contrib;
    margin[k] = tr.margin;
  }
}

// Depth complexity of a subset of pixels: how many entries of the pixel's tile list have
// an alpha (capped, as in the blend) of at least 1/255, over the whole list, with no early
// stop.  This is the quantity the high depth-complexity workload is built to make large
// (a median of at least 200 entries per pixel); the alpha is the blend's, [GST] opacity
// slide and [GSG] "The painting itself".
void or_overlap_pixels_f32(int64_t n, const float* uv, const float* conic, const float* opac, const uint32_t* vals,
                           const uint32_t* ranges, const Camera* cam, int64_t npix, const int32_t* px,
                           const int32_t* py, uint32_t* count) {
  const int tx = tiles_x(*cam), ty = tiles_y(*cam);
  const int64_t nt = int64_t(tx) * ty;
  for (int64_t k = 0; k < npix; ++k) {
    const float fx = float(px[k]) + 0.5f, fy = float(py[k]) + 0.5f;
    const int64_t t = int64_t(py[k] / kTile) * tx + px[k] / kTile;
    uint32_t c = 0;
    for (uint32_t i = ranges[t]; i < ranges[nt + t]; ++i) {
      const uint32_t g = vals[i];
      const float dx = fx - uv[g], dy = fy - uv[n + g];
      const float e = 0.5f * (conic[g] * dx * dx + conic[2 * n + g] * dy * dy) + conic[n + g] * dx * dy;
      const float alpha = std::min(float(kAlphaCap), opac[g] * exp_r(-e));
      if (!(alpha < alpha_min<float>())) ++c;
    }
    count[k] = c;
  }
}

// Tiled backward blend: gscreen [9][n] is overwritten; mass ([2][9][n]) and count
// ([n]), when given, are overwritten with the term magnitudes blend_pixel_bwd records.
void or_render_bwd_f32(int64_t n, const float* uv, const float* conic, const float* opac, const float* rgb,
                       const uint32_t* vals, const uint32_t* ranges, const Camera* cam, const float* T_final,
                       const uint32_t* n_contrib, const float* dLdI, float* gscreen, double* mass,
                       uint32_t* count) {
  const int W = cam->width, H = cam->height, tx = tiles_x(*cam);
  const int64_t HW = int64_t(W) * H;
  const float bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
  for (int64_t k = 0; k < 9 * n; ++k) gscreen[k] = 0.0f;
  if (mass)
    for (int64_t k = 0; k < 18 * n; ++k) mass[k] = 0.0;
  if (count)
    for (int64_t k = 0; k < n; ++k) count[k] = 0u;
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      const int64_t t = int64_t(y / kTile) * tx + x / kTile;
      const uint32_t s = ranges[t];
      const int64_t p = int64_t(y) * W + x;
      const float gI[3] = {dLdI[p], dLdI[HW + p], dLdI[2 * HW + p]};
      blend_pixel_bwd<float>(float(x) + 0.5f, float(y) + 0.5f, vals + s, n_contrib[p], uv, conic, opac, rgb, n,
                             bg, false, T_final[p], gI, gscreen, nullptr, mass, count);
    }
}

// The same backward in double (thresholds and the walk of or_render_bwd_f32, every
// product and sum in fp64), for checking the fp32 evaluation's rounding.
void or_render_bwd_f64(int64_t n, const double* uv, const double* conic, const double* opac, const double* rgb,
                       const uint32_t* vals, const uint32_t* ranges, const Camera* cam, const double* T_final,
                       const uint32_t* n_contrib, const double* dLdI, double* gscreen) {
  const int W = cam->width, H = cam->height, tx = tiles_x(*cam);
  const int64_t HW = int64_t(W) * H;
  const double bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
  for (int64_t k = 0; k < 9 * n; ++k) gscreen[k] = 0.0;
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      const int64_t t = int64_t(y / kTile) * tx + x / kTile;
      const int64_t p = int64_t(y) * W + x;
      const double gI[3] = {dLdI[p], dLdI[HW + p], dLdI[2 * HW + p]};
      blend_pixel_bwd<double>(double(x) + 0.5, double(y) + 0.5, vals + ranges[t], n_contrib[p], uv, conic, opac,
                              rgb, n, bg, false, T_final[p], gI, gscreen);
    }
}

// What rounding could change.  For every pixel, each decision whose margin (see
// exponent_scale) is below `below` is taken the other way, one at a time, and the
// pixel is blended forward and backward again (the backward from the flipped
// forward's transmittance and last entry, with the incoming image gradient dLdI
// unchanged).  Summed over those flips:
//   px_risk [2][H][W]  absolute change of the colour (largest channel) and of T;
//   nc_lo, nc_hi [H][W] the range of last-entry counts the flips produce (the
//                       unflipped count included);
//   grisk [9][n]        absolute change of each Gaussian's nine screen partials.
// Pixels with no such decision add nothing.  Optional (nullable): nflip [H][W], the
// number of decisions taken the other way at the pixel, and alt_rgb [3][H][W], alt_T,
// alt_nc [H][W], the pixel's colour, T and last-entry count with its last such decision
// taken the other way (the only one where nflip is 1).
// Optional obs_rgb [3][H][W], obs_T, obs_nc [H][W]: a render to be checked (another
// evaluation's forward).  Then grisk leaves out each flip that render rules out: at a
// pixel whose observed colour and T are within obs_atol of this walk's and whose count
// is this walk's, a flip that would move the colour or T by more than 2 obs_atol or
// change the count was not taken there.  (A cap flip never shows in the forward and is
// always kept.)  px_risk, nc_lo, nc_hi and the flip count are unchanged by this.
// Returns the number of flips taken.
int64_t or_flip_risk_f32(int64_t n, const float* uv, const float* conic, const float* opac, const float* rgb,
                         const uint32_t* vals, const uint32_t* ranges, const Camera* cam, const float* dLdI,
                         double below, float* px_risk, uint32_t* nc_lo, uint32_t* nc_hi, float* grisk,
                         uint32_t* nflip, float* alt_rgb, float* alt_T, uint32_t* alt_nc, const float* obs_rgb,
                         const float* obs_T, const uint32_t* obs_nc, double obs_atol) {
  const int W = cam->width, H = cam->height, tx = tiles_x(*cam), ty = tiles_y(*cam);
  const int64_t nt = int64_t(tx) * ty, HW = int64_t(W) * H;
  const float bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
  for (int64_t k = 0; k < 9 * n; ++k) grisk[k] = 0.0f;
  std::vector<Decision> close;
  // one pixel's partials, unflipped and flipped, kept at zero outside the entries just written
  std::vector<float> g0(size_t(9 * n), 0.0f), g1(size_t(9 * n), 0.0f);
  int64_t flips = 0;
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      const int64_t t = int64_t(y / kTile) * tx + x / kTile, p = int64_t(y) * W + x;
      const uint32_t s = ranges[t];
      const uint32_t* list = vals + s;
      const int64_t len = int64_t(ranges[nt + t]) - s;
      const float px = float(x) + 0.5f, py = float(y) + 0.5f;
      float out[3], T;
      PixelTrace tr;
      close.clear();
      blend_pixel<float>(px, py, list, len, uv, conic, opac, rgb, n, bg, false, out, &T, &tr, nullptr, nullptr,
                         &close, below);
      px_risk[p] = px_risk[HW + p] = 0.0f;
      nc_lo[p] = nc_hi[p] = tr.n_contrib;
      if (nflip) nflip[p] = uint32_t(close.size());
      if (alt_rgb)
        for (int ch = 0; ch < 3; ++ch) alt_rgb[ch * HW + p] = out[ch];
      if (alt_T) alt_T[p] = T;
      if (alt_nc) alt_nc[p] = tr.n_contrib;
      if (close.empty()) continue;
      const float gI[3] = {dLdI[p], dLdI[HW + p], dLdI[2 * HW + p]};
      blend_pixel_bwd<float>(px, py, list, tr.n_contrib, uv, conic, opac, rgb, n, bg, false, T, gI, g0.data());
      // does the observed render show this walk's outcome at the pixel?
      bool matched = obs_rgb != nullptr && obs_nc[p] == tr.n_contrib &&
                     std::fabs(double(obs_T[p]) - double(T)) <= obs_atol;
      for (int ch = 0; matched && ch < 3; ++ch)
        matched = std::fabs(double(obs_rgb[ch * HW + p]) - double(out[ch])) <= obs_atol;
      for (const Decision& f : close) {
        float out1[3], T1;
        PixelTrace tr1;
        blend_pixel<float>(px, py, list, len, uv, conic, opac, rgb, n, bg, false, out1, &T1, &tr1, nullptr, &f);
        float dc = 0.0f;
        for (int ch = 0; ch < 3; ++ch) dc = std::max(dc, std::fabs(out1[ch] - out[ch]));
        px_risk[p] += dc;
        px_risk[HW + p] += std::fabs(T1 - T);
        const bool visible = f.kind != kDecCap && (double(dc) > 2.0 * obs_atol ||
                                                   std::fabs(double(T1) - double(T)) > 2.0 * obs_atol ||
                                                   tr1.n_contrib != tr.n_contrib);
        const bool ruled_out = matched && visible;
        if (alt_rgb)
          for (int ch = 0; ch < 3; ++ch) alt_rgb[ch * HW + p] = out1[ch];
        if (alt_T) alt_T[p] = T1;
        if (alt_nc) alt_nc[p] = tr1.n_contrib;
        nc_lo[p] = std::min(nc_lo[p], tr1.n_contrib);
        nc_hi[p] = std::max(nc_hi[p], tr1.n_contrib);
        blend_pixel_bwd<float>(px, py, list, tr1.n_contrib, uv, conic, opac, rgb, n, bg, false, T1, gI, g1.data(),
                               &f);
        const uint32_t upto = std::max(tr.n_contrib, tr1.n_contrib);
        for (uint32_t j = 0; j < upto; ++j)
          for (int c = 0; c < 9; ++c) {
            const size_t o = size_t(c) * n + list[j];
            if (!ruled_out) grisk[o] += std::fabs(g1[o] - g0[o]);
            g1[o] = 0.0f;
          }
        ++flips;
      }
      for (uint32_t j = 0; j < tr.n_contrib; ++j)
        for (int c = 0; c < 9; ++c) g0[size_t(c) * n + list[j]] = 0.0f;
    }
  return flips;
}

#define OR_SMOOTH(R, SUF)                                                                                      \
  void or_render_smooth_fwd_##SUF(int64_t n, const R* uv, const R* conic, const R* opac, const R* rgb,        \
                                  const R* depth, const uint8_t* visible, const Camera* cam, R* out_rgb,      \
                                  R* T_final) {                                                                 \
    const int W = cam->width, H = cam->height;                                                                 \
    const int64_t HW = int64_t(W) * H;                                                                         \
    const R bg[3] = {R(cam->bg[0]), R(cam->bg[1]), R(cam->bg[2])};                                            \
    std::vector<uint32_t> list;                                                                                \
    smooth_order<R>(n, depth, visible, list);                                                                  \
    for (int y = 0; y < H; ++y)                                                                                \
      for (int x = 0; x < W; ++x) {                                                                            \
        R out[3], T;                                                                                           \
        blend_pixel<R>(R(x) + R(0.5), R(y) + R(0.5), list.data(), int64_t(list.size()), uv, conic, opac, rgb, \
                       n, bg, true, out, &T, nullptr, nullptr);                                                \
        const int64_t p = int64_t(y) * W + x;                                                                  \
        for (int ch = 0; ch < 3; ++ch) out_rgb[ch * HW + p] = out[ch];                                         \
        T_final[p] = T;                                                                                        \
      }                                                                                                        \
  }                                                                                                            \
  void or_render_smooth_bwd_##SUF(int64_t n, const R* uv, const R* conic, const R* opac, const R* rgb,        \
                                  const R* depth, const uint8_t* visible, const Camera* cam, const R* T_final, \
                                  const R* dLdI, R* gscreen) {                                                  \
    const int W = cam->width, H = cam->height;                                                                 \
    const int64_t HW = int64_t(W) * H;                                                                         \
    const R bg[3] = {R(cam->bg[0]), R(cam->bg[1]), R(cam->bg[2])};                                            \
    std::vector<uint32_t> list;                                                                                \
    smooth_order<R>(n, depth, visible, list);                                                                  \
    for (int64_t k = 0; k < 9 * n; ++k) gscreen[k] = R(0);                                                     \
    for (int y = 0; y < H; ++y)                                                                                \
      for (int x = 0; x < W; ++x) {                                                                            \
        const int64_t p = int64_t(y) * W + x;                                                                  \
        const R gI[3] = {dLdI[p], dLdI[HW + p], dLdI[2 * HW + p]};                                             \
        blend_pixel_bwd<R>(R(x) + R(0.5), R(y) + R(0.5), list.data(), int64_t(list.size()), uv, conic, opac,  \
                           rgb, n, bg, true, T_final[p], gI, gscreen);                                         \
      }                                                                                                        \
  }
OR_SMOOTH(float, f32)
OR_SMOOTH(double, f64)

#define OR_CHAIN(R, SUF)                                                                                        \
  void or_preprocess_bwd_##SUF(int64_t n, int deg, const R* params, const Camera* cam, int smooth,             \
                               const R* gscreen, R* gparams) {                                                 \
    for (int64_t i = 0; i < n; ++i) chain_one<R>(params, n, i, deg, *cam, smooth != 0, gscreen, gparams);      \
  }
OR_CHAIN(float, f32)
OR_CHAIN(double, f64)

#define OR_CAMERA_GRAD(R, SUF)                                                                                  \
  void or_camera_grad_##SUF(int64_t n, int deg, const R* params, const Camera* cam, int smooth, const R* gscreen, \
                            int position_only, double* out6) {                                                  \
    std::vector<R> scratch(size_t(num_planes(deg)) * size_t(n));                                              \
    for (int k = 0; k < 6; ++k) out6[k] = 0.0;                                                                \
    for (int64_t i = 0; i < n; ++i)                                                                           \
      chain_one<R>(params, n, i, deg, *cam, smooth != 0, gscreen, scratch.data(), out6, position_only != 0);  \
  }
OR_CAMERA_GRAD(float, f32)
OR_CAMERA_GRAD(double, f64)

#define OR_LOSS(R, SUF)                                                                                      \
  void or_loss_##SUF(const R* img, const R* tgt, int H, int W, R lambda, R* out3, R* grad, double* mag) {     \
    loss_l1_dssim<R>(img, tgt, H, W, lambda, out3, grad, mag);                                               \
  }
OR_LOSS(float, f32)
OR_LOSS(double, f64)

void or_adam_f64(double* params, const double* grads, double* m, double* v, int64_t n, int deg, const double* lr,
                 double b1, double b2, double eps, int step) {
  adam<double>(params, grads, m, v, n, deg, lr, b1, b2, eps, step);
}
void or_adam_f32(float* params, const float* grads, float* m, float* v, int64_t n, int deg, const double* lr,
                 double b1, double b2, double eps, int step) {
  adam<float>(params, grads, m, v, n, deg, lr, b1, b2, eps, step);
}

void or_loss_charbonnier_f32(const float* img, const float* tgt, int64_t count, float delta, float log_gain,
                             float bias, float* out3, float* grad) {
  loss_charbonnier<float>(img, tgt, count, delta, log_gain, bias, out3, grad);
}
void or_loss_charbonnier_f64(const double* img, const double* tgt, int64_t count, double delta, double log_gain,
                             double bias, double* out3, double* grad) {
  loss_charbonnier<double>(img, tgt, count, delta, log_gain, bias, out3, grad);
}

void or_densify_accumulate_f32(int64_t n, const uint32_t* tiles, const float* gscreen, float* stats) {
  densify_accumulate(n, tiles, gscreen, stats);
}

int64_t or_relocate_f32(int64_t n, int deg, float* params, float* m, float* v, const float* rand, float logit_dead,
                        float logit_donor, float lscale_shrink, int64_t max_moves) {
  return relocate(n, deg, params, m, v, rand, logit_dead, logit_donor, lscale_shrink, max_moves);
}

int64_t or_densify_f32(int64_t n, int deg, const float* params, const float* m, const float* v, const float* stats,
                       const float* rand, float grad_thr, float logit_prune, float lscale_prune, float lscale_split,
                       float lscale_shrink, int reset, float logit_cap, int64_t cap, float* params_out, float* m_out,
                       float* v_out, float* stats_out, int64_t* counts) {
  return densify(n, deg, params, m, v, stats, rand, grad_thr, logit_prune, lscale_prune, lscale_split, lscale_shrink,
                 reset, logit_cap, cap, params_out, m_out, v_out, stats_out, counts);
}

}  // extern "C"
