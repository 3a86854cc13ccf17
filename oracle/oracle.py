"""ctypes front end of the CPU oracle (oracle/gs_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the HIP library or its binding.

Every function takes and returns numpy arrays in the planar layouts of the
library ([plane][n] per Gaussian, [ch][H][W] per image).
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# GS_ORACLE_LIB selects another build of the same source (the sanitizer build of the
# CPU test job); the default is the one oracle/build.py writes.
LIB_PATH = os.environ.get("GS_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")


class OrCamera(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("campos", C.c_float * 3),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("width", C.c_int32), ("height", C.c_int32), ("znear", C.c_float), ("bg", C.c_float * 3)]


def make_camera(cam) -> OrCamera:
    c = OrCamera()
    c.R[:] = [float(x) for x in np.asarray(cam.R, dtype=np.float32).reshape(9)]
    c.t[:] = [float(x) for x in np.asarray(cam.t, dtype=np.float32)]
    c.campos[:] = [float(x) for x in np.asarray(cam.campos, dtype=np.float32)]
    c.fx, c.fy, c.cx, c.cy = cam.fx, cam.fy, cam.cx, cam.cy
    c.width, c.height = cam.width, cam.height
    c.znear = cam.znear
    c.bg[:] = [float(x) for x in cam.bg]
    return c


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433 (build on first use)
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p
I64 = C.c_int64
I32 = C.c_int


def _declare(L):
    L.or_num_planes.argtypes = [I32]
    L.or_set_active_sh_degree.argtypes = [I32]
    L.or_set_mip_compensation.argtypes = [I32]
    for suf in ("f32", "f64"):
        getattr(L, f"or_camera_grad_{suf}").argtypes = [I64, I32, P, P, I32, P, I32, P]
    L.or_num_planes.restype = I32
    L.or_sh_norm.argtypes = [I32, I32]
    L.or_sh_norm.restype = C.c_double
    L.or_sh_basis_f64.argtypes = [P, P, P]
    for suf in ("f32", "f64"):
        getattr(L, f"or_preprocess_{suf}").argtypes = [I64, I32, P, P, I32] + [P] * 10
        getattr(L, f"or_render_smooth_fwd_{suf}").argtypes = [I64] + [P] * 7 + [P, P]
        getattr(L, f"or_render_smooth_bwd_{suf}").argtypes = [I64] + [P] * 7 + [P, P, P]
        getattr(L, f"or_preprocess_bwd_{suf}").argtypes = [I64, I32, P, P, I32, P, P]
        getattr(L, f"or_adam_{suf}").argtypes = [P, P, P, P, I64, I32, P, C.c_double, C.c_double,
                                                 C.c_double, I32]
    L.or_loss_f32.argtypes = [P, P, I32, I32, C.c_float, P, P, P]
    L.or_loss_f64.argtypes = [P, P, I32, I32, C.c_double, P, P, P]
    L.or_bin_sort.argtypes = [I64, P, P, P, I32, I32, P, P, P]
    L.or_render_fwd_f32.argtypes = [I64] + [P] * 6 + [P] + [P] * 5
    L.or_render_fwd_f32.restype = I64
    L.or_render_fwd_f64.argtypes = [I64] + [P] * 6 + [P] + [P] * 4
    L.or_render_fwd_f64.restype = I64
    L.or_render_untiled_f32.argtypes = [I64] + [P] * 6 + [P, P, P]
    L.or_render_pixels_f32.argtypes = [I64] + [P] * 6 + [P, I64, P, P, P, P, P, P]
    L.or_overlap_pixels_f32.argtypes = [I64] + [P] * 5 + [P, I64, P, P, P]
    L.or_render_bwd_f32.argtypes = [I64] + [P] * 6 + [P] + [P] * 6
    L.or_render_bwd_f64.argtypes = [I64] + [P] * 6 + [P] + [P] * 4
    L.or_flip_risk_f32.argtypes = [I64] + [P] * 6 + [P, P, C.c_double, P, P, P, P, P, P, P, P, P, P, P,
                                                     C.c_double]
    L.or_flip_risk_f32.restype = I64
    L.or_densify_accumulate_f32.argtypes = [I64, P, P, P]
    L.or_loss_charbonnier_f32.argtypes = [P, P, I64, C.c_float, C.c_float, C.c_float, P, P]
    L.or_loss_charbonnier_f64.argtypes = [P, P, I64, C.c_double, C.c_double, C.c_double, P, P]
    F = C.c_float
    L.or_densify_f32.argtypes = [I64, I32, P, P, P, P, P, F, F, F, F, F, I32, F, I64, P, P, P, P, P]
    L.or_densify_f32.restype = I64
    L.or_relocate_f32.argtypes = [I64, I32, P, P, P, P, F, F, F, I64]
    L.or_relocate_f32.restype = I64


@contextlib.contextmanager
def library(path):
    """Run the oracle functions against another build of gs_oracle.cpp (the tests'
    planted-mistake variants) for the duration of the block."""
    global _lib
    saved = lib()
    alt = C.CDLL(path)
    _declare(alt)
    _lib = alt
    try:
        yield
    finally:
        _lib = saved


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_planes(deg):
    return lib().or_num_planes(deg)


def set_active_sh_degree(d):
    """SH degree ramp: only bands up to d are evaluated and receive gradients (-1: all)."""
    lib().or_set_active_sh_degree(int(d))


def set_mip_compensation(on):
    """Mip-Splatting opacity compensation: the record's opacity becomes
    sigmoid(logit) sqrt(det V / det(V + 0.3 I)) (off by default)."""
    lib().or_set_mip_compensation(int(bool(on)))


# ----------------------------------------------------------------- forward
def preprocess(params, sh_degree, cam, smooth=False, dtype=np.float32):
    """Per-Gaussian projection. Returns a dict of planar arrays."""
    params = _c(params, dtype)
    n = params.shape[1]
    out = dict(uv=np.zeros((2, n), dtype), conic=np.zeros((3, n), dtype), opac=np.zeros(n, dtype),
               rgb=np.zeros((3, n), dtype), depth=np.zeros(n, dtype), rect=np.zeros((4, n), np.int32),
               tiles=np.zeros(n, np.uint32), visible=np.zeros(n, np.uint8), cov2d=np.zeros((3, n), dtype),
               extent=np.zeros(n, dtype))
    fn = lib().or_preprocess_f32 if dtype == np.float32 else lib().or_preprocess_f64
    c = make_camera(cam)
    fn(n, sh_degree, _p(params), C.byref(c), int(smooth), _p(out["uv"]), _p(out["conic"]), _p(out["opac"]),
       _p(out["rgb"]), _p(out["depth"]), _p(out["rect"]), _p(out["tiles"]), _p(out["visible"]),
       _p(out["cov2d"]), _p(out["extent"]))
    out["n"] = n
    return out


def bin_sort(pre, cam):
    """Keys, ids and per-tile ranges ([2][tiles]) of the stable (tile, depth, id) order."""
    n = pre["n"]
    total = int(pre["tiles"].astype(np.int64).sum())
    keys = np.zeros(total, np.uint64)
    vals = np.zeros(total, np.uint32)
    nt = cam.tiles_x * cam.tiles_y
    ranges = np.zeros((2, nt), np.uint32)
    lib().or_bin_sort(n, _p(_c(pre["depth"], np.float32)), _p(pre["rect"]), _p(pre["tiles"]), cam.tiles_x,
                      cam.tiles_y, _p(keys), _p(vals), _p(ranges))
    return keys, vals, ranges


def render_fwd(pre, vals, ranges, cam):
    n = pre["n"]
    H, W = cam.height, cam.width
    out = dict(rgb=np.zeros((3, H, W), np.float32), T=np.zeros((H, W), np.float32),
               n_contrib=np.zeros((H, W), np.uint32), n_examined=np.zeros((H, W), np.uint32),
               margin=np.zeros((H, W), np.float64))
    c = make_camera(cam)
    out["evals"] = int(lib().or_render_fwd_f32(
        n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]), _p(_c(vals, np.uint32)),
        _p(_c(ranges, np.uint32)), C.byref(c), _p(out["rgb"]), _p(out["T"]), _p(out["n_contrib"]),
        _p(out["n_examined"]), _p(out["margin"])))
    return out


def render_thresholded(params, sh_degree, cam):
    """The thresholded path (cull, tile rectangle, sort, skip, cap, stop, colour clamp) with
    every operation in fp64: image, T, n_contrib and each pixel's decision signature
    (`sig`), with the projection, the sorted ids and the ranges it used."""
    pre = preprocess(params, sh_degree, cam, dtype=np.float64)
    _, vals, ranges = bin_sort(pre, cam)
    n = pre["n"]
    H, W = cam.height, cam.width
    out = dict(rgb=np.zeros((3, H, W), np.float64), T=np.zeros((H, W), np.float64),
               n_contrib=np.zeros((H, W), np.uint32), sig=np.zeros((H, W), np.uint64))
    c = make_camera(cam)
    lib().or_render_fwd_f64(n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]), _p(vals),
                            _p(ranges), C.byref(c), _p(out["rgb"]), _p(out["T"]), _p(out["n_contrib"]),
                            _p(out["sig"]))
    out.update(pre=pre, vals=vals, ranges=ranges)
    return out


def decisions(r):
    """Everything a thresholded render decides, from render_thresholded's result: culls,
    tile rectangles, clamped colour channels (a clamped channel is exactly 0), the pair
    order, and per pixel the skip / cap / stop outcomes.  Two renders with equal decisions
    lie on one smooth piece of the rendering function."""
    pre = r["pre"]
    return (pre["visible"], pre["rect"], pre["tiles"], pre["rgb"] == 0.0, r["vals"], r["ranges"], r["sig"])


def same_decisions(a, b):
    return all(np.array_equal(x, y) for x, y in zip(decisions(a), decisions(b)))


def thresholded_grad(params, sh_degree, cam, dLdI):
    """Analytic gradient, in fp64, of sum(dLdI * render_thresholded(params)) with respect
    to the parameters (the blend's backward walk and the chain with every threshold in place)."""
    r = render_thresholded(params, sh_degree, cam)
    gscreen = render_bwd_f64(r["pre"], r["vals"], r["ranges"], cam, r, dLdI)
    return preprocess_bwd(params, sh_degree, cam, gscreen, dtype=np.float64), gscreen, r


def render_untiled(pre, cam):
    H, W = cam.height, cam.width
    img = np.zeros((3, H, W), np.float32)
    T = np.zeros((H, W), np.float32)
    c = make_camera(cam)
    lib().or_render_untiled_f32(pre["n"], _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]),
                                _p(pre["depth"]), _p(pre["visible"]), C.byref(c), _p(img), _p(T))
    return img, T


def render_pixels(pre, vals, ranges, cam, xs, ys):
    n = pre["n"]
    xs = _c(xs, np.int32)
    ys = _c(ys, np.int32)
    k = xs.shape[0]
    rgb = np.zeros((k, 3), np.float32)
    T = np.zeros(k, np.float32)
    nc = np.zeros(k, np.uint32)
    margin = np.zeros(k, np.float64)
    c = make_camera(cam)
    lib().or_render_pixels_f32(n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]),
                               _p(_c(vals, np.uint32)), _p(_c(ranges, np.uint32)), C.byref(c), k, _p(xs),
                               _p(ys), _p(rgb), _p(T), _p(nc), _p(margin))
    return dict(rgb=rgb, T=T, n_contrib=nc, margin=margin)


def overlap_pixels(pre, vals, ranges, cam, xs, ys):
    """Per listed pixel, the entries of its tile's list whose alpha reaches 1/255, counted
    over the whole list (no early stop): the depth complexity a workload puts on it."""
    xs = _c(xs, np.int32)
    ys = _c(ys, np.int32)
    count = np.zeros(xs.shape[0], np.uint32)
    c = make_camera(cam)
    lib().or_overlap_pixels_f32(pre["n"], _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(_c(vals, np.uint32)),
                                _p(_c(ranges, np.uint32)), C.byref(c), xs.shape[0], _p(xs), _p(ys), _p(count))
    return count


def render_bwd(pre, vals, ranges, cam, fwd, dLdI, with_mass=False):
    """Screen-space partials [9][n] (u, v, A, B, C, opacity, r, g, b).  With with_mass,
    also (mass [2][9][n], count [n]): the magnitudes of the terms each partial sums
    (plain, and weighted by twice the walk length plus 16) and the contributing pixels."""
    n = pre["n"]
    gscreen = np.zeros((9, n), np.float32)
    mass = np.zeros((2, 9, n), np.float64) if with_mass else None
    count = np.zeros(n, np.uint32) if with_mass else None
    c = make_camera(cam)
    lib().or_render_bwd_f32(n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]),
                            _p(_c(vals, np.uint32)), _p(_c(ranges, np.uint32)), C.byref(c), _p(fwd["T"]),
                            _p(fwd["n_contrib"]), _p(_c(dLdI, np.float32)), _p(gscreen),
                            _p(mass) if with_mass else None, _p(count) if with_mass else None)
    return (gscreen, mass, count) if with_mass else gscreen


def render_bwd_f64(pre, vals, ranges, cam, fwd, dLdI):
    """render_bwd with every operation in fp64 (same thresholds, same walk lengths)."""
    n = pre["n"]
    d = lambda a: _c(a, np.float64)
    gscreen = np.zeros((9, n), np.float64)
    c = make_camera(cam)
    lib().or_render_bwd_f64(n, _p(d(pre["uv"])), _p(d(pre["conic"])), _p(d(pre["opac"])), _p(d(pre["rgb"])),
                            _p(_c(vals, np.uint32)), _p(_c(ranges, np.uint32)), C.byref(c), _p(d(fwd["T"])),
                            _p(fwd["n_contrib"]), _p(d(dLdI)), _p(gscreen))
    return gscreen


def rounding_slack(mass, count):
    """Bound [9][n] on the difference between two fp32 evaluations of the screen partials
    that sum the same terms in different orders with differently rounded terms: each
    term carries at most about (2 walk + 16) roundings of its magnitude, and a sum of
    count terms at most count roundings of their total magnitude (unit 2^-24, both
    sides)."""
    return (2.0 ** -22) * mass[1] + (2.0 ** -23) * count.astype(np.float64) * mass[0]


# Decisions whose conditioned margin is below this are taken the other way by
# flip_risk.  Two fp32 evaluations of alpha (different operation order, FMA, a
# one-ulp exp) differ by at most about 14 roundings, 8.4e-7, per unit of the
# conditioning scale; 1e-5 leaves a factor of twelve.
RISK_BELOW = 1e-5


def flip_risk(pre, vals, ranges, cam, dLdI, below=RISK_BELOW, observed=None, obs_atol=1e-5):
    """How much an fp32 evaluation other than the oracle's could move each output:
    px [2][H][W] (colour, largest channel; T), nc_lo / nc_hi [H][W] (range of
    n_contrib), g [9][n] (screen partials), and the number of flips taken.  Per pixel
    also nflip [H][W] (its decisions near a threshold) and alt_rgb [3][H][W], alt_T,
    alt_nc [H][W]: the pixel with its (last) near decision taken the other way, which
    is the pixel's one alternative where nflip is 1.  With observed (a dict with rgb, T,
    n_contrib of another evaluation's forward), g leaves out the flips that render shows
    were not taken (see or_flip_risk_f32)."""
    n = pre["n"]
    H, W = cam.height, cam.width
    out = dict(px=np.zeros((2, H, W), np.float32), nc_lo=np.zeros((H, W), np.uint32),
               nc_hi=np.zeros((H, W), np.uint32), g=np.zeros((9, n), np.float32),
               nflip=np.zeros((H, W), np.uint32), alt_rgb=np.zeros((3, H, W), np.float32),
               alt_T=np.zeros((H, W), np.float32), alt_nc=np.zeros((H, W), np.uint32))
    c = make_camera(cam)
    out["flips"] = int(lib().or_flip_risk_f32(
        n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]), _p(_c(vals, np.uint32)),
        _p(_c(ranges, np.uint32)), C.byref(c), _p(_c(dLdI, np.float32)), float(below), _p(out["px"]),
        _p(out["nc_lo"]), _p(out["nc_hi"]), _p(out["g"]), _p(out["nflip"]), _p(out["alt_rgb"]),
        _p(out["alt_T"]), _p(out["alt_nc"]),
        _p(_c(observed["rgb"], np.float32)) if observed is not None else None,
        _p(_c(observed["T"], np.float32)) if observed is not None else None,
        _p(_c(observed["n_contrib"], np.uint32)) if observed is not None else None, float(obs_atol)))
    return out


def preprocess_bwd(params, sh_degree, cam, gscreen, smooth=False, dtype=np.float32):
    params = _c(params, dtype)
    gscreen = _c(gscreen, dtype)
    n = params.shape[1]
    g = np.zeros_like(params)
    fn = lib().or_preprocess_bwd_f32 if dtype == np.float32 else lib().or_preprocess_bwd_f64
    c = make_camera(cam)
    fn(n, sh_degree, _p(params), C.byref(c), int(smooth), _p(gscreen), _p(g))
    return g


# ------------------------------------------------------------- smooth mode
def smooth_render(params, sh_degree, cam, dtype=np.float64):
    """Render with every threshold off (all Gaussians, all pixels, depth order)."""
    pre = preprocess(params, sh_degree, cam, smooth=True, dtype=dtype)
    H, W = cam.height, cam.width
    img = np.zeros((3, H, W), dtype)
    T = np.zeros((H, W), dtype)
    fn = lib().or_render_smooth_fwd_f64 if dtype == np.float64 else lib().or_render_smooth_fwd_f32
    c = make_camera(cam)
    fn(pre["n"], _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]), _p(pre["depth"]),
       _p(pre["visible"]), C.byref(c), _p(img), _p(T))
    return img, T, pre


def smooth_grad(params, sh_degree, cam, dLdI, dtype=np.float64):
    """Analytic gradient of sum(dLdI * smooth_render) with respect to the parameters."""
    img, T, pre = smooth_render(params, sh_degree, cam, dtype)
    n = pre["n"]
    gscreen = np.zeros((9, n), dtype)
    fn = lib().or_render_smooth_bwd_f64 if dtype == np.float64 else lib().or_render_smooth_bwd_f32
    c = make_camera(cam)
    fn(n, _p(pre["uv"]), _p(pre["conic"]), _p(pre["opac"]), _p(pre["rgb"]), _p(pre["depth"]),
       _p(pre["visible"]), C.byref(c), _p(T), _p(_c(dLdI, dtype)), _p(gscreen))
    return preprocess_bwd(params, sh_degree, cam, gscreen, smooth=True, dtype=dtype), gscreen, img


# -------------------------------------------------------------------- loss
def loss(img, tgt, lam=0.2, dtype=np.float64, with_grad=True, with_mag=False):
    """0.8 L1 + 0.2 (1 - SSIM); returns ((total, L1, SSIM), dL/dimg), and with with_mag
    also the per-element magnitude of the SSIM terms the gradient sums ([3][H][W])."""
    img = _c(img, dtype)
    tgt = _c(tgt, dtype)
    _, H, W = img.shape
    out = np.zeros(3, dtype)
    grad = np.zeros_like(img) if (with_grad or with_mag) else None
    mag = np.zeros(img.shape, np.float64) if with_mag else None
    fn = lib().or_loss_f64 if dtype == np.float64 else lib().or_loss_f32
    fn(_p(img), _p(tgt), H, W, lam, _p(out), _p(grad), _p(mag))
    terms = tuple(float(x) for x in out)
    return (terms, grad, mag) if with_mag else (terms, grad)


# -------------------------------------------------------------------- Adam
def adam(params, grads, m, v, sh_degree, lr, step, b1=0.9, b2=0.999, eps=1e-8, dtype=np.float64):
    """Returns updated (params, m, v) as new arrays."""
    params = np.array(params, dtype=dtype, copy=True)
    m = np.array(m, dtype=dtype, copy=True)
    v = np.array(v, dtype=dtype, copy=True)
    grads = _c(grads, dtype)
    lr = np.ascontiguousarray(lr, dtype=np.float64)
    n = params.shape[1]
    fn = lib().or_adam_f64 if dtype == np.float64 else lib().or_adam_f32
    fn(_p(params), _p(grads), _p(m), _p(v), n, sh_degree, _p(lr), b1, b2, eps, step)
    return params, m, v


def sh_basis(d):
    d = np.ascontiguousarray(d, np.float64)
    Y = np.zeros(16)
    dY = np.zeros(48)
    lib().or_sh_basis_f64(_p(d), _p(Y), _p(dY))
    return Y, dY.reshape(16, 3)


# ------------------------------------------------------------ full forward
def forward(scene_params, sh_degree, cam):
    """Preprocess, bin/sort and render: everything the forward path produces."""
    pre = preprocess(scene_params, sh_degree, cam)
    keys, vals, ranges = bin_sort(pre, cam)
    fwd = render_fwd(pre, vals, ranges, cam)
    return pre, keys, vals, ranges, fwd


def train_step(scene_params, sh_degree, cam, target, lam=0.2, with_mass=False):
    """The method's step for one camera: forward, loss, backward blend and chain (Adam is
    oracle.adam).  Returns a dict of every stage's output; with_mass adds the term
    magnitudes of the screen partials (render_bwd)."""
    pre, keys, vals, ranges, fwd = forward(scene_params, sh_degree, cam)
    (total, l1, ssim), dLdI = loss(fwd["rgb"], target, lam)
    r = render_bwd(pre, vals, ranges, cam, fwd, dLdI.astype(np.float32), with_mass=with_mass)
    gscreen = r[0] if with_mass else r
    gparams = preprocess_bwd(scene_params, sh_degree, cam, gscreen)
    out = dict(pre=pre, keys=keys, vals=vals, ranges=ranges, fwd=fwd, loss=(total, l1, ssim), dLdI=dLdI,
               gscreen=gscreen, gparams=gparams)
    if with_mass:
        out["mass"], out["count"] = r[1], r[2]
    return out


def train_step_grads(scene_params, sh_degree, cam, target, lam=0.2):
    """train_step plus what the parity checks need: the flip risk of the blend decisions
    and the rounding slack of the screen partials."""
    out = train_step(scene_params, sh_degree, cam, target, lam, with_mass=True)
    out["risk"] = flip_risk(out["pre"], out["vals"], out["ranges"], cam, out["dLdI"].astype(np.float32))
    out["slack"] = rounding_slack(out.pop("mass"), out.pop("count"))
    return out


# ---------------------------------------------------------- density control
def densify_thresholds(prune_opacity, prune_scale, split_scale, opacity_cap, shrink=1.6):
    """The thresholds in the domains the parameters are stored in, each formed in fp64
    and rounded once to fp32: logit of the prune opacity and of the reset cap, log of the
    prune and split scales and of the split shrink factor."""
    import math

    def logit(p):
        return math.log(p / (1.0 - p))

    def log_or_inf(x):
        return math.inf if math.isinf(x) else math.log(x)
    return dict(logit_prune=np.float32(logit(prune_opacity)), lscale_prune=np.float32(log_or_inf(prune_scale)),
                lscale_split=np.float32(math.log(split_scale)), logit_cap=np.float32(logit(opacity_cap)),
                lscale_shrink=np.float32(math.log(shrink)))


def densify_accumulate(tiles, gscreen, stats):
    """One step's observations added to stats [n][2] (a new array): a Gaussian with a
    nonzero tile count adds the length of its screen-position gradient (du, dv) and 1."""
    stats = np.array(stats, dtype=np.float32, copy=True)
    n = stats.shape[0]
    lib().or_densify_accumulate_f32(n, _p(_c(tiles, np.uint32)), _p(_c(gscreen, np.float32)), _p(stats))
    return stats


def densify(params, m, v, stats, rand, sh_degree, grad_threshold, prune_opacity, prune_scale, split_scale,
            reset_opacity=False, opacity_cap=0.01, shrink=1.6):
    """One densification of the planar [P][n] population (see gs_oracle.cpp): returns the
    new params, m, v ([P][n_new]), zeroed stats [n_new][2] and the counts (kept, cloned,
    split).  rand [n][2][3]: the standard normals of each Gaussian's two split children."""
    params = _c(params, np.float32)
    m = _c(m, np.float32)
    v = _c(v, np.float32)
    stats = _c(stats, np.float32)
    rand = _c(rand, np.float32)
    P, n = params.shape
    t = densify_thresholds(prune_opacity, prune_scale, split_scale, opacity_cap, shrink)
    counts = np.zeros(3, np.int64)
    args = (n, sh_degree, _p(params), _p(m), _p(v), _p(stats), _p(rand), float(np.float32(grad_threshold)),
            float(t["logit_prune"]), float(t["lscale_prune"]), float(t["lscale_split"]), float(t["lscale_shrink"]),
            int(bool(reset_opacity)), float(t["logit_cap"]))
    total = lib().or_densify_f32(*args, 0, None, None, None, None, _p(counts))
    po, mo, vo = (np.zeros((P, total), np.float32) for _ in range(3))
    so = np.zeros((total, 2), np.float32)
    lib().or_densify_f32(*args, total, _p(po), _p(mo), _p(vo), _p(so), _p(counts))
    return dict(params=po, m=mo, v=vo, stats=so, counts=counts)


def relocate(params, m, v, rand, sh_degree, dead_opacity=0.02, donor_opacity=0.4, shrink=1.6, max_moves=-1):
    """The MCMC-style relocation of the dead Gaussians to the largest donors (see
    gs_oracle.cpp): returns new params, m, v ([P][n]) and the number of moves.  rand [n][3]:
    each Gaussian's normals for the place it would be moved to."""
    import math
    params = np.array(params, dtype=np.float32, copy=True, order="C")
    m = np.array(m, dtype=np.float32, copy=True, order="C")
    v = np.array(v, dtype=np.float32, copy=True, order="C")
    rand = _c(rand, np.float32)
    n = params.shape[1]
    lg = lambda p: float(np.float32(math.log(p / (1.0 - p))))   # noqa: E731
    moves = lib().or_relocate_f32(n, sh_degree, _p(params), _p(m), _p(v), _p(rand), lg(dead_opacity),
                                  lg(donor_opacity), float(np.float32(math.log(shrink))), int(max_moves))
    return dict(params=params, m=m, v=v, moves=int(moves))


# ------------------------------------------- Charbonnier loss with exposure
def loss_charbonnier(img, tgt, delta=0.03, log_gain=0.0, bias=0.0, dtype=np.float64):
    """Mean over the elements of sqrt((gain img + bias - tgt)^2 + delta^2) - delta, gain =
    exp(log_gain); returns (loss, dL/dimg, dL/dlog_gain, dL/dbias)."""
    img = _c(img, dtype)
    tgt = _c(tgt, dtype)
    out = np.zeros(3, dtype)
    grad = np.zeros_like(img)
    fn = lib().or_loss_charbonnier_f64 if dtype == np.float64 else lib().or_loss_charbonnier_f32
    fn(_p(img), _p(tgt), img.size, delta, log_gain, bias, _p(out), _p(grad))
    return out[0], grad, out[1], out[2]


# ------------------------------------------------------ camera-pose gradient
def camera_grad(params, sh_degree, cam, gscreen, smooth=False, dtype=np.float32, position_only=False):
    """Gradient of the loss with respect to the camera pose from the screen partials
    ([9][n]): (rotation, perturbed on the left as W <- (I + [w]x) W; translation), summed
    over the visible Gaussians in fp64 (see camera_grad_terms in gs_oracle.cpp).  With
    position_only, the trainer's terms: the torque (p - t) x dp and dp alone."""
    params = _c(params, dtype)
    gscreen = _c(gscreen, dtype)
    out = np.zeros(6, np.float64)
    c = make_camera(cam)
    fn = lib().or_camera_grad_f64 if dtype == np.float64 else lib().or_camera_grad_f32
    fn(params.shape[1], sh_degree, _p(params), C.byref(c), int(smooth), _p(gscreen), int(bool(position_only)),
       _p(out))
    return out
