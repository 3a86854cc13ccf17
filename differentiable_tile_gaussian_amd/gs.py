"""ctypes binding of libgs.so (include/gs.h).

The functions below have the names of the C entry points and do argument
marshalling only: torch tensors supply device memory and the current HIP stream,
every step of the rasteriser runs in the library's HIP kernels.  There is no CPU
fallback: if libgs.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime the library then binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgs.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_CAPACITY, GS_ERR_UNSUPPORTED, GS_ERR_HIP = 0, -1, -2, -3, -4
GS_WS_PREPROCESS, GS_WS_BIN_SORT, GS_WS_LOSS, GS_WS_RENDER, GS_WS_DENSIFY, GS_WS_LOSS_CHARBONNIER = 0, 1, 2, 3, 4, 5
GS_WS_CAMERA_GRAD, GS_WS_RELOCATE = 6, 7
GS_GRAD_SUMS_FLOAT, GS_GRAD_SUMS_FIXED = 0, 1

EXPORTED = ("gs_preprocess", "gs_bin_sort", "gs_render_fwd", "gs_loss_l1_dssim", "gs_render_bwd",
            "gs_adam_step", "gs_render_bwd_adam", "gs_render_bwd_adam_project", "gs_render_bwd_weighted",
            "gs_camera_grad", "gs_densify_accumulate", "gs_densify", "gs_relocate", "gs_loss_charbonnier",
            "gs_workspace_bytes", "gs_loss_l1_dssim_noalloc", "gs_profile_enable", "gs_profile_query", "gs_param_floats", "gs_params_to_blocked",
            "gs_params_from_blocked", "gs_last_error")


class GsError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"gs status {status}: {message}")
        self.status = status


class GsCamera(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("campos", C.c_float * 3),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("width", C.c_int32), ("height", C.c_int32), ("znear", C.c_float), ("bg", C.c_float * 3)]


class GsScene(C.Structure):
    _fields_ = [("n", C.c_int64), ("sh_degree", C.c_int32), ("params", C.c_void_p)]


class GsConfig(C.Structure):
    """gs_config: the per-call settings (defaults: float sums, every SH band, no Mip
    compensation, the default split sizes)."""
    _fields_ = [("grad_sums", C.c_int32), ("active_sh_degree", C.c_int32), ("mip_compensation", C.c_int32),
                ("split_first", C.c_int32), ("split_chunk", C.c_int32)]

    def __init__(self, grad_sums=GS_GRAD_SUMS_FLOAT, active_sh_degree=-1, mip_compensation=False, split_first=0,
                 split_chunk=0):
        super().__init__(int(grad_sums), int(active_sh_degree), int(bool(mip_compensation)), int(split_first),
                         int(split_chunk))


def _cfg(cfg):
    return None if cfg is None else C.byref(cfg)


class GsProj(C.Structure):
    _fields_ = [("splat", C.c_void_p), ("depth", C.c_void_p), ("rect", C.c_void_p), ("tiles", C.c_void_p),
                ("order", C.c_void_p), ("n_visible", C.c_void_p), ("offs", C.c_void_p), ("rect_order", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    P, I64, I32, U32 = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32
    lib.gs_preprocess.argtypes = [P, P, P, P, P, C.c_size_t, P, P]
    lib.gs_bin_sort.argtypes = [P, I64, P, U32, P, P, U32, P, P, C.c_size_t, P]
    lib.gs_render_fwd.argtypes = [P, I64, P, P, U32, P, P, P, P, P, C.c_size_t, P, P]
    lib.gs_loss_l1_dssim.argtypes = [P, P, I32, I32, C.c_float, P, P, P, C.c_size_t, P]
    lib.gs_render_bwd.argtypes = [P, P, P, P, U32, P, P, P, P, P, P, P, C.c_size_t, P, P]
    lib.gs_render_bwd_adam.argtypes = [P, I64, I32, P, P, P, U32, P, P, P, P, P, P, P, P, C.c_double, C.c_double,
                                       C.c_double, I32, P, C.c_size_t, P, P]
    lib.gs_render_bwd_adam.restype = I32
    lib.gs_render_bwd_adam_project.argtypes = [P, I64, I32, P, P, P, U32, P, P, P, P, P, P, P, P, C.c_double,
                                               C.c_double, C.c_double, I32, P, C.c_size_t, P, P, P, P, C.c_size_t,
                                               P, P, P]
    lib.gs_render_bwd_adam_project.restype = I32
    lib.gs_loss_l1_dssim_noalloc.argtypes = [P, P, I32, I32, C.c_float, P, P, P]
    lib.gs_loss_l1_dssim_noalloc.restype = I32
    lib.gs_loss_charbonnier.argtypes = [P, P, I32, I32, C.c_float, P, P, P, P, P, C.c_size_t, P]
    lib.gs_loss_charbonnier.restype = I32
    lib.gs_render_bwd_weighted.argtypes = [P, P, P, P, U32, P, P, P, P, P, P, C.c_float, I32, P, C.c_size_t, P, P]
    lib.gs_render_bwd_weighted.restype = I32
    lib.gs_camera_grad.argtypes = [P, P, P, P, I32, P, P, C.c_size_t, P, P]
    lib.gs_relocate.argtypes = [P, P, P, I64, I32, P, C.c_double, C.c_double, I64, P, P, C.c_size_t, P]
    lib.gs_relocate.restype = I32
    lib.gs_camera_grad.restype = I32
    lib.gs_densify_accumulate.argtypes = [P, I64, P, P, P]
    lib.gs_densify_accumulate.restype = I32
    D = C.c_double
    lib.gs_densify.argtypes = [P, P, P, P, P, I64, I32, D, D, D, D, I32, D, P, P, P, P, I64, P, P, P, C.c_size_t, P]
    lib.gs_densify.restype = I32
    lib.gs_adam_step.argtypes = [P, P, P, P, I64, I32, P, C.c_double, C.c_double, C.c_double, I32, P]
    lib.gs_profile_enable.argtypes = [I32, C.c_char_p]
    lib.gs_profile_enable.restype = I32
    lib.gs_profile_query.argtypes = [I32, P, P, P]
    lib.gs_profile_query.restype = I32
    lib.gs_param_floats.argtypes = [I64, I32]
    lib.gs_param_floats.restype = C.c_size_t
    lib.gs_params_to_blocked.argtypes = [P, P, I64, I32, P]
    lib.gs_params_to_blocked.restype = I32
    lib.gs_params_from_blocked.argtypes = [P, P, I64, I32, P]
    lib.gs_params_from_blocked.restype = I32
    lib.gs_workspace_bytes.argtypes = [I32, I64, U32, I32, I32, P]
    lib.gs_workspace_bytes.restype = C.c_size_t
    lib.gs_last_error.restype = C.c_char_p
    for name in ("gs_preprocess", "gs_bin_sort", "gs_render_fwd", "gs_loss_l1_dssim", "gs_render_bwd",
                 "gs_adam_step"):
        getattr(lib, name).restype = I32
    return lib


_lib = _load()


def lib():
    return _lib


def _check(status):
    if status != GS_OK:
        raise GsError(status, _lib.gs_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def make_camera(cam) -> GsCamera:
    c = GsCamera()
    c.R[:] = [float(x) for x in np.asarray(cam.R, np.float32).reshape(9)]
    c.t[:] = [float(x) for x in np.asarray(cam.t, np.float32)]
    c.campos[:] = [float(x) for x in np.asarray(cam.campos, np.float32)]
    c.fx, c.fy, c.cx, c.cy = cam.fx, cam.fy, cam.cx, cam.cy
    c.width, c.height = cam.width, cam.height
    c.znear = cam.znear
    c.bg[:] = [float(x) for x in cam.bg]
    return c


class Proj:
    """Device buffers of the projected state (gs_proj) for n Gaussians."""

    def __init__(self, n, device="cuda"):
        self.n = n
        self.splat = torch.empty((max(n, 1), 12), dtype=torch.float32, device=device)
        self.depth = torch.empty(max(n, 1), dtype=torch.float32, device=device)
        self.rect = torch.empty((max(n, 1), 2), dtype=torch.int32, device=device)
        self.tiles = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.order = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.n_visible = torch.empty(1, dtype=torch.int32, device=device)
        self.offs = torch.empty(n + 1, dtype=torch.int32, device=device)
        self.rect_order = torch.empty((max(n, 1), 2), dtype=torch.int32, device=device)
        self.struct = GsProj(self.splat.data_ptr(), self.depth.data_ptr(), self.rect.data_ptr(),
                             self.tiles.data_ptr(), self.order.data_ptr(), self.n_visible.data_ptr(),
                             self.offs.data_ptr(), self.rect_order.data_ptr())


def workspace(which, n=0, pairs=0, W=0, H=0, device="cuda", cfg=None):
    nbytes = int(_lib.gs_workspace_bytes(which, n, pairs, W, H, _cfg(cfg)))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def gs_workspace_bytes(which, n=0, pairs=0, W=0, H=0, cfg=None):
    return int(_lib.gs_workspace_bytes(which, n, pairs, W, H, _cfg(cfg)))


def gs_param_floats(n, sh_degree):
    return int(_lib.gs_param_floats(n, sh_degree))


def _blocked(t, n, sh_degree):
    """Check that a tensor can hold a blocked parameter array for n Gaussians."""
    need = gs_param_floats(n, sh_degree)
    if t is None or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < need:
        raise ValueError(f"expected a contiguous float32 tensor of at least {need} floats (blocked layout)")
    return t


def empty_blocked(n, sh_degree, device="cuda", zero=False):
    """A device tensor of gs_param_floats(n, sh_degree) floats, shaped [groups][P][64]."""
    P = 11 + 3 * (sh_degree + 1) ** 2
    groups = max((n + 63) // 64, 1)
    f = torch.zeros if zero else torch.empty
    return f((groups, P, 64), dtype=torch.float32, device=device)


def to_blocked(planar, sh_degree, out=None, stream=None):
    """[P][n] device tensor -> blocked layout (gs_params_to_blocked)."""
    assert planar.dim() == 2 and planar.is_contiguous() and planar.dtype == torch.float32
    n = planar.shape[1]
    out = empty_blocked(n, sh_degree, planar.device) if out is None else _blocked(out, n, sh_degree)
    _check(_lib.gs_params_to_blocked(_ptr(planar), _ptr(out), n, sh_degree, _stream(stream)))
    return out


def from_blocked(blocked, n, sh_degree, out=None, stream=None):
    """Blocked layout -> [P][n] device tensor (gs_params_from_blocked)."""
    _blocked(blocked, n, sh_degree)
    P = 11 + 3 * (sh_degree + 1) ** 2
    out = torch.empty((P, n), dtype=torch.float32, device=blocked.device) if out is None else out
    assert out.shape == (P, n) and out.is_contiguous()
    _check(_lib.gs_params_from_blocked(_ptr(blocked), _ptr(out), n, sh_degree, _stream(stream)))
    return out


def gs_preprocess(params, sh_degree, cam: GsCamera, proj: Proj, ws, cfg=None, stream=None) -> int:
    """Projection + tile-count scan; returns the pair count (synchronises the stream once).
    params: blocked layout for proj.n Gaussians."""
    n = proj.n
    _blocked(params, n, sh_degree)
    scene = GsScene(n, sh_degree, params.data_ptr() if n else None)
    total = C.c_uint32(0)
    _check(_lib.gs_preprocess(C.byref(scene), C.byref(cam), C.byref(proj.struct), C.byref(total), _ptr(ws),
                              ws.numel(), _cfg(cfg), _stream(stream)))
    return int(total.value)


def gs_bin_sort(proj: Proj, cam: GsCamera, total_pairs, keys, vals, ranges, ws, stream=None):
    cap = keys.numel() if keys is not None else 0
    _check(_lib.gs_bin_sort(C.byref(proj.struct), proj.n, C.byref(cam), total_pairs, _ptr(keys), _ptr(vals), cap,
                            _ptr(ranges), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def gs_render_fwd(proj: Proj, vals, ranges, total_pairs, cam: GsCamera, rgb, T_final, n_contrib, ws, cfg=None,
                  stream=None):
    _check(_lib.gs_render_fwd(C.byref(proj.struct), proj.n, _ptr(vals), _ptr(ranges), total_pairs, C.byref(cam),
                              _ptr(rgb), _ptr(T_final), _ptr(n_contrib), _ptr(ws), ws.numel(), _cfg(cfg),
                              _stream(stream)))


def gs_loss_l1_dssim(img, target, lambda_dssim, loss_out, dL_dimg, ws, stream=None):
    _, H, W = img.shape
    _check(_lib.gs_loss_l1_dssim(_ptr(img), _ptr(target), H, W, float(lambda_dssim), _ptr(loss_out),
                                 _ptr(dL_dimg), _ptr(ws), ws.numel(), _stream(stream)))


def gs_loss_l1_dssim_noalloc(img, target, lambda_dssim, loss_out, dL_dimg, stream=None):
    """gs_loss_l1_dssim without a workspace: the library's static scratch (no allocation)."""
    _, H, W = img.shape
    _check(_lib.gs_loss_l1_dssim_noalloc(_ptr(img), _ptr(target), H, W, float(lambda_dssim), _ptr(loss_out),
                                         _ptr(dL_dimg), _stream(stream)))


def gs_render_bwd(params, sh_degree, proj: Proj, vals, ranges, total_pairs, cam: GsCamera, T_final, n_contrib, dL_dimg,
                  gscreen, gparams, ws, cfg=None, stream=None):
    n = proj.n
    _blocked(params, n, sh_degree)
    _blocked(gparams, n, sh_degree)
    scene = GsScene(n, sh_degree, params.data_ptr() if n else None)
    _check(_lib.gs_render_bwd(C.byref(scene), C.byref(proj.struct), _ptr(vals), _ptr(ranges), total_pairs,
                              C.byref(cam),
                              _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimg), _ptr(gscreen), _ptr(gparams),
                              _ptr(ws), ws.numel(), _cfg(cfg), _stream(stream)))


def gs_render_bwd_weighted(params, sh_degree, proj: Proj, vals, ranges, total_pairs, cam: GsCamera, T_final,
                           n_contrib, dL_dimg, gscreen, gparams, ws, weight, accumulate, cfg=None, stream=None):
    n = proj.n
    _blocked(params, n, sh_degree)
    _blocked(gparams, n, sh_degree)
    scene = GsScene(n, sh_degree, params.data_ptr() if n else None)
    _check(_lib.gs_render_bwd_weighted(C.byref(scene), C.byref(proj.struct), _ptr(vals), _ptr(ranges), total_pairs,
                                       C.byref(cam), _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimg), _ptr(gscreen),
                                       _ptr(gparams), float(weight), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                       _cfg(cfg), _stream(stream)))


def gs_relocate(params, m, v, n, sh_degree, rand, ws, dead_opacity=0.02, donor_opacity=0.4, max_moves=-1,
                stream=None):
    """Moves the dead Gaussians to the largest donors in place; returns the number of moves."""
    for t in (params, m, v):
        _blocked(t, n, sh_degree)
    moves = C.c_int64(0)
    _check(_lib.gs_relocate(_ptr(params), _ptr(m), _ptr(v), n, sh_degree, _ptr(rand), float(dead_opacity),
                            float(donor_opacity), int(max_moves), C.byref(moves), _ptr(ws), ws.numel(),
                            _stream(stream)))
    return int(moves.value)


def gs_camera_grad(params, sh_degree, proj: Proj, cam: GsCamera, gscreen, grad_out, ws, position_only=False,
                   cfg=None, stream=None):
    """grad_out: device float64[6] = (rotation, translation) gradient of the camera pose
    (with position_only, the trainer's position-path terms alone)."""
    n = proj.n
    _blocked(params, n, sh_degree)
    if grad_out.dtype != torch.float64 or grad_out.numel() < 6:
        raise ValueError("grad_out must hold 6 float64 values")
    scene = GsScene(n, sh_degree, params.data_ptr() if n else None)
    _check(_lib.gs_camera_grad(C.byref(scene), C.byref(proj.struct), C.byref(cam), _ptr(gscreen),
                               int(bool(position_only)), _ptr(grad_out), _ptr(ws), ws.numel(), _cfg(cfg),
                               _stream(stream)))


def gs_adam_step(params, grads, m, v, n, sh_degree, lr, beta1, beta2, eps, step, stream=None):
    for t in (params, grads, m, v):
        _blocked(t, n, sh_degree)
    lr_arr = (C.c_float * 5)(*[float(x) for x in lr])
    _check(_lib.gs_adam_step(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), n, sh_degree, lr_arr, float(beta1),
                             float(beta2), float(eps), int(step), _stream(stream)))


def gs_render_bwd_adam(params, sh_degree, proj: Proj, vals, ranges, total_pairs, cam: GsCamera, T_final,
                       n_contrib, dL_dimg, gscreen, m, v, lr, beta1, beta2, eps, step, ws, cfg=None, stream=None):
    for t in (params, m, v):
        _blocked(t, proj.n, sh_degree)
    lr_arr = (C.c_float * 5)(*[float(x) for x in lr])
    _check(_lib.gs_render_bwd_adam(_ptr(params), proj.n, sh_degree, C.byref(proj.struct), _ptr(vals), _ptr(ranges),
                                   total_pairs, C.byref(cam), _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimg),
                                   _ptr(gscreen), _ptr(m), _ptr(v), lr_arr, float(beta1), float(beta2),
                                   float(eps), int(step), _ptr(ws), ws.numel(), _cfg(cfg), _stream(stream)))


def gs_render_bwd_adam_project(params, sh_degree, proj: Proj, vals, ranges, total_pairs, cam: GsCamera, T_final,
                               n_contrib, dL_dimg, gscreen, m, v, lr, beta1, beta2, eps, step, ws,
                               next_cam: GsCamera, next_proj: Proj, pre_ws, densify_stats=None, cfg=None,
                               stream=None) -> int:
    """gs_render_bwd_adam, then the projection of the updated scene for next_cam into
    next_proj (may be proj); returns the next pair count (synchronises once).  With
    densify_stats ([n][2]), this step's observations are added to it."""
    for t in (params, m, v):
        _blocked(t, proj.n, sh_degree)
    assert next_proj.n == proj.n
    lr_arr = (C.c_float * 5)(*[float(x) for x in lr])
    total = C.c_uint32(0)
    _check(_lib.gs_render_bwd_adam_project(
        _ptr(params), proj.n, sh_degree, C.byref(proj.struct), _ptr(vals), _ptr(ranges), total_pairs, C.byref(cam),
        _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimg), _ptr(gscreen), _ptr(m), _ptr(v), lr_arr, float(beta1),
        float(beta2), float(eps), int(step), _ptr(ws), ws.numel(), C.byref(next_cam), C.byref(next_proj.struct),
        C.byref(total), _ptr(pre_ws), pre_ws.numel(), _ptr(densify_stats), _cfg(cfg), _stream(stream)))
    return int(total.value)


def gs_densify_accumulate(proj: Proj, gscreen, stats, stream=None):
    """Adds one step's screen-position gradient lengths and observation counts to stats [n][2]."""
    _check(_lib.gs_densify_accumulate(C.byref(proj.struct), proj.n, _ptr(gscreen), _ptr(stats), _stream(stream)))


def gs_densify(params, m, v, stats, rand, n, sh_degree, grad_threshold, prune_opacity, prune_scale, split_scale,
               ws, reset_opacity=False, opacity_cap=0.01, params_out=None, m_out=None, v_out=None, stats_out=None,
               capacity=0, stream=None):
    """One densification; returns (new count, (kept, cloned, split)).  Without params_out
    only the counts are computed."""
    n_out = C.c_int64(0)
    counts = (C.c_int64 * 3)()
    _check(_lib.gs_densify(_ptr(params), _ptr(m), _ptr(v), _ptr(stats), _ptr(rand), n, sh_degree,
                           float(grad_threshold), float(prune_opacity), float(prune_scale), float(split_scale),
                           1 if reset_opacity else 0, float(opacity_cap), _ptr(params_out), _ptr(m_out),
                           _ptr(v_out), _ptr(stats_out), int(capacity), C.byref(n_out), counts, _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)))
    return int(n_out.value), tuple(int(c) for c in counts)


def gs_loss_charbonnier(img, target, exposure, loss_out, dL_dimg, ws, delta=0.03, dL_dexposure=None, stream=None):
    """Charbonnier loss with exposure (log gain, bias): mean of sqrt(err^2 + delta^2) - delta."""
    _, H, W = img.shape
    _check(_lib.gs_loss_charbonnier(_ptr(img), _ptr(target), H, W, float(delta), _ptr(exposure), _ptr(loss_out),
                                    _ptr(dL_dimg), _ptr(dL_dexposure), _ptr(ws), ws.numel(), _stream(stream)))


def gs_profile_enable(on, only=None):
    """Start (on=True) or stop per-kernel event timing; `only` restricts it to one kernel name."""
    _check(_lib.gs_profile_enable(1 if on else 0, only.encode() if only else None))


def gs_profile_query(max_names=64):
    """{kernel name: (launches, summed milliseconds)} for the launches recorded since enabling."""
    names = C.create_string_buffer(64 * max_names)
    launches = (C.c_int64 * max_names)()
    total_ms = (C.c_double * max_names)()
    k = _lib.gs_profile_query(max_names, C.cast(names, C.c_void_p), C.cast(launches, C.c_void_p),
                              C.cast(total_ms, C.c_void_p))
    _check(min(k, 0))
    return {names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode(): (int(launches[i]), float(total_ms[i]))
            for i in range(k)}


def gs_last_error():
    return _lib.gs_last_error().decode()
