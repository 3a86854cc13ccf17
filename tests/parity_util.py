"""Helpers for the GPU-vs-oracle parity tests: run the HIP path through the C ABI
and pull every stage's output back to numpy; tolerance checks."""
from __future__ import annotations

import numpy as np

# A blend decision (skip below 1/255, stop below 1e-4, cap at 0.99) whose
# conditioned distance to its threshold is within the reach of fp32 rounding may
# come out the other way on the GPU.  The oracle's flip_risk takes each such
# decision the other way and reports how far that moves every pixel and every
# screen partial; the checks below add that amount to their tolerance.
PIXEL_ATOL = 1e-5          # rendered pixels, absolute
GRAD_RTOL = 1e-3           # parameter gradients, relative
CALM = 0.1                 # parameter gradients are checked where flips move no screen partial
                           # by more than this fraction of its tolerance
SSIM_REACH = 10            # a pixel's loss gradient depends on pixels up to this far away


def gpu_forward(params_np, deg, cam, cfg=None):
    """A Pipeline over the scene (cfg: its gs_config, None for the defaults) after one
    forward for cam."""
    import torch
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    params = torch.from_numpy(np.ascontiguousarray(params_np, np.float32)).cuda()
    pl = Pipeline(params, deg, cam.width, cam.height, cfg=cfg)
    c = gs.make_camera(cam)
    pl.forward(c)
    torch.cuda.synchronize()
    return pl, c


def tile_of_key(keys64):
    """Tile ids of the oracle's 64-bit sort keys (tile << 32 | depth bits)."""
    return (np.asarray(keys64, np.uint64) >> np.uint64(32)).astype(np.uint32)


def proj_to_numpy(pl):
    n = pl.n
    splat = pl.proj.splat[:n].cpu().numpy()
    rect = pl.proj.rect[:n].cpu().numpy().view(np.uint32)
    out = dict(uv=splat[:, 0:2].T.copy(), conic=splat[:, 2:5].T.copy(), opac=splat[:, 5].copy(),
               rgb=splat[:, 6:9].T.copy(), box=splat[:, 9:11].T.copy(), cull_t=splat[:, 11].copy(), depth=pl.proj.depth[:n].cpu().numpy(),
               tiles=pl.proj.tiles[:n].cpu().numpy().view(np.uint32),
               offs=pl.proj.offs.cpu().numpy().view(np.uint32),
               order=pl.proj.order[:n].cpu().numpy().view(np.uint32),
               rect_order=pl.proj.rect_order[:n].cpu().numpy().view(np.uint32),
               n_visible=int(pl.proj.n_visible.cpu().numpy().view(np.uint32)[0]))
    r = np.zeros((4, n), np.int64)
    r[0] = rect[:, 0] & 0xFFFF
    r[1] = rect[:, 0] >> 16
    r[2] = rect[:, 1] & 0xFFFF
    r[3] = rect[:, 1] >> 16
    out["rect"] = r
    return out


def sorted_to_numpy(pl):
    P = pl.pairs
    keys = pl.keys[:P].cpu().numpy().view(np.uint32)    # tile id of each sorted pair
    vals = pl.vals[:P].cpu().numpy().view(np.uint32)
    ranges = pl.ranges.cpu().numpy().view(np.uint32)
    return keys, vals, ranges


def render_to_numpy(pl):
    return dict(rgb=pl.rgb.cpu().numpy(), T=pl.T.cpu().numpy(), n_contrib=pl.nc.cpu().numpy().view(np.uint32))


def check_preprocess(gpu, ora):
    vis = ora["tiles"] > 0
    np.testing.assert_array_equal(gpu["tiles"], ora["tiles"])
    np.testing.assert_array_equal(gpu["rect"][:, vis], ora["rect"][:, vis])
    np.testing.assert_array_equal(gpu["depth"][vis].view(np.uint32), ora["depth"][vis].view(np.uint32))
    np.testing.assert_array_equal(gpu["uv"][:, vis], ora["uv"][:, vis])
    np.testing.assert_array_equal(gpu["conic"][:, vis], ora["conic"][:, vis])
    np.testing.assert_allclose(gpu["opac"][vis], ora["opac"][vis], rtol=2e-7, atol=0)
    np.testing.assert_allclose(gpu["rgb"][:, vis], ora["rgb"][:, vis], rtol=1e-6, atol=1e-6)
    check_blend_box(gpu, vis)
    # depth order of the visible Gaussians: by the depth's bits, then by id
    ids = np.nonzero(vis)[0]
    order = ids[np.lexsort((ids, ora["depth"][ids].view(np.uint32)))]
    assert gpu["n_visible"] == len(order)
    np.testing.assert_array_equal(gpu["order"][:len(order)], order)
    # the rectangles in that order, packed as in rect (x0 | y0 << 16, x1 | y1 << 16)
    ro = gpu["rect_order"][:len(order)].astype(np.int64)
    np.testing.assert_array_equal(np.stack([ro[:, 0] & 0xFFFF, ro[:, 0] >> 16, ro[:, 1] & 0xFFFF, ro[:, 1] >> 16]),
                                  ora["rect"][:, order])
    # the pair offsets in depth order: the first n_visible + 1 entries (the rest unspecified)
    counts = ora["tiles"][order].astype(np.int64)
    expect_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    np.testing.assert_array_equal(gpu["offs"][:len(order) + 1], expect_offs)


def check_blend_box(gpu, vis):
    """The box (u +- hx, v +- hy) must contain every point where o exp(-e) >= 1/255 for
    e = (A dx^2 + C dy^2) / 2 + B dx dy with the record's own conic: the ellipse's
    half-widths sqrt(2 t C / (A C - B^2)), sqrt(2 t A / (A C - B^2)), t = ln(255 o);
    the record's exponent bound tm may not be below t."""
    A, B, C = (gpu["conic"][k][vis].astype(np.float64) for k in range(3))
    o = gpu["opac"][vis].astype(np.float64)
    hx, hy = gpu["box"][0][vis], gpu["box"][1][vis]
    t = np.log(255.0 * o)
    none = t <= -1e-3
    assert np.all(hx[none] < 0) and np.all(hy[none] < 0)
    det = A * C - B * B
    ok = ~none & (det > 0)
    need_x = np.sqrt(2 * np.maximum(t[ok], 0) * C[ok] / det[ok])
    need_y = np.sqrt(2 * np.maximum(t[ok], 0) * A[ok] / det[ok])
    assert np.all(hx[ok] >= need_x) and np.all(hy[ok] >= need_y)
    assert np.all(np.isinf(hx[~none & ~(det > 0)]))
    # the exponent bound the blend's per-quadrant ellipse test uses: at least t where
    # the box is finite, infinite with it
    tm = gpu["cull_t"][vis]
    fin = np.isfinite(hx)
    assert np.all(tm[~none & fin] >= t[~none & fin]) and np.all(np.isinf(tm[~none & ~fin]))


def flipped_pixels(risk):
    """Pixels that some near-threshold decision, taken the other way, changes."""
    return (risk["px"][0] > 0) | (risk["px"][1] > 0) | (risk["nc_lo"] != risk["nc_hi"])


# Ceilings on what may pass only through a threshold decision taken the other way (or,
# for screen partials, through the rounding slack): shares of all pixels, of all screen
# partials and of the Gaussians with a partial.  The checks print the shares; on the
# full-size workloads (100k to 6M Gaussians) they measured at most 8.7e-6 of the pixels
# equal to a flipped outcome, none on the summed bound, 3.3e-7 of the partials beyond the
# plain bar and 3.2e-2 of the Gaussians (the 3M-Gaussian stress scene; 1.3e-3 elsewhere)
# left out; the ceilings leave roughly a factor of ten (the last: of 1.5).
MAX_SHARE_PIXELS_FLIPPED = 1e-4       # pixels equal to a flipped outcome rather than the oracle's
MAX_SHARE_PIXELS_ADDITIVE = 1e-5      # pixels with several near decisions, held to the summed bound
MAX_SHARE_PARTIALS_SLACK = 1e-5       # screen partials beyond the plain 1e-3 bar
MAX_SHARE_NOT_CALM = 0.05             # Gaussians with a partial left out of the plain parameter bar


def observed_risk(oracle, ref, cam, gpu_render, dLdI):
    """The oracle's flip risk with the flips the GPU's own render rules out left out of
    the screen-partial risk (a flip whose effect on a pixel would show in the render,
    at a pixel where the GPU matches the oracle's unflipped walk)."""
    return oracle.flip_risk(ref["pre"], ref["vals"], ref["ranges"], cam, np.asarray(dLdI, np.float32),
                            observed=gpu_render, obs_atol=PIXEL_ATOL)


def check_render(gpu, ora, risk):
    """Pixel by pixel, within PIXEL_ATOL (colour and T) and with the same n_contrib:
    * a pixel with no decision within fp32 reach of its threshold: the oracle's render;
    * one such decision: the oracle's render or the render with that decision taken the
      other way (either / or, not a widened bound);
    * several: within PIXEL_ATOL plus the sum of what each flip changes, n_contrib in the
      range the flips produce.
    Returns counts: pixels with any near decision, equal only to the flipped outcome,
    held to the summed bound."""
    rgb, T, nc = gpu["rgb"], gpu["T"], gpu["n_contrib"]
    d0 = np.abs(rgb - ora["rgb"]).max(axis=0)
    t0 = np.abs(T - ora["T"])
    ok0 = (d0 <= PIXEL_ATOL) & (t0 <= PIXEL_ATOL) & (nc == ora["n_contrib"])
    nfl = risk["nflip"]
    d1 = np.abs(rgb - risk["alt_rgb"]).max(axis=0)
    t1 = np.abs(T - risk["alt_T"])
    ok1 = (nfl == 1) & (d1 <= PIXEL_ATOL) & (t1 <= PIXEL_ATOL) & (nc == risk["alt_nc"])
    okm = (nfl >= 2) & (d0 <= PIXEL_ATOL + risk["px"][0]) & (t0 <= PIXEL_ATOL + risk["px"][1]) & \
        (risk["nc_lo"] <= nc) & (nc <= risk["nc_hi"])
    bad = ~(ok0 | ok1 | okm)
    assert not bad.any(), (f"{int(bad.sum())} pixels off (near decisions there: "
                           f"{np.bincount(np.minimum(nfl[bad], 3).astype(np.int64), minlength=4).tolist()}), "
                           f"max colour error {d0[bad].max()}")
    npx = nfl.size
    st = dict(near=int((nfl > 0).sum()), flipped=int((ok1 & ~ok0).sum()), additive=int((okm & ~ok0 & ~ok1).sum()))
    print(f"  pixels: {npx}, with a near decision {st['near']}, equal to a flipped outcome {st['flipped']} "
          f"({st['flipped'] / npx:.2e}), on the summed bound {st['additive']} ({st['additive'] / npx:.2e})",
          flush=True)
    assert st["flipped"] + st["additive"] <= MAX_SHARE_PIXELS_FLIPPED * npx
    assert st["additive"] <= MAX_SHARE_PIXELS_ADDITIVE * npx
    return st


def check_loss(loss, dLdI, ref, target):
    """Loss terms and the image gradient of a full step.  With no flippable pixel the
    loss (total, L1, SSIM) is held to 2e-5 relative; otherwise L1 to that plus the
    mean colour risk (L1 moves by at most |change| per channel).  dL/dimage: within
    1e-4 of its largest element on the pixels no flip can reach through the SSIM
    window and whose L1 sign is decided (|image - target| above what the pixel
    may move).  Returns the number of image-gradient elements checked."""
    from scipy.ndimage import maximum_filter
    risk = ref["risk"]
    flipped = flipped_pixels(risk)
    if not flipped.any():
        np.testing.assert_allclose(loss, ref["loss"], rtol=2e-5)
    else:
        H, W = flipped.shape
        tol = 2e-5 * abs(ref["loss"][1]) + float(risk["px"][0].astype(np.float64).sum()) / (H * W)
        assert abs(loss[1] - ref["loss"][1]) <= tol, f"L1 {loss[1]} vs {ref['loss'][1]} (tol {tol})"
    reach = maximum_filter(flipped, size=2 * SSIM_REACH + 1, mode="constant")
    decided = np.abs(ref["fwd"]["rgb"] - target) > PIXEL_ATOL + risk["px"][0]
    keep = decided & ~reach
    scale = np.abs(ref["dLdI"]).max()
    err = np.abs(dLdI - ref["dLdI"])[keep]
    assert err.max(initial=0.0) <= 1e-4 * scale, f"dL/dimage off by {err.max()} (scale {scale})"
    return int(keep.sum())


LOSS_MAG_RTOL = 1e-4     # image gradient: per element, of the magnitude of the SSIM terms it sums


def check_loss_everywhere(loss, dLdI, ref_loss, ref_dLdI, mag):
    """The loss of one image pair, the GPU's against the fp64 oracle's on the same images:
    total, L1 and SSIM within 2e-5 relative, and every element of dL/dimage within
    2e-6 of itself (the L1 part: the same sign decision on both sides) plus LOSS_MAG_RTOL
    of the summed magnitude of the SSIM terms behind it (the scale of what fp32 sums
    in another order can change).  Returns (elements, worst error over its bound)."""
    np.testing.assert_allclose(loss, ref_loss, rtol=2e-5)
    g = np.asarray(ref_dLdI, np.float64)
    d = np.abs(np.asarray(dLdI, np.float64) - g)
    tol = 2e-6 * np.abs(g) + LOSS_MAG_RTOL * mag
    bad = d > tol
    assert not bad.any(), f"dL/dimage: {int(bad.sum())} of {g.size} elements off, max excess {(d - tol).max()}"
    worst = float((d / np.maximum(tol, 1e-300)).max())
    print(f"  image gradient: all {g.size} elements checked, worst error {worst:.3f} of its bound, "
          f"{d.max() / np.abs(g).max():.2e} of the largest element", flush=True)
    return g.size, worst


def grad_groups(deg):
    P = 11 + 3 * (deg + 1) ** 2
    groups = {"mean": slice(0, 3), "logscale": slice(3, 6), "quat": slice(6, 10), "logit": slice(10, 11),
              "dc": slice(11, 14)}
    if P > 14:
        groups["sh"] = slice(14, P)
    return groups


def check_grad(g_gpu, g_ref, mask=None, rtol=GRAD_RTOL, name="", risk=None):
    """Per element |d| <= rtol |ref| + rtol rms(ref) + risk, and ||d|| <= rtol ||ref|| + ||risk||.
    Returns the number of elements beyond the plain bar (those passing through risk)."""
    if mask is None:
        mask = np.ones(g_ref.shape[-1], bool)
    a = g_gpu[..., mask].astype(np.float64)
    b = g_ref[..., mask].astype(np.float64)
    r = np.zeros_like(b) if risk is None else risk[..., mask].astype(np.float64)
    if b.size == 0:
        return 0
    rms = np.sqrt((b * b).mean())
    d = np.abs(a - b)
    plain = rtol * np.abs(b) + rtol * rms
    bad = d > plain + r
    assert not bad.any(), f"{name}: {int(bad.sum())} of {b.size} elements off, max {d.max()} (rms {rms})"
    nb = np.linalg.norm(b)
    if nb > 0:
        assert np.linalg.norm(a - b) <= rtol * nb + np.linalg.norm(r), \
            f"{name}: relative norm {np.linalg.norm(a - b) / nb}"
    return int((d > plain).sum())


SCREEN = ["u", "v", "A", "B", "C", "opacity", "r", "g", "b"]


def check_screen_grads(gscreen, ref_gscreen, grisk, slack=None, planes=range(9)):
    """The nine screen partials of every Gaussian, to GRAD_RTOL plus their flip risk and,
    when given, the oracle's rounding slack (atomic reordering and per-term rounding).
    Prints, and holds below MAX_SHARE_PARTIALS_SLACK, the share of partials beyond the
    plain bar."""
    beyond = total = 0
    for k in planes:
        r = grisk[k].astype(np.float64) + (0.0 if slack is None else slack[k])
        beyond += check_grad(gscreen[k], ref_gscreen[k], name=SCREEN[k], risk=r)
        total += ref_gscreen[k].size
    print(f"  screen partials: {total}, beyond the plain 1e-3 bar (within flip risk and rounding slack) {beyond} "
          f"({beyond / max(total, 1):.2e})", flush=True)
    assert beyond <= MAX_SHARE_PARTIALS_SLACK * total
    return beyond


def calm(grisk, ref_gscreen, rtol=GRAD_RTOL):
    """Gaussians whose screen partials no flip moves by more than CALM of their tolerance;
    their parameter gradients are held to the plain tolerance.  Prints, and holds below
    MAX_SHARE_NOT_CALM, the share of the visible Gaussians (those with a partial) left out."""
    g = ref_gscreen.astype(np.float64)
    rms = np.sqrt((g * g).mean(axis=1, keepdims=True))
    keep = np.all(grisk <= CALM * rtol * (np.abs(g) + rms), axis=0)
    seen = np.any(g != 0, axis=0)
    out = int((~keep).sum())
    print(f"  Gaussians with a partial: {int(seen.sum())}, left out of the parameter bar (not calm) {out} "
          f"({out / max(int(seen.sum()), 1):.2e})", flush=True)
    assert out <= MAX_SHARE_NOT_CALM * max(int(seen.sum()), 1)
    return keep


def check_param_grads(g_gpu, ref, oracle, params, deg, cam, keep, rtol=GRAD_RTOL):
    """Parameter gradients of the calm Gaussians, group by group: GRAD_RTOL of the element
    plus GRAD_RTOL of the group's rms, and, for the Gaussians where that is not enough,
    the screen-level flip risk and rounding slack carried through the chain by the oracle
    (the chain is linear in the screen partials, so each plane's bound is chained on its
    own and the magnitudes added)."""
    bound_screen = ref["risk"]["g"].astype(np.float64) + ref["slack"]
    for name, sl in grad_groups(deg).items():
        a = g_gpu[sl][:, keep].astype(np.float64)
        b = ref["gparams"][sl][:, keep].astype(np.float64)
        if b.size == 0:
            continue
        rms = np.sqrt((b * b).mean())
        d = np.abs(a - b)
        tol = rtol * np.abs(b) + rtol * rms
        bad_cols = np.nonzero((d > tol).any(axis=0))[0]
        if bad_cols.size:
            idx = np.nonzero(keep)[0][bad_cols]
            sub = np.ascontiguousarray(params[:, idx])
            extra = np.zeros((params.shape[0], idx.size))
            for k in range(9):
                gs_k = np.zeros((9, idx.size), np.float32)
                gs_k[k] = bound_screen[k, idx]
                extra += np.abs(oracle.preprocess_bwd(sub, deg, cam, gs_k).astype(np.float64))
            tol[:, bad_cols] += extra[sl]
        bad = d > tol
        assert not bad.any(), (f"{name}: {int(bad.sum())} of {b.size} elements off, max excess "
                               f"{(d - tol).max()} (rms {rms})")
        nb = np.linalg.norm(b)
        if nb > 0:
            assert np.linalg.norm(d) <= rtol * nb + np.linalg.norm(tol - rtol * np.abs(b) - rtol * rms), \
                f"{name}: relative norm {np.linalg.norm(d) / nb}"
