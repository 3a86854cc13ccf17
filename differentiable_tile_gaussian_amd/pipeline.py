"""One training step for one camera through the C ABI, with the device buffers
it needs kept between calls (grown only when a larger pair count appears).

torch allocates memory and provides the stream; every stage runs in libgs.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import gs

DEFAULT_LR = (1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3)   # means, log-scales, quaternion, opacity, colour


def position_lr_decay(lr_final, max_steps, lr=DEFAULT_LR):
    """A schedule for Pipeline(lr_schedule=...): the means' rate decays from lr[0] to
    lr_final over max_steps steps, log-linearly (then stays at lr_final); the other
    groups keep their constant rates.  One choice of decay among many: the pages say only
    that position has its own decaying schedule."""
    import math
    l0, l1 = math.log(lr[0]), math.log(lr_final)

    def rates(t):
        f = min(max((t - 1) / max(max_steps - 1, 1), 0.0), 1.0)
        return (math.exp(l0 + f * (l1 - l0)),) + tuple(lr[1:])
    return rates


def blocked_to_planar(blocked: np.ndarray, n: int) -> np.ndarray:
    """Host copy of a blocked parameter array ([groups][P][64]: parameter p of Gaussian i at
    [i // 64][p][i % 64]) as [P][n]."""
    groups, P, w = blocked.shape
    assert w == 64 and groups * 64 >= n
    return np.ascontiguousarray(blocked.transpose(1, 0, 2).reshape(P, groups * 64)[:, :n])


class TrainingSchedule:
    """When the trainer's discrete operations happen, by Adam step t >= 1 (host logic; the
    operations themselves are library calls).

    Density control ([GST] density-control slide, its explanation of the usual settings:
    densification starts after step 500, repeats every 100 steps and stops at 15000, and
    opacity is reset every 3000 steps, capped at 0.01), read as: densify after the steps
    t with start < t < stop and t % every == 0; reset opacity after the steps t with
    t < stop and t % reset_every == 0 (resets belong to the densification phase); a reset
    at a densification step is made by that densification's gs_densify call.

    SH degree ramp ([GSG] "Spherical harmonics": one more band about every 1000 steps),
    read as: step t sums the bands up to min(scene degree, t // sh_every)."""

    def __init__(self, start=500, every=100, stop=15000, reset_every=3000, opacity_cap=0.01, sh_every=1000):
        assert every > 0 and reset_every > 0 and sh_every > 0 and 0.0 < opacity_cap < 1.0
        self.start, self.every, self.stop, self.reset_every = start, every, stop, reset_every
        self.opacity_cap, self.sh_every = opacity_cap, sh_every

    def densify_after(self, t):
        return self.start < t < self.stop and t % self.every == 0

    def reset_after(self, t):
        return t < self.stop and t % self.reset_every == 0

    def sh_degree(self, t, scene_degree):
        return min(scene_degree, t // self.sh_every)


class Pipeline:
    def __init__(self, params: torch.Tensor, sh_degree: int, width: int, height: int, lam: float = 0.2,
                 lr=DEFAULT_LR, betas=(0.9, 0.999), eps=1e-8, cfg: gs.GsConfig = None, lr_schedule=None):
        """params: [P][n] float32 device tensor (plane-major); it is copied into the
        library's blocked layout, in which params, grads, m and v are then kept.
        cfg: the settings every call of this pipeline passes (gs_config; None: defaults).
        lr_schedule: None for the constant rates `lr`, or a function of the Adam step
        t >= 1 returning the five group rates (means, log-scales, quaternion, opacity,
        colour) that step's update uses; the pages give the means their own decaying
        rate ([DR] "From a pixel error back to a quaternion") but no formula, so the
        schedule is the caller's (see position_lr_decay)."""
        assert params.is_cuda and params.dtype == torch.float32 and params.is_contiguous()
        self.cfg = cfg if cfg is not None else gs.GsConfig()
        self.lr_schedule = lr_schedule
        self.deg = sh_degree
        self.n = params.shape[1]
        self.params = gs.to_blocked(params, sh_degree)
        self.W, self.H = width, height
        self.lam, self.lr, self.betas, self.eps = lam, lr, betas, eps
        dev = params.device
        self.proj = gs.Proj(self.n, dev)
        self.ws_pre = gs.workspace(gs.GS_WS_PREPROCESS, n=self.n, device=dev)
        tx, ty = (width + 15) // 16, (height + 15) // 16
        self.num_tiles = tx * ty
        self.ranges = torch.empty((2, self.num_tiles), dtype=torch.int32, device=dev)
        self.keys = torch.empty(0, dtype=torch.int32, device=dev)
        self.vals = torch.empty(0, dtype=torch.int32, device=dev)
        self.ws_sort = torch.empty(0, dtype=torch.uint8, device=dev)
        self.rgb = torch.empty((3, height, width), dtype=torch.float32, device=dev)
        self.T = torch.empty((height, width), dtype=torch.float32, device=dev)
        self.nc = torch.empty((height, width), dtype=torch.int32, device=dev)
        self.ws_loss = gs.workspace(gs.GS_WS_LOSS, W=width, H=height, device=dev)
        self.ws_render = torch.empty(0, dtype=torch.uint8, device=dev)
        self.loss = torch.zeros(3, dtype=torch.float32, device=dev)
        self.dLdI = torch.empty((3, height, width), dtype=torch.float32, device=dev)
        self.gscreen = torch.empty((max(self.n, 1), 9), dtype=torch.float32, device=dev)
        self.grads = gs.empty_blocked(self.n, sh_degree, dev, zero=True)
        self.m = gs.empty_blocked(self.n, sh_degree, dev, zero=True)
        self.v = gs.empty_blocked(self.n, sh_degree, dev, zero=True)
        self.t = 0
        self.pairs = 0
        self.projected_for = None   # set by a fused update that projected for the next step's camera
        self.dstats = None          # [n][2] density statistics, once enable_density_stats() is called

    def planar(self, blocked: torch.Tensor) -> torch.Tensor:
        """[P][n] copy of one of the blocked arrays (params, grads, m, v)."""
        return gs.from_blocked(blocked, self.n, self.deg)

    def set_planar(self, blocked: torch.Tensor, planar: torch.Tensor):
        """Overwrite one of the blocked arrays from a [P][n] tensor."""
        gs.to_blocked(planar.to(blocked.device).contiguous(), self.deg, out=blocked)
        self.projected_for = None

    def _reserve(self, pairs):
        if self.keys.numel() < pairs:
            cap = int(pairs * 1.25) + 1024
            self.keys = torch.empty(cap, dtype=torch.int32, device=self.params.device)
            self.vals = torch.empty(cap, dtype=torch.int32, device=self.params.device)
        need = gs.gs_workspace_bytes(gs.GS_WS_BIN_SORT, self.n, pairs, self.W, self.H)
        if self.ws_sort.numel() < need:
            self.ws_sort = torch.empty(int(need * 1.25) + 4096, dtype=torch.uint8, device=self.params.device)
        need = gs.gs_workspace_bytes(gs.GS_WS_RENDER, self.n, pairs, self.W, self.H, self.cfg)
        if self.ws_render.numel() < need:
            self.ws_render = torch.empty(int(need * 1.25) + 4096, dtype=torch.uint8, device=self.params.device)

    def rates(self, t):
        """The five group learning rates of Adam step t (t >= 1)."""
        lr = self.lr if self.lr_schedule is None else self.lr_schedule(t)
        lr = tuple(float(x) for x in lr)
        assert len(lr) == 5
        return lr

    def forward(self, cam: gs.GsCamera):
        if self.projected_for is not cam:
            self.pairs = gs.gs_preprocess(self.params, self.deg, cam, self.proj, self.ws_pre, cfg=self.cfg)
        self.projected_for = None
        self._reserve(self.pairs)
        gs.gs_bin_sort(self.proj, cam, self.pairs, self.keys, self.vals, self.ranges, self.ws_sort)
        gs.gs_render_fwd(self.proj, self.vals, self.ranges, self.pairs, cam, self.rgb, self.T, self.nc,
                         self.ws_render, cfg=self.cfg)
        return self.rgb

    def backward(self, cam: gs.GsCamera, target: torch.Tensor):
        gs.gs_loss_l1_dssim(self.rgb, target, self.lam, self.loss, self.dLdI, self.ws_loss)
        gs.gs_render_bwd(self.params, self.deg, self.proj, self.vals, self.ranges, self.pairs, cam, self.T, self.nc,
                         self.dLdI, self.gscreen, self.grads, self.ws_render, cfg=self.cfg)

    def adam(self):
        self.t += 1
        gs.gs_adam_step(self.params, self.grads, self.m, self.v, self.n, self.deg, self.rates(self.t), self.betas[0],
                        self.betas[1], self.eps, self.t)

    def backward_adam(self, cam: gs.GsCamera, target: torch.Tensor, next_cam: gs.GsCamera = None):
        """Loss, backward and Adam with the chain and Adam fused (no gradient written).
        With next_cam, the update also projects the scene for next_cam, and the next
        forward(next_cam) (the same camera object) uses that projection."""
        gs.gs_loss_l1_dssim(self.rgb, target, self.lam, self.loss, self.dLdI, self.ws_loss)
        self.t += 1
        if next_cam is None:
            gs.gs_render_bwd_adam(self.params, self.deg, self.proj, self.vals, self.ranges, self.pairs, cam, self.T,
                                  self.nc, self.dLdI, self.gscreen, self.m, self.v, self.rates(self.t), self.betas[0],
                                  self.betas[1], self.eps, self.t, self.ws_render, cfg=self.cfg)
            return
        self.pairs = gs.gs_render_bwd_adam_project(self.params, self.deg, self.proj, self.vals, self.ranges,
                                                   self.pairs, cam, self.T, self.nc, self.dLdI, self.gscreen, self.m,
                                                   self.v, self.rates(self.t), self.betas[0], self.betas[1], self.eps,
                                                   self.t, self.ws_render, next_cam, self.proj, self.ws_pre,
                                                   self.dstats, cfg=self.cfg)
        self.projected_for = next_cam

    def step(self, cam: gs.GsCamera, target: torch.Tensor, adam: bool = True, fused: bool = True,
             next_cam: gs.GsCamera = None):
        """One training step; with next_cam (fused Adam only) the update also projects
        the scene for the camera of the following step.  With density statistics enabled,
        the step's observations are added to them (from this step's projection and
        screen gradients, before any projection for the next camera replaces them)."""
        self.forward(cam)
        if adam and fused:
            self.backward_adam(cam, target, next_cam)   # accumulates the statistics when projecting
            if self.dstats is not None and next_cam is None:
                gs.gs_densify_accumulate(self.proj, self.gscreen, self.dstats)
            return self.loss
        self.backward(cam, target)
        if self.dstats is not None:
            gs.gs_densify_accumulate(self.proj, self.gscreen, self.dstats)
        if adam:
            self.adam()
        return self.loss

    def step_views(self, cams, targets):
        """One training step over several views: each view is rendered and differentiated
        in turn, its parameter gradients added into one buffer with weight 1/B (the mean
        over the B views), then one Adam update.  Returns the losses of the views
        ([B][3]: total, L1, SSIM).  With density statistics enabled, every view's
        observations are added to them."""
        B = len(cams)
        assert B == len(targets) and B > 0
        losses = torch.empty((B, 3), dtype=torch.float32, device=self.params.device)
        for k, (cam, target) in enumerate(zip(cams, targets)):
            self.forward(cam)
            gs.gs_loss_l1_dssim(self.rgb, target, self.lam, losses[k], self.dLdI, self.ws_loss)
            gs.gs_render_bwd_weighted(self.params, self.deg, self.proj, self.vals, self.ranges, self.pairs, cam, self.T,
                                      self.nc, self.dLdI, self.gscreen, self.grads, self.ws_render, 1.0 / B, k > 0,
                                      cfg=self.cfg)
            if self.dstats is not None:
                gs.gs_densify_accumulate(self.proj, self.gscreen, self.dstats)
        self.adam()
        return losses

    # ------------------------------------------------------------ density control
    def enable_density_stats(self):
        """Start accumulating each step's screen-position gradient lengths and observation
        counts (zeroed)."""
        self.dstats = torch.zeros((max(self.n, 1), 2), dtype=torch.float32, device=self.params.device)

    def densify(self, grad_threshold, prune_opacity, prune_scale, split_scale, reset_opacity=False,
                opacity_cap=0.01, generator=None):
        """One densification (gs_densify): the population, its Adam moments and the
        statistics are replaced by arrays of the new size.  Split children are sampled
        with standard normals drawn on the device from `generator`.  Returns the counts
        (kept, cloned, split)."""
        dev = self.params.device
        if self.dstats is None:
            self.enable_density_stats()
        rand = torch.randn((max(self.n, 1), 2, 3), dtype=torch.float32, device=dev, generator=generator)
        ws = gs.workspace(gs.GS_WS_DENSIFY, n=self.n, device=dev)
        args = (self.params, self.m, self.v, self.dstats, rand, self.n, self.deg, grad_threshold, prune_opacity,
                prune_scale, split_scale, ws)
        n_new, _ = gs.gs_densify(*args, reset_opacity=reset_opacity, opacity_cap=opacity_cap)
        params = gs.empty_blocked(n_new, self.deg, dev, zero=True)
        m = gs.empty_blocked(n_new, self.deg, dev, zero=True)
        v = gs.empty_blocked(n_new, self.deg, dev, zero=True)
        stats = torch.zeros((max(n_new, 1), 2), dtype=torch.float32, device=dev)
        n_chk, counts = gs.gs_densify(*args, reset_opacity=reset_opacity, opacity_cap=opacity_cap, params_out=params,
                                      m_out=m, v_out=v, stats_out=stats, capacity=n_new)
        assert n_chk == n_new
        self.params, self.m, self.v, self.dstats = params, m, v, stats
        self._resize(n_new)
        return counts

    def after_step(self, sched: TrainingSchedule, grad_threshold, prune_opacity, prune_scale, split_scale,
                   generator=None):
        """What `sched` puts after the Adam step just made (step self.t): a densification
        (with the opacity reset if one also falls there), or the reset alone (a gs_densify
        that prunes, clones and splits nothing; like every densification it also zeroes the
        statistics); then the active SH degree of the next step.  Returns the counts
        (kept, cloned, split) of a densification, else None."""
        t = self.t
        counts = None
        reset = sched.reset_after(t)
        if sched.densify_after(t):
            counts = self.densify(grad_threshold, prune_opacity, prune_scale, split_scale, reset_opacity=reset,
                                  opacity_cap=sched.opacity_cap, generator=generator)
        elif reset:
            self.densify(float("inf"), 0.0, float("inf"), 1.0, reset_opacity=True, opacity_cap=sched.opacity_cap,
                         generator=generator)
        deg = sched.sh_degree(t + 1, self.deg)
        if deg != self.cfg.active_sh_degree:   # a new settings object: the caller's is not changed
            c = self.cfg
            self.cfg = gs.GsConfig(c.grad_sums, deg, c.mip_compensation, c.split_first, c.split_chunk)
            self.projected_for = None   # a projection made for the next camera used the old degree
        return counts

    # ------------------------------------------------------------ checkpoint / resume
    def checkpoint_state(self) -> dict:
        """The training state as host arrays: the Gaussian count, SH degree, Adam step, the
        parameters and both Adam moments in the blocked layout ([groups][P][64]), the
        density statistics (an empty array when not kept), and the settings (image size,
        loss weight, rates, betas, eps, the gs_config fields).  A learning-rate schedule
        is code, not state: pass it again when resuming."""
        c = self.cfg
        return {
            "n": np.int64(self.n), "sh_degree": np.int64(self.deg), "t": np.int64(self.t),
            "size": np.array([self.W, self.H], np.int64), "lam": np.float64(self.lam),
            "lr": np.array(self.lr, np.float64), "betas": np.array(self.betas, np.float64),
            "eps": np.float64(self.eps),
            "cfg": np.array([c.grad_sums, c.active_sh_degree, c.mip_compensation, c.split_first, c.split_chunk],
                            np.int64),
            "params": self.params.cpu().numpy(), "m": self.m.cpu().numpy(), "v": self.v.cpu().numpy(),
            "dstats": (self.dstats.cpu().numpy() if self.dstats is not None else np.zeros((0, 2), np.float32)),
        }

    def save_checkpoint(self, path):
        """checkpoint_state() to an uncompressed .npz file (plain arrays, no pickled objects)."""
        np.savez(path, **self.checkpoint_state())

    @classmethod
    def from_checkpoint(cls, path, device="cuda", lr_schedule=None) -> "Pipeline":
        """A pipeline in the state save_checkpoint wrote: the next step is Adam step t + 1 on
        the same parameters and moments (the next camera is projected again)."""
        with np.load(path) as z:
            st = {k: z[k] for k in z.files}
        n, deg = int(st["n"]), int(st["sh_degree"])
        P = 11 + 3 * (deg + 1) ** 2
        groups = max((n + 63) // 64, 1)
        for k in ("params", "m", "v"):
            assert st[k].shape == (groups, P, 64) and st[k].dtype == np.float32, k
        planar = blocked_to_planar(st["params"], n)
        cfg = gs.GsConfig(*(int(x) for x in st["cfg"]))
        W, H = (int(x) for x in st["size"])
        pl = cls(torch.from_numpy(planar).to(device), deg, W, H, lam=float(st["lam"]),
                 lr=tuple(float(x) for x in st["lr"]), betas=tuple(float(x) for x in st["betas"]),
                 eps=float(st["eps"]), cfg=cfg, lr_schedule=lr_schedule)
        pl.m = torch.from_numpy(st["m"]).to(device)
        pl.v = torch.from_numpy(st["v"]).to(device)
        pl.t = int(st["t"])
        if st["dstats"].shape[0] > 0:
            pl.dstats = torch.from_numpy(st["dstats"]).to(device)
        return pl

    def _resize(self, n):
        """Buffers sized by the Gaussian count, after the population changed."""
        dev = self.params.device
        self.n = n
        self.proj = gs.Proj(n, dev)
        self.ws_pre = gs.workspace(gs.GS_WS_PREPROCESS, n=n, device=dev)
        self.gscreen = torch.empty((max(n, 1), 9), dtype=torch.float32, device=dev)
        self.grads = gs.empty_blocked(n, self.deg, dev, zero=True)
        self.projected_for = None
