"""One training step for one camera through the C ABI, with the device buffers
it needs kept between calls (grown only when a larger pair count appears).

torch allocates memory and provides the stream; every stage runs in libgs.so.
"""
from __future__ import annotations

import torch

from . import gs

DEFAULT_LR = (1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3)   # means, log-scales, quaternion, opacity, colour


class Pipeline:
    def __init__(self, params: torch.Tensor, sh_degree: int, width: int, height: int, lam: float = 0.2,
                 lr=DEFAULT_LR, betas=(0.9, 0.999), eps=1e-8):
        """params: [P][n] float32 device tensor (plane-major); it is copied into the
        library's blocked layout, in which params, grads, m and v are then kept."""
        assert params.is_cuda and params.dtype == torch.float32 and params.is_contiguous()
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
        need = gs.gs_workspace_bytes(gs.GS_WS_RENDER, self.n, pairs, self.W, self.H)
        if self.ws_render.numel() < need:
            self.ws_render = torch.empty(int(need * 1.25) + 4096, dtype=torch.uint8, device=self.params.device)

    def forward(self, cam: gs.GsCamera):
        if self.projected_for is not cam:
            self.pairs = gs.gs_preprocess(self.params, self.deg, cam, self.proj, self.ws_pre)
        self.projected_for = None
        self._reserve(self.pairs)
        gs.gs_bin_sort(self.proj, cam, self.pairs, self.keys, self.vals, self.ranges, self.ws_sort)
        gs.gs_render_fwd(self.proj, self.vals, self.ranges, self.pairs, cam, self.rgb, self.T, self.nc,
                         self.ws_render)
        return self.rgb

    def backward(self, cam: gs.GsCamera, target: torch.Tensor):
        gs.gs_loss_l1_dssim(self.rgb, target, self.lam, self.loss, self.dLdI, self.ws_loss)
        gs.gs_render_bwd(self.params, self.deg, self.proj, self.vals, self.ranges, self.pairs, cam, self.T, self.nc,
                         self.dLdI,
                         self.gscreen, self.grads, self.ws_render)

    def adam(self):
        self.t += 1
        gs.gs_adam_step(self.params, self.grads, self.m, self.v, self.n, self.deg, self.lr, self.betas[0],
                        self.betas[1], self.eps, self.t)

    def backward_adam(self, cam: gs.GsCamera, target: torch.Tensor, next_cam: gs.GsCamera = None):
        """Loss, backward and Adam with the chain and Adam fused (no gradient written).
        With next_cam, the update also projects the scene for next_cam, and the next
        forward(next_cam) (the same camera object) uses that projection."""
        gs.gs_loss_l1_dssim(self.rgb, target, self.lam, self.loss, self.dLdI, self.ws_loss)
        self.t += 1
        if next_cam is None:
            gs.gs_render_bwd_adam(self.params, self.deg, self.proj, self.vals, self.ranges, self.pairs, cam, self.T,
                                  self.nc, self.dLdI, self.gscreen, self.m, self.v, self.lr, self.betas[0],
                                  self.betas[1], self.eps, self.t, self.ws_render)
            return
        self.pairs = gs.gs_render_bwd_adam_project(self.params, self.deg, self.proj, self.vals, self.ranges,
                                                   self.pairs, cam, self.T, self.nc, self.dLdI, self.gscreen, self.m,
                                                   self.v, self.lr, self.betas[0], self.betas[1], self.eps, self.t,
                                                   self.ws_render, next_cam, self.proj, self.ws_pre, self.dstats)
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
                                      self.nc, self.dLdI, self.gscreen, self.grads, self.ws_render, 1.0 / B, k > 0)
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

    def _resize(self, n):
        """Buffers sized by the Gaussian count, after the population changed."""
        dev = self.params.device
        self.n = n
        self.proj = gs.Proj(n, dev)
        self.ws_pre = gs.workspace(gs.GS_WS_PREPROCESS, n=n, device=dev)
        self.gscreen = torch.empty((max(n, 1), 9), dtype=torch.float32, device=dev)
        self.grads = gs.empty_blocked(n, self.deg, dev, zero=True)
        self.projected_for = None
