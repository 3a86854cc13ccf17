"""Benchmark: full training steps of the 6M-Gaussian, SH-degree-3, 1920x1080 workload.

One step = preprocess + bin/sort + forward blend + L1/D-SSIM loss + backward
blend and chain with Adam applied to every parameter, for one of 100 seeded orbit
cameras (in order).  Prints one JSON line.

The roofline object describes the kernel that takes the most time per step (found
from a warm-up with every launch timed); during the timed steps the library brackets
that kernel's launches with HIP events on its own stream.

    python bench.py [--gpus 1] [--steps 100] [--warmup 5] [--no-cpu-baseline]

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD_CFG = 5
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published


def kernel_bytes(kernel, n, deg, P, fuse=True):
    """Algorithmic HBM bytes of one launch of the streaming kernels (fp32 everywhere).

    adam_vec4       per parameter: read theta, g, m, v; write theta, m, v            28 B
    chain           (Adam fused) per Gaussian: tile count 4, the nine screen gradients
                    36, read + write theta/m/v of all P planes 24 each; with the next
                    camera's projection also its record: splat 48, depth 4, rect 8,
                    tile count 4
    preprocess_fwd  per Gaussian: read all P planes, write splat 48, depth 4, rect 8,
                    tile count 4
    """
    record = 48 + 4 + 8 + 4
    table = {
        "adam_vec4": 28 * P * n,
        "chain": (4 + 36 + 24 * P + (record if fuse else 0)) * n,
        "preprocess_fwd": (4 * P + record) * n,
    }
    return table.get(kernel)


# kernels by stage (the names the library's per-kernel timing uses)
STAGE_KERNELS = {
    "preprocess": ("preprocess_fwd", "sum_counts"),
    "bin_sort": ("radix_upsweep", "radix_scan", "radix_downsweep", "scan_reduce", "scan_apply", "block_starts", "emit_pairs",
                 "tile_ranges", "fill_u32"),
    "render_fwd": ("render_fwd", "tile_order", "split_reset", "split_combine", "split_rewalk",
                   "split_finalize"),
    "loss": ("ssim", "loss_finalize"),
    "render_bwd": ("render_bwd", "zero_f32", "fixed_decode", "zero_u64"),
    "chain_adam": ("chain",),
}
# the blend kernels proper (forward walk with its split path, backward walk)
BLEND_KERNELS = STAGE_KERNELS["render_fwd"] + ("render_bwd",)
LLC_BYTES = 256 << 20               # MI355X Infinity Cache


def stage_kernel_ms(kernel_ms):
    """Kernel milliseconds per stage from {kernel: ms}."""
    return {st: round(sum(kernel_ms.get(k, 0.0) for k in ks), 4) for st, ks in STAGE_KERNELS.items()}


def sort_bytes(n, vis, pairs, num_tiles, depth_passes):
    """Algorithmic HBM bytes of one bin/sort (the passes the kernels make):

    per Gaussian      counts zeroed 4, pass 0 reads depth and tile count twice (upsweep,
                      downsweep) 16, the offsets scan reads counts twice and writes offsets 12
    per visible one   pass 0 writes key and id 8; every further depth pass reads the key
                      (upsweep) 4 and key and id 8 (downsweep) and writes them 8, the last
                      one writing no key but the id 4, the gathered rectangle 8 and tile
                      count 4 (and reading the rectangle 8); the emit reads two offsets, the
                      id and the rectangle 20
    per pair          emit writes tile and id 8; every tile pass reads the tile (upsweep) 4
                      and reads and writes tile and id (downsweep) 16
    per tile          the range search writes both ends 8 (its reads are a few per tile)"""
    tile_bits = max(int(num_tiles - 1).bit_length(), 0)
    tile_passes = (tile_bits + 8) // 9
    per_vis = 8 + (depth_passes - 2) * 20 + (4 + 8 + 4 + 4 + 8 + 8) + 20
    per_pair = 8 + 20 * tile_passes
    return 32 * n + per_vis * vis + per_pair * pairs + 8 * num_tiles


def depth_passes_of(pl, cam, torch):
    """Passes the depth sort made for the last projection: three, or four when some visible
    depth's bits exceed znear's by 2^27 or more."""
    vis = pl.proj.tiles[:pl.n] != 0
    if not bool(vis.any()):
        return 3
    bits = pl.proj.depth[:pl.n][vis].view(torch.int32).to(torch.int64)
    base = int(np.array([cam.znear], np.float32).view(np.int32)[0])
    return 4 if int(bits.max()) - base >= (1 << 27) else 3


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=WORKLOAD_CFG, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", default=None,
                    help="FIRST,CHUNK: pairs every tile walks in one block, and the chunk size of the "
                         "parallel walk of longer lists (library defaults if omitted)")
    ap.add_argument("--stage-report", action="store_true", help="also print per-stage times to stderr")
    ap.add_argument("--no-densify", action="store_true", help="skip the density-control measurement")
    ap.add_argument("--fixed-sums", action="store_true",
                    help="sum the backward's gradients in fixed point (reproducible; gs_config.grad_sums)")
    ap.add_argument("--no-fuse-projection", action="store_true",
                    help="project each step's camera in its own preprocess call instead of in the previous "
                         "step's update")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration block (configurations 1-4, measured after the headline)")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps per configuration in that block")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy a 1 GiB buffer three times (a plain copy of known size, the "
                         "reference for hardware byte counters)")
    return ap.parse_args()


def make_targets(wl, cams, Pipeline, torch):
    """Target images: renders of the perturbed copy of the scene (or of the second scene),
    one per camera, computed before timing."""
    tp = torch.from_numpy(wl.target_scene.params).cuda()
    tpl = Pipeline(tp, wl.target_scene.sh_degree, wl.cameras[0].width, wl.cameras[0].height)
    out = [tpl.forward(c).clone() for c in cams]
    del tpl, tp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


class StageTimer:
    """HIP events on the stream the library launches on (torch's current stream).  With
    the projection fused into the previous step's update, "preprocess" is empty and
    "render_bwd_adam" also holds the next camera's projection and depth order."""

    NAMES = ("preprocess", "bin_sort", "render_fwd", "loss", "render_bwd_adam")

    def __init__(self, torch, steps):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.NAMES) + 1)] for _ in range(steps)]

    def mark(self, step, k):
        self.ev[step][k].record()

    def per_stage_ms(self):
        t = np.array([[self.ev[s][k].elapsed_time(self.ev[s][k + 1]) for k in range(len(self.NAMES))]
                      for s in range(len(self.ev))])
        return t


def run_steps(pl, cams, targets, first, count, timer=None, gs=None, fuse=True):
    """Steps first .. first + count - 1 of the camera sequence.  With fuse, each step's
    update also projects the scene for the next step's camera (so a step's projection
    is normally done by the step before it; the very first is done on its own)."""
    for s in range(count):
        idx = (first + s) % len(cams)
        c, tgt = cams[idx], targets[idx]
        if timer: timer.mark(s, 0)
        if not (fuse and pl.projected_for is c):
            pl.pairs = gs.gs_preprocess(pl.params, pl.deg, c, pl.proj, pl.ws_pre, cfg=pl.cfg)
        pl.projected_for = None
        pl._reserve(pl.pairs)
        if timer: timer.mark(s, 1)
        gs.gs_bin_sort(pl.proj, c, pl.pairs, pl.keys, pl.vals, pl.ranges, pl.ws_sort)
        if timer: timer.mark(s, 2)
        gs.gs_render_fwd(pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.rgb, pl.T, pl.nc, pl.ws_render, cfg=pl.cfg)
        if timer: timer.mark(s, 3)
        gs.gs_loss_l1_dssim(pl.rgb, tgt, pl.lam, pl.loss, pl.dLdI, pl.ws_loss)
        if timer: timer.mark(s, 4)
        pl.t += 1
        if fuse:
            nxt = (idx + 1) % len(cams)
            pl.pairs = gs.gs_render_bwd_adam_project(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c,
                                                     pl.T, pl.nc, pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr,
                                                     pl.betas[0], pl.betas[1], pl.eps, pl.t, pl.ws_render,
                                                     cams[nxt], pl.proj, pl.ws_pre, pl.dstats, cfg=pl.cfg)
            pl.projected_for = cams[nxt]
        else:
            gs.gs_render_bwd_adam(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc,
                                  pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr, pl.betas[0], pl.betas[1], pl.eps, pl.t,
                                  pl.ws_render, cfg=pl.cfg)
        if timer: timer.mark(s, 5)


def measure_densify(pl, cams, targets, first, torch, gs, steps=3):
    """Density control on the benchmark's population (untimed by the step clock): the
    statistics of `steps` training steps (added by the projecting update), then one
    densification (gs_densify: count, then write) timed with HIP events.  The gradient
    threshold is the 95th percentile of the observed averages, so that about one
    Gaussian in twenty observed is cloned or split; prune opacity 0.005, prune scale 1,
    split scale 0.05 (world units)."""
    pl.enable_density_stats()
    run_steps(pl, cams, targets, first, steps, gs=gs, fuse=True)
    st = pl.dstats[:pl.n]
    seen = st[:, 1] > 0
    avg = st[seen, 0] / st[seen, 1]
    thr = float(torch.quantile(avg[:1 << 24], 0.95)) if avg.numel() else 1.0
    n, deg = pl.n, pl.deg
    gen = torch.Generator(device=pl.params.device).manual_seed(5)
    rand = torch.randn((max(n, 1), 2, 3), dtype=torch.float32, device=pl.params.device, generator=gen)
    ws = gs.workspace(gs.GS_WS_DENSIFY, n=n)
    thr_args = dict(grad_threshold=thr, prune_opacity=0.005, prune_scale=1.0, split_scale=0.05)
    n_new, counts = gs.gs_densify(pl.params, pl.m, pl.v, pl.dstats, rand, n, deg, ws=ws, **thr_args)
    outs = [gs.empty_blocked(n_new, deg) for _ in range(3)]
    so = torch.empty((max(n_new, 1), 2), dtype=torch.float32, device=pl.params.device)

    def write():
        gs.gs_densify(pl.params, pl.m, pl.v, pl.dstats, rand, n, deg, ws=ws, params_out=outs[0], m_out=outs[1],
                      v_out=outs[2], stats_out=so, capacity=n_new, **thr_args)
    write()   # untimed: the kernels' first launch (the inputs are not modified, so it can be repeated)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    gs.gs_densify(pl.params, pl.m, pl.v, pl.dstats, rand, n, deg, ws=ws, **thr_args)
    ev[1].record()
    torch.cuda.synchronize()
    ev[2].record()
    write()
    end = torch.cuda.Event(enable_timing=True)
    end.record()
    torch.cuda.synchronize()
    count_ms, write_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(end)
    P = 11 + 3 * (deg + 1) ** 2
    # the write phase reads theta, m, v of every source Gaussian, its flags and prefix sums,
    # and a split parent's normals; it writes theta, m, v and the zeroed statistics of every output
    wbytes = (12 * P + 24) * n + 24 * counts[2] + (12 * P + 8) * n_new
    return {"steps_of_statistics": steps, "grad_threshold": thr, "n_in": n, "n_out": n_new,
            "kept_cloned_split": list(counts), "count_ms": round(count_ms, 4), "write_ms": round(write_ms, 4),
            "write_bytes": wbytes, "write_GBps": round(wbytes / (write_ms / 1000.0) / 1e9, 1)}


def measure_charbonnier(pl, targets, torch, gs, reps=20):
    """The Charbonnier loss with exposure on the benchmark's image (an alternative to the
    L1 + D-SSIM loss, not part of the step): average of `reps` calls, HIP events."""
    dev = pl.params.device
    exposure = torch.tensor([0.05, -0.01], dtype=torch.float32, device=dev)
    loss = torch.zeros(1, device=dev)
    dexp = torch.zeros(2, device=dev)
    grad = torch.empty_like(pl.rgb)
    ws = gs.workspace(gs.GS_WS_LOSS_CHARBONNIER, W=pl.W, H=pl.H)
    gs.gs_loss_charbonnier(pl.rgb, targets[0], exposure, loss, grad, ws, dL_dexposure=dexp)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        gs.gs_loss_charbonnier(pl.rgb, targets[0], exposure, loss, grad, ws, dL_dexposure=dexp)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    nbytes = 3 * pl.H * pl.W * 12   # image and target read, gradient written
    return {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(nbytes / (ms / 1000.0) / 1e9, 1)}


def measure_camera_grad(pl, cam, torch, gs, reps=20):
    """The camera-pose gradient (optional, not part of the step) over the benchmark's
    population, on the screen partials and tile counts the last step left: average of `reps`
    calls, HIP events.  Algorithmic bytes: every Gaussian's tile count, eleven geometry
    planes and six screen partials; and, in every 64-Gaussian group with a visible member,
    the colour planes and colour partials of the whole group (a wave reads a plane's
    256-byte row when any of its lanes needs it, as the projection does)."""
    dev = pl.params.device
    out = torch.zeros(6, dtype=torch.float64, device=dev)
    ws = gs.workspace(gs.GS_WS_CAMERA_GRAD, n=pl.n)
    gs.gs_camera_grad(pl.params, pl.deg, pl.proj, cam, pl.gscreen, out, ws, cfg=pl.cfg)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        gs.gs_camera_grad(pl.params, pl.deg, pl.proj, cam, pl.gscreen, out, ws, cfg=pl.cfg)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    vis = (pl.proj.tiles[:pl.n] != 0).int()
    pad = (-pl.n) % 64
    groups_vis = int((torch.nn.functional.pad(vis, (0, pad)).view(-1, 64).sum(1) > 0).sum().item())
    nbytes = pl.n * (4 + 11 * 4 + 6 * 4) + groups_vis * 64 * (3 * (pl.deg + 1) ** 2 * 4 + 3 * 4)
    return {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(nbytes / (ms / 1000.0) / 1e9, 1)}


def count_evals(pl, torch):
    """Gaussian-pixel evaluations of the last forward/backward: the forward examines
    entries up to the stopping one (n_contrib for stopped pixels, the whole tile list
    otherwise); the backward walks n_contrib entries."""
    H, W = pl.H, pl.W
    tx = (W + 15) // 16
    ys = torch.arange(H, device="cuda") // 16
    xs = torch.arange(W, device="cuda") // 16
    tile = ys[:, None] * tx + xs[None, :]
    rng = pl.ranges.long()
    length = (rng[1] - rng[0])[tile]
    nc = pl.nc.long()
    stopped = pl.T < 1e-4
    fwd = torch.where(stopped, nc, length).sum().item()
    bwd = nc.sum().item()
    return int(fwd), int(bwd)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if
    the sources the kernel is built from are unchanged since the counters were taken
    (sha256 over their contents, in the listed order); otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic_train_step_6m_1080p.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and parts[0] == "traffic" and parts[1] == kernel:
            kv = dict(p.split("=", 1) for p in parts[2:])
            h = hashlib.sha256()
            for src in kv["sources"].split(","):
                h.update(open(os.path.join(ROOT, src), "rb").read())
            if h.hexdigest() != kv["sha256"]:
                return None
            return round((float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                          float(kv["write_kib"]) * float(kv["write_scale"])) * 1024.0)
    return None


VALU_PEAK = 256 * 4 * 2.4e9 / 4      # wave64 VALU instructions/s: one per SIMD every 4 cycles


def measured_valu():
    """VALU issue fraction of the blend kernels from the committed rocprofv3 SQ counter
    summary (wave instructions per dispatch over that run's average duration, against
    VALU_PEAK), for each kernel whose sources are unchanged since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_valu_blend_6m_1080p.md")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and parts[0] == "valu":
            kv = dict(p.split("=", 1) for p in parts[2:])
            h = hashlib.sha256()
            for src in kv["sources"].split(","):
                h.update(open(os.path.join(ROOT, src), "rb").read())
            if h.hexdigest() != kv["sha256"]:
                continue
            insts, ns = float(kv["wave_insts"]), float(kv["avg_ns"])
            out[parts[1]] = {"wave_insts": insts, "avg_us": round(ns / 1000.0, 1),
                             "frac": round(insts / (ns * 1e-9) / VALU_PEAK, 3)}
    return out


def cpu_baseline(wl):
    """The oracle (test infrastructure) on one training step: camera 0, all stages, one core."""
    from oracle import oracle as O
    cam = wl.cameras[0]
    p = wl.scene.params
    deg = wl.scene.sh_degree
    # a seeded synthetic target: the oracle's cost does not depend on the target's content
    tgt = np.random.default_rng(7).random((3, cam.height, cam.width), dtype=np.float32)
    lr = np.array([1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3])
    t0 = time.perf_counter()
    r = O.train_step(p, deg, cam, tgt)
    z = np.zeros_like(p)
    O.adam(p, r["gparams"], z, z, deg, lr, step=1, dtype=np.float32)
    dt = time.perf_counter() - t0
    return dict(value=1.0 / dt, unit="iter/s", cores=1, kind="oracle",
                sample=f"one full training step (camera 0 of {len(wl.cameras)}: preprocess, bin/sort, forward, "
                       f"loss, backward, chain, Adam over {p.size} parameters) of the same workload, "
                       f"single-threaded fp32 oracle, seeded synthetic target; {dt:.1f} s",
                seconds=dt, evals=int(r["fwd"]["evals"] + int(r["fwd"]["n_contrib"].sum())))


def oracle_step_seconds(wl):
    """The oracle (test infrastructure) on one training step of a workload's first camera:
    all stages including Adam, one core, seeded synthetic target."""
    from oracle import oracle as O
    cam = wl.cameras[0]
    p, deg = wl.scene.params, wl.scene.sh_degree
    tgt = np.random.default_rng(7).random((3, cam.height, cam.width), dtype=np.float32)
    lr = np.array([1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3])
    t0 = time.perf_counter()
    r = O.train_step(p, deg, cam, tgt)
    z = np.zeros_like(p)
    O.adam(p, r["gparams"], z, z, deg, lr, step=1, dtype=np.float32)
    return time.perf_counter() - t0, r


def hbm_entry(nbytes, ms, working_set):
    """Achieved GB/s of a stage; its fraction of the HBM peak only when its working set is at
    least twice the 256 MB last-level cache (otherwise the time is reported as it is)."""
    gbps = nbytes / (ms / 1000.0) / 1e9 if ms > 0 else None
    frac = round(gbps / HBM_PEAK_GBS, 4) if gbps and working_set >= 2 * LLC_BYTES else None
    return {"ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(gbps, 1) if gbps else None, "frac": frac,
            "working_set": int(working_set)}


def measure_config(k, steps, torch, gs, scenes, Pipeline, cfg, with_oracle):
    """One configuration's block: the same fused training step as the headline, on its own
    cameras and target.  Per-stage kernel times, eval counts and the pairs of each sort come
    from profiled steps (every launch timed, counts read between steps); iter/s from
    separately timed steps; the projection alone from repeated gs_preprocess calls."""
    t_setup = time.perf_counter()
    wl = scenes.CONFIGS[k]()
    cams = [gs.make_camera(c) for c in wl.cameras]
    targets = make_targets(wl, cams, Pipeline, torch)
    params = torch.from_numpy(wl.scene.params).cuda()
    n, deg = wl.scene.n, wl.scene.sh_degree
    P = params.shape[0]
    cam0 = wl.cameras[0]
    pl = Pipeline(params, deg, cam0.width, cam0.height, cfg=cfg)
    setup_s = time.perf_counter() - t_setup
    warm = 3
    run_steps(pl, cams, targets, 0, warm, gs=gs)
    torch.cuda.synchronize()
    prof = min(steps, 10)
    ev_f = ev_b = 0
    vis_sum = pairs_sum = sbytes = 0
    num_tiles = pl.num_tiles
    gs.gs_profile_enable(True)
    for i in range(prof):
        c = wl.cameras[(warm + i) % len(wl.cameras)]
        if pl.projected_for is not cams[(warm + i) % len(cams)]:
            pl.pairs = gs.gs_preprocess(pl.params, pl.deg, cams[(warm + i) % len(cams)], pl.proj, pl.ws_pre,
                                        cfg=pl.cfg)
            pl.projected_for = cams[(warm + i) % len(cams)]
        vis = int(pl.proj.n_visible.item())
        dp = depth_passes_of(pl, c, torch)
        vis_sum += vis
        pairs_sum += pl.pairs
        sbytes += sort_bytes(n, vis, pl.pairs, num_tiles, dp)
        run_steps(pl, cams, targets, warm + i, 1, gs=gs)
        f, b = count_evals(pl, torch)
        ev_f += f
        ev_b += b
    torch.cuda.synchronize()
    kernel_ms = {kk: ms / prof for kk, (cnt, ms) in gs.gs_profile_query().items()}
    gs.gs_profile_enable(False)
    stage = stage_kernel_ms(kernel_ms)
    blend_ms = sum(kernel_ms.get(kk, 0.0) for kk in BLEND_KERNELS)
    # timed steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(pl, cams, targets, warm + prof, steps, gs=gs)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / steps
    # the projection on its own
    gs.gs_profile_enable(True, "preprocess_fwd")
    reps = 5
    for _ in range(reps):
        gs.gs_preprocess(pl.params, pl.deg, cams[0], pl.proj, pl.ws_pre, cfg=pl.cfg)
    torch.cuda.synchronize()
    pre = gs.gs_profile_query().get("preprocess_fwd", (1, 0.0))
    gs.gs_profile_enable(False)
    pl.projected_for = None
    pre_ms = pre[1] / max(pre[0], 1)
    pre_bytes = kernel_bytes("preprocess_fwd", n, deg, P)
    chain_bytes = kernel_bytes("chain", n, deg, P, True)
    pairs_avg = pairs_sum / prof
    out = {
        "workload": wl.name, "gaussians": n, "sh_degree": deg, "image": [cam0.width, cam0.height],
        "pairs_per_step": int(pairs_avg), "visible_per_step": int(vis_sum / prof),
        "iter_per_s": round(1000.0 / ms_step, 2), "ms_per_step": round(ms_step, 4), "steps": steps,
        "stage_kernel_ms": stage,
        "evals_per_step": {"fwd": ev_f // prof, "bwd": ev_b // prof},
        "blend_ms": round(blend_ms, 4),
        "blend_evals_per_s": round((ev_f + ev_b) / prof / (blend_ms / 1000.0), 1) if blend_ms > 0 else None,
        "hbm": {
            "preprocess_fwd": hbm_entry(pre_bytes, pre_ms, pre_bytes),
            "bin_sort": hbm_entry(sbytes / prof, stage["bin_sort"], 16 * pairs_avg + 12 * n),
            "chain_adam": hbm_entry(chain_bytes, kernel_ms.get("chain", 0.0), chain_bytes),
        },
        "setup_s": round(setup_s, 2),
    }
    if with_oracle:
        dt, r = oracle_step_seconds(wl)
        model, _ = host_cpu()
        out["oracle"] = {"iter_per_s": round(1.0 / dt, 4), "s_per_step": round(dt, 3), "cores": 1,
                         "cpu": model, "evals_per_step": int(r["fwd"]["evals"] + int(r["fwd"]["n_contrib"].sum()))}
    del pl, params, targets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this rasteriser runs on one GPU; runs on several GPUs are not supported "
                                   f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})"}))
        sys.exit(2)
    if args.warmup < 1 or args.steps < 1:
        print(json.dumps({"error": "--warmup and --steps must be at least 1 (a warm-up step picks the kernel "
                                   "whose roofline the timed steps measure)"}))
        sys.exit(2)
    import torch
    from differentiable_tile_gaussian_amd import gs, scenes
    from differentiable_tile_gaussian_amd.pipeline import Pipeline

    torch.cuda.set_device(0)
    split = [2048, 512]
    if args.split:
        split = [int(x) for x in args.split.split(",")]
    fuse = not args.no_fuse_projection
    cfg = gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED if args.fixed_sums else gs.GS_GRAD_SUMS_FLOAT,
                      split_first=split[0], split_chunk=split[1])
    t_setup = time.perf_counter()
    wl = scenes.CONFIGS[args.workload]()
    cams = [gs.make_camera(c) for c in wl.cameras]
    cam0 = wl.cameras[0]
    targets = make_targets(wl, cams, Pipeline, torch)
    params = torch.from_numpy(wl.scene.params).cuda()
    n, deg = wl.scene.n, wl.scene.sh_degree
    P = params.shape[0]
    pl = Pipeline(params, deg, cam0.width, cam0.height, cfg=cfg)
    setup_s = time.perf_counter() - t_setup

    # warm-up: the first step untimed (code objects load, caches are cold), then every
    # kernel launch of the remaining warm-up steps timed: per-kernel time per step and the
    # dominant kernel
    cold = 1 if args.warmup >= 2 else 0
    run_steps(pl, cams, targets, 0, cold, gs=gs, fuse=fuse)
    torch.cuda.synchronize()
    gs.gs_profile_enable(True)
    run_steps(pl, cams, targets, cold, args.warmup - cold, gs=gs, fuse=fuse)
    torch.cuda.synchronize()
    warm = gs.gs_profile_query()
    kernel_ms = {k: ms / max(args.warmup - cold, 1) for k, (cnt, ms) in warm.items()}
    dominant = max(kernel_ms, key=kernel_ms.get)
    # timed steps: only the dominant kernel's launches carry events
    gs.gs_profile_enable(True, dominant)
    timer = StageTimer(torch, args.steps)
    t0 = time.perf_counter()
    run_steps(pl, cams, targets, args.warmup, args.steps, timer=timer, gs=gs, fuse=fuse)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    live = gs.gs_profile_query()[dominant]
    gs.gs_profile_enable(False)
    stage = timer.per_stage_ms()
    ms_per_step = wall * 1000.0 / args.steps

    # evaluation counts: replay the same cameras from the same starting state, untimed
    params2 = torch.from_numpy(wl.scene.params).cuda()
    pl2 = Pipeline(params2, deg, cam0.width, cam0.height, cfg=cfg)
    run_steps(pl2, cams, targets, 0, args.warmup, gs=gs, fuse=fuse)
    torch.cuda.synchronize()
    gs.gs_profile_enable(True)   # the replayed steps' kernel times, for the blend-only rate
    ev_f = ev_b = 0
    for s in range(args.steps):
        run_steps(pl2, cams, targets, args.warmup + s, 1, gs=gs, fuse=fuse)
        f, b = count_evals(pl2, torch)
        ev_f += f
        ev_b += b
    torch.cuda.synchronize()
    replay_ms = {k: ms / args.steps for k, (cnt, ms) in gs.gs_profile_query().items()}
    gs.gs_profile_enable(False)
    blend_ms = sum(replay_ms.get(k, 0.0) for k in BLEND_KERNELS)
    del pl2, params2
    densify = measure_densify(pl, cams, targets, args.warmup + args.steps, torch, gs) if not args.no_densify else None
    charbonnier = measure_charbonnier(pl, targets, torch, gs)
    camera_grad = measure_camera_grad(pl, cams[0], torch, gs)

    # roofline of the dominant kernel from its live launch times
    dom_launches, dom_ms = live
    dom_avg_ms = dom_ms / dom_launches
    dom_bytes = kernel_bytes(dominant, n, deg, P, fuse)
    if dom_bytes is not None:
        achieved = dom_bytes / (dom_avg_ms / 1000.0) / 1e9
        roof = {"kernel": dominant + "_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dominant + "_kernel"), "bytes_per_launch": dom_bytes,
                "avg_launch_ms": round(dom_avg_ms, 4), "launches": dom_launches}
    else:
        roof = {"kernel": dominant + "_kernel", "bound": None, "achieved": None, "peak": None, "unit": None,
                "frac": None, "traffic": None, "avg_launch_ms": round(dom_avg_ms, 4), "launches": dom_launches}
    out = {
        "metric": "fwd+bwd raster iterations/sec and Gaussian-pixel evals/s; % of HBM/VALU roofline",
        "value": round(1000.0 / ms_per_step, 3),
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "gaussians": n, "sh_degree": deg, "image": [cam0.width, cam0.height],
                   "cameras": len(cams), "step": ("sort+fwd+loss+bwd+chain+adam+projection of the next camera (fused; one projection per step)"
                            if fuse else "preprocess+sort+fwd+loss+bwd+chain+adam (fused)"), "parallelism": "none",
                   "blend_split": split, "grad_sums": "fixed" if args.fixed_sums else "float"},
        "evals_per_s": round((ev_f + ev_b) / args.steps / (blend_ms / 1000.0), 1),
        "evals_basis": "Gaussian-pixel evaluations of the forward and backward walks over the blend kernels' "
                       "time (forward walk with its split path, backward walk), same cameras replayed",
        "evals_per_step": {"fwd": ev_f // args.steps, "bwd": ev_b // args.steps},
        "blend_ms_per_step": round(blend_ms, 4),
        "stage_kernel_ms": stage_kernel_ms(replay_ms),
        "stage_ms": {k: round(float(stage[:, i].mean()), 4) for i, k in enumerate(StageTimer.NAMES)},
        "stage_ms_median": {k: round(float(np.median(stage[:, i])), 4) for i, k in enumerate(StageTimer.NAMES)},
        "kernel_ms_per_step": {k: round(v, 4) for k, v in sorted(kernel_ms.items(), key=lambda kv: -kv[1])},
        "blend_valu": {"bound": "alu", "peak": VALU_PEAK, "unit": "wave instr/s", "kernels": measured_valu()},
        "roofline": roof,
        "densify": densify,
        "charbonnier_loss": charbonnier,
        "camera_grad": camera_grad,
        "setup_s": round(setup_s, 2),
    }
    if not args.no_configs and args.workload == WORKLOAD_CFG:
        del pl, params, targets
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["configs"] = {str(k): measure_config(k, args.config_steps, torch, gs, scenes, Pipeline, cfg,
                                                 with_oracle=not args.no_cpu_baseline and k <= 2)
                          for k in (1, 2, 3, 4)}
    if not args.no_cpu_baseline and args.workload == WORKLOAD_CFG:
        cb = cpu_baseline(wl)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        out["cpu_baseline"]["cpu"], out["cpu_baseline"]["host_cpus"] = host_cpu()
    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = int(src.numel() * 4)
    if args.stage_report:
        print(json.dumps({"stage_ms_all": stage.round(4).tolist()}), file=sys.stderr)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
