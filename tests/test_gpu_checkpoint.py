"""Resume from a checkpoint on the GPU: with fixed-point gradient sums every step is
reproducible bit for bit, so steps after Pipeline.from_checkpoint equal the same steps of
the pipeline that wrote the checkpoint (parameters, moments, statistics, step count)."""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes

pytestmark = pytest.mark.gpu


def test_resume_equals_uninterrupted_training(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s = scenes.random_scene(61, 4000, 2, spread=1.3, logscale_std=0.5)
    s.params[0:3] *= 0.8
    cams = [gs.make_camera(scenes.look_at_origin((0.6, 0.4, -4.5), 160, 120, 150.0)),
            gs.make_camera(scenes.look_at_origin((-2.5, 0.2, -3.8), 160, 120, 150.0))]
    rng = np.random.default_rng(9)
    targets = [torch.from_numpy(rng.random((3, 120, 160), dtype=np.float32)).cuda() for _ in cams]
    pl = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120, cfg=gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED))
    pl.enable_density_stats()
    for k in range(3):
        pl.step(cams[k % 2], targets[k % 2], next_cam=cams[(k + 1) % 2])
    path = tmp_path / "state.npz"
    pl.save_checkpoint(path)
    pl2 = Pipeline.from_checkpoint(path)
    assert (pl2.t, pl2.n, pl2.cfg.grad_sums) == (3, pl.n, gs.GS_GRAD_SUMS_FIXED)
    for k in range(3, 5):
        for p in (pl, pl2):
            p.step(cams[k % 2], targets[k % 2], next_cam=cams[(k + 1) % 2])
    torch.cuda.synchronize()
    assert pl2.t == pl.t == 5
    for name in ("params", "m", "v"):
        a = pl.planar(getattr(pl, name)).cpu().numpy()
        b = pl2.planar(getattr(pl2, name)).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
    assert np.array_equal(pl.dstats[:pl.n].cpu().numpy(), pl2.dstats[:pl2.n].cpu().numpy())
