"""Checkpoint files (host logic): the blocked-to-planar copy against the layout's index
formula, and the arrays save_checkpoint writes (plain arrays that load without pickle)."""
import numpy as np
import torch

from differentiable_tile_gaussian_amd import gs
from differentiable_tile_gaussian_amd.pipeline import Pipeline, blocked_to_planar


def test_blocked_to_planar_follows_the_layout():
    rng = np.random.default_rng(0)
    for n, P in ((1, 14), (64, 59), (130, 23)):
        groups = (n + 63) // 64
        blocked = rng.standard_normal((groups, P, 64)).astype(np.float32)
        flat = blocked.reshape(-1)
        want = np.array([[flat[((i // 64) * P + p) * 64 + i % 64] for i in range(n)] for p in range(P)], np.float32)
        assert np.array_equal(blocked_to_planar(blocked, n), want)


def _stub(n=70, deg=1, with_stats=True):
    P = 11 + 3 * (deg + 1) ** 2
    groups = (n + 63) // 64
    st = Pipeline.__new__(Pipeline)
    g = torch.Generator().manual_seed(1)
    st.n, st.deg, st.t, st.W, st.H, st.lam = n, deg, 17, 160, 120, 0.2
    st.lr, st.betas, st.eps = (1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3), (0.9, 0.999), 1e-8
    st.cfg = gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED, active_sh_degree=0, mip_compensation=True,
                         split_first=64, split_chunk=32)
    st.params, st.m, st.v = (torch.randn((groups, P, 64), generator=g) for _ in range(3))
    st.dstats = torch.rand((n, 2), generator=g) if with_stats else None
    return st


def test_checkpoint_file_holds_the_state(tmp_path):
    st = _stub()
    path = tmp_path / "state.npz"
    Pipeline.save_checkpoint(st, path)
    with np.load(path, allow_pickle=False) as z:
        assert int(z["n"]) == 70 and int(z["sh_degree"]) == 1 and int(z["t"]) == 17
        assert list(z["size"]) == [160, 120] and float(z["lam"]) == 0.2 and float(z["eps"]) == 1e-8
        assert tuple(z["lr"]) == st.lr and tuple(z["betas"]) == st.betas
        assert list(z["cfg"]) == [gs.GS_GRAD_SUMS_FIXED, 0, 1, 64, 32]
        for k in ("params", "m", "v", "dstats"):
            assert np.array_equal(z[k], getattr(st, k).numpy()), k
    st = _stub(with_stats=False)
    Pipeline.save_checkpoint(st, path)
    with np.load(path, allow_pickle=False) as z:
        assert z["dstats"].shape == (0, 2)
