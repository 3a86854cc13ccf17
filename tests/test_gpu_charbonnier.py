"""The Charbonnier loss with exposure on the GPU against the oracle (fp64): the loss and
the two exposure gradients to 1e-5 relative, dL/dimg element by element to 1e-5 relative
of its largest magnitude; two runs give identical words (fixed summation order)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("h,w,lg,b", [(128, 128, 0.0, 0.0), (37, 53, 0.15, -0.02), (1080, 1920, -0.1, 0.05)])
def test_charbonnier_matches_oracle(torch_cuda, oracle, h, w, lg, b):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    rng = np.random.default_rng(h + w)
    img = rng.random((3, h, w), dtype=np.float32)
    tgt = np.clip(img + rng.normal(0, 0.1, img.shape), 0, 1).astype(np.float32)
    tgt[:, : h // 4] = rng.random((3, h // 4, w), dtype=np.float32)   # some large errors
    loss_r, g_r, dlg_r, db_r = oracle.loss_charbonnier(img, tgt, delta=0.03, log_gain=lg, bias=b)
    dev = "cuda"
    ti, tt = torch.from_numpy(img).to(dev), torch.from_numpy(tgt).to(dev)
    exp_ = torch.tensor([lg, b], dtype=torch.float32, device=dev)
    loss = torch.zeros(1, device=dev)
    grad = torch.empty_like(ti)
    dexp = torch.zeros(2, device=dev)
    ws = gs.workspace(gs.GS_WS_LOSS_CHARBONNIER, W=w, H=h)
    outs = []
    for _ in range(2):
        gs.gs_loss_charbonnier(ti, tt, exp_, loss, grad, ws, delta=0.03, dL_dexposure=dexp)
        torch.cuda.synchronize()
        outs.append((loss.cpu().numpy().copy(), grad.cpu().numpy().copy(), dexp.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][2], outs[1][2])
    assert np.array_equal(outs[0][1], outs[1][1])
    l, g, d = outs[0]
    assert abs(l[0] - loss_r) <= 1e-5 * abs(loss_r)
    assert abs(d[0] - dlg_r) <= 1e-5 * abs(dlg_r) + 1e-9
    assert abs(d[1] - db_r) <= 1e-5 * abs(db_r) + 1e-9
    np.testing.assert_allclose(g, g_r, rtol=1e-5, atol=1e-5 * np.abs(g_r).max())
