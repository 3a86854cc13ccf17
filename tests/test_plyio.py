""".ply export (differentiable_tile_gaussian_amd.plyio), on the CPU.

Pins: a viewer's colour formula applied to the file's fields (0.5 + C0 f_dc + the higher
bands, f_rest in channel-major order, with the basis of [GSG] "Spherical harmonics":
the printed degree-1 and degree-2 constants, degree 3 from the same real basis) equals the
oracle's colour of every Gaussian before the clamp; the header lists the properties
viewers read; reading the file back returns the parameters (the DC up to one rounding of
the conversion).
"""
import math

import numpy as np
import pytest

from differentiable_tile_gaussian_amd import plyio, scenes


def _viewer_basis(d):
    """Real SH basis of degrees 1-3 at unit directions d [n][3], in the viewers' order."""
    x, y, z = d[:, 0], d[:, 1], d[:, 2]
    xx, yy, zz = x * x, y * y, z * z
    c1 = 0.4886025119029199
    c2 = (1.0925484305920792, -1.0925484305920792, 0.31539156525252005, -1.0925484305920792, 0.5462742152960396)
    c3 = (-0.5900435899266435, 2.890611442640554, -0.4570457994644658, 0.3731763325901154, -0.4570457994644658,
          1.445305721320277, -0.5900435899266435)
    return np.stack([-c1 * y, c1 * z, -c1 * x,
                     c2[0] * x * y, c2[1] * y * z, c2[2] * (2 * zz - xx - yy), c2[3] * x * z, c2[4] * (xx - yy),
                     c3[0] * y * (3 * xx - yy), c3[1] * x * y * z, c3[2] * y * (4 * zz - xx - yy),
                     c3[3] * z * (2 * zz - 3 * xx - 3 * yy), c3[4] * x * (4 * zz - xx - yy),
                     c3[5] * z * (xx - yy), c3[6] * x * (xx - 3 * yy)], axis=1)


def _read_fields(path):
    with open(path, "rb") as f:
        names, n = [], 0
        assert f.readline() == b"ply\n"
        assert f.readline() == b"format binary_little_endian 1.0\n"
        while True:
            line = f.readline().decode().strip()
            if line == "end_header":
                break
            parts = line.split()
            if parts[0] == "element":
                n = int(parts[2])
            else:
                assert parts[:2] == ["property", "float"]
                names.append(parts[2])
        return np.frombuffer(f.read(), dtype=[(k, "<f4") for k in names], count=n), names


@pytest.mark.parametrize("deg", [0, 1, 3])
def test_viewer_colour_equals_the_oracle(oracle, tmp_path, deg):
    s = scenes.random_scene(7 + deg, 200, deg)
    if deg:
        s.params[14:] = np.random.default_rng(deg).normal(0, 0.3, s.params[14:].shape).astype(np.float32)
    cam = scenes.look_at_origin((0.6, -0.3, -4.0), 64, 48, 60.0)
    path = tmp_path / "cloud.ply"
    plyio.write_ply(path, s.params, deg)
    rec, names = _read_fields(path)
    K = (deg + 1) ** 2 - 1
    assert names[:9] == ["x", "y", "z", "nx", "ny", "nz", "f_dc_0", "f_dc_1", "f_dc_2"]
    assert names[9 + 3 * K:] == ["opacity", "scale_0", "scale_1", "scale_2", "rot_0", "rot_1", "rot_2", "rot_3"]
    pre = oracle.preprocess(s.params, deg, cam, smooth=True, dtype=np.float64)
    mean = np.stack([rec["x"], rec["y"], rec["z"]], 1).astype(np.float64)
    d = mean - cam.campos.astype(np.float64)
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    Y = _viewer_basis(d)
    vis = pre["visible"].astype(bool)
    for c in range(3):
        col = 0.5 + plyio.C0 * rec[f"f_dc_{c}"].astype(np.float64)
        for k in range(K):
            col = col + rec[f"f_rest_{c * K + k}"].astype(np.float64) * Y[:, k]
        np.testing.assert_allclose(col[vis], pre["rgb"][c][vis], rtol=0, atol=1e-6)
    np.testing.assert_array_equal(rec["opacity"], s.params[10])
    np.testing.assert_array_equal(rec["rot_2"], s.params[8])
    assert not rec["nx"].any()


def test_round_trip(tmp_path):
    s = scenes.random_scene(3, 130, 2)
    path = tmp_path / "cloud.ply"
    plyio.write_ply(path, s.params, 2)
    back, deg = plyio.read_ply(path)
    assert deg == 2 and back.shape == s.params.shape
    np.testing.assert_array_equal(np.delete(back, [11, 12, 13], axis=0), np.delete(s.params, [11, 12, 13], axis=0))
    np.testing.assert_allclose(back[11:14], s.params[11:14], rtol=0, atol=4 * np.finfo(np.float32).eps)
    with pytest.raises(ValueError):
        plyio.write_ply(path, s.params, 3)
    assert math.isclose(plyio.C0, 0.28209479177387814, rel_tol=1e-15)
