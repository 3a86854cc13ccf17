"""Writing and reading the Gaussian cloud as a .ply file ([GSG] closing section: what
training keeps is every Gaussian's position, scale, quaternion, colour with its SH extras
and opacity, written to a standard .ply file that Gaussian-splat viewers open).

The layout is the one those viewers read (binary little-endian, one float32 property per
field, in this order): x y z, nx ny nz (zero), f_dc_0..2, f_rest_0..3K-1 (the K higher
bands of channel 0, then of channel 1, then of channel 2), opacity (the logit), scale_0..2
(the log-scales), rot_0..3 (the quaternion w x y z as stored).  Viewers form the colour as
0.5 + C0 f_dc + sum_k f_rest_k Y_k with C0 = 1 / (2 sqrt(pi)) the degree-0 basis value and
the same higher-band basis as here, while this library's colour is dc + sum_k sh_k Y_k, so
f_dc = (dc - 0.5) / C0 and the bands are written as they are.

Host code on planar [P][n] float32 arrays (gs.from_blocked gives them from the device).
"""
from __future__ import annotations

import math

import numpy as np

C0 = 1.0 / (2.0 * math.sqrt(math.pi))


def _num_planes(deg):
    return 11 + 3 * (deg + 1) ** 2


def _fields(deg):
    K = (deg + 1) ** 2 - 1
    return (["x", "y", "z", "nx", "ny", "nz", "f_dc_0", "f_dc_1", "f_dc_2"] +
            [f"f_rest_{j}" for j in range(3 * K)] + ["opacity", "scale_0", "scale_1", "scale_2",
                                                      "rot_0", "rot_1", "rot_2", "rot_3"])


def write_ply(path, params, sh_degree):
    """params: planar [P][n] (mean 0-2, log-scales 3-5, quaternion 6-9, logit 10, DC 11-13,
    then band k of channel c at 14 + 3 (k - 1) + c)."""
    p = np.asarray(params, dtype=np.float64)
    P, n = p.shape
    if P != _num_planes(sh_degree):
        raise ValueError(f"{P} planes do not match SH degree {sh_degree}")
    K = (sh_degree + 1) ** 2 - 1
    names = _fields(sh_degree)
    rec = np.zeros(n, dtype=[(name, "<f4") for name in names])
    for a, name in enumerate("xyz"):
        rec[name] = p[a]
    for c in range(3):
        rec[f"f_dc_{c}"] = (p[11 + c] - 0.5) / C0
        for k in range(1, K + 1):
            rec[f"f_rest_{c * K + k - 1}"] = p[14 + 3 * (k - 1) + c]
    rec["opacity"] = p[10]
    for j in range(3):
        rec[f"scale_{j}"] = p[3 + j]
    for j in range(4):
        rec[f"rot_{j}"] = p[6 + j]
    header = ["ply", "format binary_little_endian 1.0", f"element vertex {n}"]
    header += [f"property float {name}" for name in names]
    header.append("end_header")
    with open(path, "wb") as f:
        f.write(("\n".join(header) + "\n").encode("ascii"))
        f.write(rec.tobytes())


def read_ply(path):
    """Reads a file in the layout write_ply writes; returns (planar float32 params, SH degree)."""
    with open(path, "rb") as f:
        names, n = [], None
        line = f.readline().decode("ascii").strip()
        if line != "ply":
            raise ValueError("not a .ply file")
        while True:
            line = f.readline().decode("ascii").strip()
            if line == "end_header":
                break
            parts = line.split()
            if parts[:2] == ["format", "binary_little_endian"]:
                continue
            if parts[:1] == ["format"]:
                raise ValueError(f"unsupported format: {line}")
            if parts[:2] == ["element", "vertex"]:
                n = int(parts[2])
            elif parts[:2] == ["property", "float"]:
                names.append(parts[2])
            elif parts and parts[0] not in ("comment", "obj_info"):
                raise ValueError(f"unsupported header line: {line}")
        rec = np.frombuffer(f.read(), dtype=[(name, "<f4") for name in names], count=n)
    rest = sum(1 for name in names if name.startswith("f_rest_"))
    K = rest // 3
    deg = int(round(math.sqrt(K + 1))) - 1
    if (deg + 1) ** 2 - 1 != K or names != _fields(deg):
        raise ValueError("unexpected property list")
    p = np.zeros((_num_planes(deg), n), np.float64)
    for a, name in enumerate("xyz"):
        p[a] = rec[name]
    for c in range(3):
        p[11 + c] = rec[f"f_dc_{c}"].astype(np.float64) * C0 + 0.5
        for k in range(1, K + 1):
            p[14 + 3 * (k - 1) + c] = rec[f"f_rest_{c * K + k - 1}"]
    p[10] = rec["opacity"]
    for j in range(3):
        p[3 + j] = rec[f"scale_{j}"]
    for j in range(4):
        p[6 + j] = rec[f"rot_{j}"]
    return p.astype(np.float32), deg
