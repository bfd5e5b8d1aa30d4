"""Seeded synthetic inputs for the ball-tree / ball-attention / BSA workloads.

This module only draws random numbers and shapes them into point clouds and
feature tensors.  It contains none of the method's arithmetic (no tree, no
attention, no pooling), so both the CPU oracle and the GPU path may consume its
arrays.  Every generator uses ``numpy.random.default_rng(seed)`` (PCG64) with a
fixed draw order: coordinates first, then q, k, v, then any gate weights.

Workloads (sizes and distributions):

* ``uniform_cube``  -- points uniform in [0,1]^3.
* ``deformed_sphere`` -- surface of a unit sphere whose radius is modulated by
  eight random real spherical harmonics of degree 1..3 (amplitude 0.2), plus
  N(0, 0.01^2) jitter; a stand-in for a car-surface point cloud such as the
  ShapeNet-Car surfaces the BSA paper measures on (Pith review of
  arXiv 2506.12541, Figure 2 caption and Figure 3 sweep to length 65,536).
* ``gaussian_mixture`` -- 256 isotropic clusters in [0,100]^3 with
  log-uniform widths in [0.5, 5] and Dirichlet(1) weights; a stand-in for the
  large cosmology clouds of the Erwin thread (Bluesky, posts 11/N and 12/N).
* ``box_4x1x1`` -- points uniform in [0,4]x[0,1]x[0,1], used for the rotated
  tree pair.
* ``random_rotation`` -- a uniform random rotation from a normalised 4-D
  Gaussian quaternion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# point clouds
# ---------------------------------------------------------------------------


def uniform_cube(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.random((n, 3)).astype(np.float32)


def _real_sh(l: int, m: int, x, y, z):
    """Real orthonormal spherical harmonic Y_lm on the unit sphere, l <= 3."""
    pi = math.pi
    if l == 1:
        c = math.sqrt(3.0 / (4 * pi))
        return c * {-1: y, 0: z, 1: x}[m]
    if l == 2:
        if m == -2:
            return 0.5 * math.sqrt(15 / pi) * x * y
        if m == -1:
            return 0.5 * math.sqrt(15 / pi) * y * z
        if m == 0:
            return 0.25 * math.sqrt(5 / pi) * (3 * z * z - 1)
        if m == 1:
            return 0.5 * math.sqrt(15 / pi) * x * z
        return 0.25 * math.sqrt(15 / pi) * (x * x - y * y)
    if l == 3:
        if m == -3:
            return 0.25 * math.sqrt(35 / (2 * pi)) * y * (3 * x * x - y * y)
        if m == -2:
            return 0.5 * math.sqrt(105 / pi) * x * y * z
        if m == -1:
            return 0.25 * math.sqrt(21 / (2 * pi)) * y * (5 * z * z - 1)
        if m == 0:
            return 0.25 * math.sqrt(7 / pi) * z * (5 * z * z - 3)
        if m == 1:
            return 0.25 * math.sqrt(21 / (2 * pi)) * x * (5 * z * z - 1)
        if m == 2:
            return 0.25 * math.sqrt(105 / pi) * z * (x * x - y * y)
        return 0.25 * math.sqrt(35 / (2 * pi)) * x * (x * x - 3 * y * y)
    raise ValueError(l)


def deformed_sphere(rng: np.random.Generator, n: int, n_terms: int = 8,
                    amp: float = 0.2, jitter: float = 0.01) -> np.ndarray:
    ls = rng.integers(1, 4, size=n_terms)
    ms = np.array([rng.integers(-l, l + 1) for l in ls])
    signs = rng.choice(np.array([-1.0, 1.0]), size=n_terms)
    g = rng.standard_normal((n, 3))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    x, y, z = u[:, 0], u[:, 1], u[:, 2]
    r = np.ones(n)
    for l, m, s in zip(ls, ms, signs):
        r += amp * s * _real_sh(int(l), int(m), x, y, z)
    r = np.maximum(r, 0.1)
    pts = r[:, None] * u + jitter * rng.standard_normal((n, 3))
    return pts.astype(np.float32)


def gaussian_mixture(rng: np.random.Generator, n: int, k: int = 256,
                     box: float = 100.0, sig_lo: float = 0.5,
                     sig_hi: float = 5.0) -> np.ndarray:
    centres = rng.random((k, 3)) * box
    sig = np.exp(rng.uniform(math.log(sig_lo), math.log(sig_hi), size=k))
    w = rng.dirichlet(np.ones(k))
    counts = rng.multinomial(n, w)
    comp = np.repeat(np.arange(k), counts)
    pts = centres[comp] + sig[comp, None] * rng.standard_normal((n, 3))
    order = rng.permutation(n)          # unordered cloud: shuffle the points
    return pts[order].astype(np.float32)


def box_4x1x1(rng: np.random.Generator, n: int) -> np.ndarray:
    return (rng.random((n, 3)) * np.array([4.0, 1.0, 1.0])).astype(np.float32)


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random rotation (fp32, row-major 3x3) from a unit quaternion."""
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    a, b, c, d = q
    R = np.array([
        [a * a + b * b - c * c - d * d, 2 * (b * c - a * d), 2 * (b * d + a * c)],
        [2 * (b * c + a * d), a * a - b * b + c * c - d * d, 2 * (c * d - a * b)],
        [2 * (b * d - a * c), 2 * (c * d + a * b), a * a - b * b - c * c + d * d],
    ])
    return R.astype(np.float32)


# ---------------------------------------------------------------------------
# features
# ---------------------------------------------------------------------------


def normal_features(rng: np.random.Generator, n: int, h: int, d: int,
                    dtype: str):
    """One [n, h, d] tensor of N(0,1) draws as a CPU torch tensor.

    fp32 draws; for ``bf16`` they are rounded to nearest-even by torch.
    """
    import torch
    x = torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32))
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    coords: np.ndarray                    # [N,3] fp32, original order
    q: "object" = None                    # torch CPU [N,H,d]
    k: "object" = None
    v: "object" = None
    leaf: int = 0
    ball: int = 0
    H: int = 0
    d: int = 0
    dtype: str = "bf16"
    R: np.ndarray | None = None           # rotation for the second tree
    gate_w: np.ndarray | None = None      # [3,d] fp32
    extra: dict = field(default_factory=dict)


def make(name: str, n: int | None = None, seed: int | None = None,
         features: bool = True) -> Workload:
    """Build one named workload.

    ``n`` overrides the point count (for scaled-down parity cases); the
    distribution and the draw order stay the same.
    """
    if name == "tiny":                       # N=1,024 cube, leaf=ball 32, fp32
        n = n or 1024
        rng = np.random.default_rng(0 if seed is None else seed)
        c = uniform_cube(rng, n)
        w = Workload(name, c, leaf=32, ball=32, H=4, d=16, dtype="f32")
    elif name == "sphere":                   # N=65,536 deformed sphere, ball 128
        n = n or 65536
        rng = np.random.default_rng(2 if seed is None else seed)
        c = deformed_sphere(rng, n)
        w = Workload(name, c, leaf=128, ball=128, H=8, d=32, dtype="bf16")
    elif name == "cosmo":                    # N=1,048,576 mixture, ball 256
        n = n or 1048576
        rng = np.random.default_rng(3 if seed is None else seed)
        c = gaussian_mixture(rng, n)
        w = Workload(name, c, leaf=256, ball=256, H=8, d=32, dtype="bf16")
    elif name == "rotpair":                  # N=262,144 4x1x1 box + rotation
        n = n or 262144
        rng = np.random.default_rng(4 if seed is None else seed)
        c = box_4x1x1(rng, n)
        R = random_rotation(rng)
        w = Workload(name, c, leaf=128, ball=128, H=8, d=32, dtype="bf16", R=R)
    elif name == "bsa":                      # the sphere draws + gate weights
        n = n or 65536
        rng = np.random.default_rng(2 if seed is None else seed)
        c = deformed_sphere(rng, n)
        w = Workload(name, c, leaf=64, ball=128, H=8, d=32, dtype="bf16")
        w.extra = dict(block=64, group=64, topk=16, mask_own_ball=1)
    else:
        raise ValueError(name)
    if features:
        w.q = normal_features(rng, n, w.H, w.d, w.dtype)
        w.k = normal_features(rng, n, w.H, w.d, w.dtype)
        w.v = normal_features(rng, n, w.H, w.d, w.dtype)
        if name == "bsa":
            w.gate_w = (0.02 * rng.standard_normal((3, w.d))).astype(np.float32)
    return w
