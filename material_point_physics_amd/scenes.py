"""Seeded synthetic scenes (inputs only).

This module produces particle positions, velocities, per-particle stiffness
and the scalar parameters of each workload.  It holds none of the MPM step's
arithmetic: it is shared by the HIP path, the oracle-based tests and the
benchmark purely as an input source, so that both sides see bit-identical
float32 inputs.

The workloads stand in for the scenes of "Principles towards Real-Time
Simulation of Material Point Method on Modern GPUs" (real-time 55K-particle
and offline 12M-particle scenes in its introduction and results; the dense
27-particles-per-cell fountain source in its Fountain results).  Those scenes
need assets and material models that are not available, so seeded synthetic
bodies of the stated particle counts, grids and materials replace them.

Conventions: domain [0,1]^3, grid of ``n`` nodes per axis at i*dx with
dx = 1/n, y is up, gravity (0, -9.8, 0), sticky walls 3 nodes thick,
rho = 1, initial C = 0 and F = I (J = 1).  Every scene is generated in
float64 from ``numpy.random.default_rng(seed)`` and rounded once to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

FIXED_COROTATED = 0
J_FLUID = 1
SAND = 2
SNOW = 3


@dataclass
class Scene:
    name: str
    description: str
    x: np.ndarray                 # (N,3) float32
    v: np.ndarray                 # (N,3) float32
    E_p: Optional[np.ndarray]     # (N,) float32 per-particle Young's modulus, or None
    n: int                        # grid nodes per axis
    dt: float
    gravity: tuple
    wall: int
    material: int
    E: float                      # Young's modulus (bulk modulus K for J_FLUID)
    nu: float
    rho: float
    p_vol: float                  # initial particle volume V0
    steps: int
    C: Optional[np.ndarray] = None   # (N,3,3) float32 initial affine matrix (None -> 0)
    F: Optional[np.ndarray] = None   # (N,3,3) float32 initial deformation gradient (None -> I)
    J: Optional[np.ndarray] = None   # (N,) float32 initial volume ratio (None -> 1)
    extra: dict = field(default_factory=dict)
    friction_deg: float = 30.0       # SAND: friction angle in degrees
    snow_M: float = 0.8              # SNOW: critical-state slope M (friction)
    snow_beta: float = 0.9           # SNOW: cohesion beta
    snow_xi: float = 5.0             # SNOW: hardening xi
    snow_alpha0: float = -0.01       # SNOW: initial log plastic volume ln J_P

    @property
    def N(self) -> int:
        return int(self.x.shape[0])

    def params(self) -> dict:
        """Scalar parameters rounded to float32 exactly as the C ABI receives them."""
        f32 = lambda a: float(np.float32(a))
        return dict(n=int(self.n), dt=f32(self.dt),
                    gravity=tuple(f32(g) for g in self.gravity),
                    wall=int(self.wall), material=int(self.material),
                    E=f32(self.E), nu=f32(self.nu), rho=f32(self.rho),
                    p_vol=f32(self.p_vol), friction_deg=f32(self.friction_deg),
                    snow_M=f32(self.snow_M), snow_beta=f32(self.snow_beta),
                    snow_xi=f32(self.snow_xi), snow_alpha0=f32(self.snow_alpha0))


def _stratified(rng, cells: np.ndarray, ppc: int, dx: float) -> np.ndarray:
    """ppc points uniformly at random inside each of the given cells (cell-major order)."""
    cells = np.asarray(cells, dtype=np.float64)
    jit = rng.random((cells.shape[0], ppc, 3))
    pts = (cells[:, None, :] + jit) * dx
    return pts.reshape(-1, 3)


def _box_cells(lo, hi) -> np.ndarray:
    """All integer cells c with lo <= c < hi componentwise, x fastest."""
    zs, ys, xs = np.meshgrid(np.arange(lo[2], hi[2]), np.arange(lo[1], hi[1]),
                             np.arange(lo[0], hi[0]), indexing="ij")
    return np.stack([xs.ravel(), ys.ravel(), zs.ravel()], axis=1)


def cube_8k(seed: int = 1) -> Scene:
    """8,192 particles in an elastic cube of side 0.25 on a 32^3 grid.

    The cube is 8^3 cells (x,z in [0.375,0.625], y in [0.5,0.75]); 16 particles
    per cell keep the stated count (8 per cell would give 4,096).
    """
    n = 32
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    cells = _box_cells((12, 16, 12), (20, 24, 20))
    x = _stratified(rng, cells, 16, dx)
    N = x.shape[0]
    return Scene("cube_8k", "elastic cube, 8192 particles, 32^3 grid",
                 x.astype(np.float32), np.zeros((N, 3), np.float32), None,
                 n=n, dt=1e-4, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=FIXED_COROTATED, E=1e4, nu=0.2, rho=1.0,
                 p_vol=0.25 ** 3 / N, steps=10)


def jelly3_55k(seed: int = 2) -> Scene:
    """55,000 particles in three jelly spheres (radius 0.08) on a 64^3 grid.

    Centres are uniform in [0.2,0.8]^3, redrawn until every pair is at least
    2r + 2dx apart; points are uniform in each ball; each sphere gets one
    velocity drawn uniformly from [-1,1]^3.
    """
    n = 64
    dx = 1.0 / n
    r = 0.08
    rng = np.random.default_rng(seed)
    while True:
        c = rng.uniform(0.2, 0.8, size=(3, 3))
        d = np.linalg.norm(c[:, None, :] - c[None, :, :], axis=-1)
        if np.all(d[np.triu_indices(3, 1)] >= 2 * r + 2 * dx):
            break
    counts = [18334, 18333, 18333]
    xs, vs = [], []
    for k in range(3):
        m = counts[k]
        dirs = rng.normal(size=(m, 3))
        dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
        rad = r * rng.random(m) ** (1.0 / 3.0)
        xs.append(c[k] + dirs * rad[:, None])
        vel = rng.uniform(-1.0, 1.0, size=3)
        vs.append(np.broadcast_to(vel, (m, 3)))
    x = np.concatenate(xs)
    v = np.concatenate(vs)
    N = x.shape[0]
    vol = 3 * (4.0 / 3.0) * np.pi * r ** 3
    return Scene("jelly3_55k", "three jelly spheres, 55000 particles, 64^3 grid",
                 x.astype(np.float32), v.astype(np.float32), None,
                 n=n, dt=5e-5, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=FIXED_COROTATED, E=5e3, nu=0.3, rho=1.0,
                 p_vol=vol / N, steps=200)


def blocks_1m(seed: int = 3, gravity: bool = True) -> Scene:
    """1,024,000 particles in two elastic blocks colliding at +-2 m/s, 128^3 grid.

    Blocks are 40^3 cells (side 0.3125, nearest to 0.3 at about 1M particles)
    at x-cells [24,64) and [65,105), y and z cells [44,84); 8 particles per cell.
    """
    n = 128
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    a = _stratified(rng, _box_cells((24, 44, 44), (64, 84, 84)), 8, dx)
    b = _stratified(rng, _box_cells((65, 44, 44), (105, 84, 84)), 8, dx)
    x = np.concatenate([a, b])
    v = np.zeros_like(x)
    v[: a.shape[0], 0] = 2.0
    v[a.shape[0]:, 0] = -2.0
    N = x.shape[0]
    g = (0.0, -9.8, 0.0) if gravity else (0.0, 0.0, 0.0)
    return Scene("blocks_1m", "two colliding elastic blocks, 1024000 particles, 128^3 grid",
                 x.astype(np.float32), v.astype(np.float32), None,
                 n=n, dt=2e-5, gravity=g, wall=3,
                 material=FIXED_COROTATED, E=1e5, nu=0.3, rho=1.0,
                 p_vol=dx ** 3 / 8, steps=100)


def slab_12m(seed: int = 4, N: int = 12_000_000) -> Scene:
    """12M particles filling the lower 40% of a 256^3 grid, heterogeneous stiffness.

    Positions are i.i.d. uniform in x,z in [3dx, 1-3dx], y in [3dx, 0.4]
    (about 1.93 particles per cell); E is log-uniform in [1e3, 1e5] per
    particle, nu = 0.25.
    """
    n = 256
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    lo = np.array([3 * dx, 3 * dx, 3 * dx])
    hi = np.array([1 - 3 * dx, 0.4, 1 - 3 * dx])
    x = lo + (hi - lo) * rng.random((N, 3))
    E_p = 10.0 ** rng.uniform(3.0, 5.0, size=N)
    vol = float(np.prod(hi - lo))
    return Scene("slab_12m", "heterogeneous elastic slab, 12M particles, 256^3 grid",
                 x.astype(np.float32), np.zeros((N, 3), np.float32), E_p.astype(np.float32),
                 n=n, dt=1e-5, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=FIXED_COROTATED, E=1e4, nu=0.25, rho=1.0,
                 p_vol=vol / N, steps=50)


def slab_12m_shard8(part: int = 3, parts: int = 8) -> Scene:
    """One GPU's share of the 12M slab split over 8 GPUs: the particles of
    slab_12m whose initial x lies in the part-th of 8 equal ranges of the
    slab's x extent (static partition by initial position, about 1.5M
    particles in a slab about 31 nodes thick), on the same 256^3 grid.  Part 3
    is an interior piece: both of its x faces border another piece."""
    full = slab_12m()
    dx = 1.0 / full.n
    lo, hi = 3 * dx, 1 - 3 * dx
    w = (hi - lo) / parts
    x0 = full.x[:, 0].astype(np.float64)
    keep = (x0 >= lo + part * w) & (x0 < lo + (part + 1) * w)
    return Scene(f"slab_12m_shard{parts}", f"piece {part} of {parts} of the 12M slab (x partition), "
                 f"{int(keep.sum())} particles, 256^3 grid",
                 np.ascontiguousarray(full.x[keep]), np.ascontiguousarray(full.v[keep]),
                 np.ascontiguousarray(full.E_p[keep]),
                 n=full.n, dt=full.dt, gravity=full.gravity, wall=full.wall, material=full.material,
                 E=full.E, nu=full.nu, rho=full.rho, p_vol=full.p_vol, steps=full.steps)


def dambreak_4m(seed: int = 5) -> Scene:
    """4,000,000 particles of weakly compressible fluid in a corner column, 256^3 grid.

    The column is 50x100x50 cells (x,z cells [3,53), y cells [3,103)) with 16
    particles per cell: this keeps the stated count, per-cell density, grid
    and the 1:2:1 aspect.  Bulk modulus K = 400.
    """
    n = 256
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    x = _stratified(rng, _box_cells((3, 3, 3), (53, 103, 53)), 16, dx)
    N = x.shape[0]
    return Scene("dambreak_4m", "weakly compressible dam break, 4M particles, 256^3 grid",
                 x.astype(np.float32), np.zeros((N, 3), np.float32), None,
                 n=n, dt=1e-5, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=J_FLUID, E=400.0, nu=0.0, rho=1.0,
                 p_vol=dx ** 3 / 16, steps=100)


def sand_3m(seed: int = 6) -> Scene:
    """3,112,960 particles in a sand column collapsing under gravity, 128^3 grid.

    Stands in for the page's falling-sand scene (3.1M particles): a column of
    64 x 95 x 64 cells (x and z cells [32,96), y cells [4,99), resting on the
    floor's wall layer), 8 particles per cell, at rest; Drucker-Prager sand
    with a 30-degree friction angle.
    """
    n = 128
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    x = _stratified(rng, _box_cells((32, 4, 32), (96, 99, 96)), 8, dx)
    v = np.zeros_like(x)
    return Scene("sand_3m", "collapsing sand column, 3112960 particles, 128^3 grid",
                 x.astype(np.float32), v.astype(np.float32), None,
                 n=n, dt=2e-5, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=SAND, E=1e5, nu=0.3, rho=1.0,
                 p_vol=dx ** 3 / 8, steps=100, friction_deg=30.0)


def snow_1m(seed: int = 7) -> Scene:
    """1,310,720 particles of snow falling onto the floor, 128^3 grid.

    Stands in for the page's snow scene (1.33M particles of non-associative
    Cam-clay snow with bulk modulus 5e5, Poisson ratio 0.3, M = 0.8,
    beta = 0.9, xi = 5; its animated crawling-figure boundary is not
    available): a block of 64 x 40 x 64 cells (x and z cells [32,96), y cells
    [3,43), so the bottom layer's stencils reach the sticky floor), 8
    particles per cell, moving down at 2 m/s.  E = 3 K (1 - 2 nu) = 6e5 gives
    the page's bulk modulus; density 400 (fresh snow; the page gives none);
    initial log plastic volume -0.01 (the page gives none).
    """
    n = 128
    dx = 1.0 / n
    rng = np.random.default_rng(seed)
    x = _stratified(rng, _box_cells((32, 3, 32), (96, 43, 96)), 8, dx)
    v = np.zeros_like(x)
    v[:, 1] = -2.0
    return Scene("snow_1m", "snow block falling onto the floor, 1310720 particles, 128^3 grid",
                 x.astype(np.float32), v.astype(np.float32), None,
                 n=n, dt=2e-5, gravity=(0.0, -9.8, 0.0), wall=3,
                 material=SNOW, E=6e5, nu=0.3, rho=400.0,
                 p_vol=dx ** 3 / 8, steps=100, snow_M=0.8, snow_beta=0.9, snow_xi=5.0,
                 snow_alpha0=-0.01)


SCENES = {
    "cube_8k": cube_8k,
    "jelly3_55k": jelly3_55k,
    "blocks_1m": blocks_1m,
    "slab_12m": slab_12m,
    "slab_12m_shard8": slab_12m_shard8,
    "dambreak_4m": dambreak_4m,
    "sand_3m": sand_3m,
    "snow_1m": snow_1m,
}


def clamp_scene(seed: int = 17, n: int = 32, dt: float = 1e-3, per_cluster: int = 300) -> Scene:
    """Four clusters of particles on a grid without walls and without gravity,
    each cluster moving at one uniform velocity (so that the grid reproduces
    it exactly), for tests of the position clamp to [2dx, (n-2)dx].

    Cluster 0 lies against the low x clamp plane (x in [2dx, 2.4dx]) and
    moves -x by 0.6 dx per step; cluster 1 lies against the high y plane and
    moves +y by 0.6 dx per step (and +x by 0.1 dx); cluster 2 lies in the
    corner at low x, low y and high z and moves out through all three planes;
    cluster 3 is interior and never reaches a plane.  The clusters are more
    than 3 cells apart, so they share no grid node.  extra["cluster"] holds
    each particle's cluster and extra["clamped_per_step"] the number of
    position components that leave the box in each step (clusters 0 and 1:
    one per particle, cluster 2: three, cluster 3: none).
    """
    rng = np.random.default_rng(seed)
    dx = 1.0 / n
    lo_p, hi_p = 2 * dx, (n - 2) * dx
    u = 0.6 * dx / dt
    boxes = [
        ((lo_p, 0.35, 0.35), (lo_p + 0.4 * dx, 0.5, 0.5), (-u, 0.0, 0.0)),
        ((0.55, hi_p - 0.4 * dx, 0.55), (0.7, hi_p, 0.7), (u / 6, u, 0.0)),
        ((lo_p, lo_p, hi_p - 0.4 * dx), (lo_p + 0.4 * dx, lo_p + 0.4 * dx, hi_p), (-u, -u, u)),
        ((0.4, 0.4, 0.45), (0.55, 0.55, 0.6), (0.3 * u, -0.2 * u, 0.1 * u)),
    ]
    xs, vs, cl = [], [], []
    for k, (lo, hi, vel) in enumerate(boxes):
        lo, hi = np.asarray(lo), np.asarray(hi)
        xs.append(lo + (hi - lo) * rng.random((per_cluster, 3)))
        vs.append(np.tile(np.asarray(vel, np.float64), (per_cluster, 1)))
        cl.append(np.full(per_cluster, k, np.int32))
    x = np.concatenate(xs)
    v = np.concatenate(vs)
    return Scene("clamp_faces", "four clusters leaving the clamp box through its faces",
                 x.astype(np.float32), v.astype(np.float32), None,
                 n=n, dt=dt, gravity=(0.0, 0.0, 0.0), wall=0,
                 material=FIXED_COROTATED, E=100.0, nu=0.3, rho=1.0,
                 p_vol=dx ** 3 / 4, steps=3,
                 extra={"cluster": np.concatenate(cl), "clamped_per_step": 5 * per_cluster})


def random_rotation(rng, m: int) -> np.ndarray:
    """m uniformly random rotations (QR of Gaussian matrices, det fixed to +1)."""
    a = rng.normal(size=(m, 3, 3))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diagonal(r, axis1=1, axis2=2))[:, None, :]
    det = np.linalg.det(q)
    q[det < 0, :, 0] *= -1.0
    return q


def random_scene(N: int, n: int, seed: int, *, lo=None, hi=None, vscale=1.0,
                 cscale=0.0, fstretch=0.0, material=FIXED_COROTATED,
                 per_particle_E=False, dt=1e-4, gravity=(0.0, -9.8, 0.0),
                 wall=3, E=1e4, nu=0.3, rho=1.0, friction_deg=30.0,
                 snow=None) -> Scene:
    """A generic seeded scene for parity and edge-case tests.

    Positions are i.i.d. uniform in the box [lo, hi] (default: the region
    whose particles keep their whole stencil off the clamp, [3dx, 1-3dx]^3);
    velocities uniform in [-vscale, vscale]; when cscale > 0 an initial C with
    entries uniform in [-cscale, cscale]; when fstretch > 0 an initial
    F = R diag(s) Q^T with random rotations and stretches s in
    [1-fstretch, 1+fstretch] (for J_FLUID: J = product of s).  snow: a dict
    of Scene's snow_* fields to override (material SNOW).
    """
    rng = np.random.default_rng(seed)
    dx = 1.0 / n
    lo = np.full(3, 3 * dx) if lo is None else np.asarray(lo, np.float64)
    hi = np.full(3, 1 - 3 * dx) if hi is None else np.asarray(hi, np.float64)
    x = lo + (hi - lo) * rng.random((N, 3))
    v = rng.uniform(-vscale, vscale, size=(N, 3))
    C = F = J = None
    if cscale > 0:
        C = rng.uniform(-cscale, cscale, size=(N, 3, 3)).astype(np.float32)
    if fstretch > 0:
        s = rng.uniform(1 - fstretch, 1 + fstretch, size=(N, 3))
        if material == J_FLUID:
            J = np.prod(s, axis=1).astype(np.float32)
        else:
            R = random_rotation(rng, N)
            Q = random_rotation(rng, N)
            F = (R * s[:, None, :]) @ np.transpose(Q, (0, 2, 1))
            F = F.astype(np.float32)
    E_p = None
    if per_particle_E:
        E_p = (E * 10.0 ** rng.uniform(-1.0, 1.0, size=N)).astype(np.float32)
    return Scene(f"random_{N}_{n}_{seed}", "random test scene",
                 x.astype(np.float32), v.astype(np.float32), E_p,
                 n=n, dt=dt, gravity=tuple(gravity), wall=wall, material=material,
                 E=E, nu=nu, rho=rho, p_vol=dx ** 3 / 4, steps=1, C=C, F=F, J=J,
                 friction_deg=friction_deg, **(snow or {}))
