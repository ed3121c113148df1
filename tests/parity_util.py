"""Helpers shared by the GPU parity tests: running the HIP path through the
C ABI, running the oracle, error metrics, and the neighbourhood-subset oracle
used to check sampled outputs at full size.  Holds no MPM arithmetic of its
own beyond selecting particles by distance."""
from __future__ import annotations

import dataclasses
import sys
import time

import numpy as np

import oracle
from material_point_physics_amd import scenes


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def gpu_run(scene, steps: int, read=("particles", "grid"), sort_policy=None, fused=False):
    """Create, step and read back through the C ABI (torch only for memory).
    sort_policy = (max_interval, mover_budget) for mpm_set_sort_policy;
    fused: mpm_set_fused_steps(1)."""
    import material_point_physics_amd as mpm
    sim = mpm.Simulation(scene)
    try:
        if sort_policy is not None:
            sim.set_sort_policy(*sort_policy)
        if fused:
            sim.set_fused_steps(True)
        sim.step(steps)
        out = {}
        if "particles" in read:
            x, v, C, F = sim.read_particles()
            out.update(x=x.cpu().numpy(), v=v.cpu().numpy(), C=C.cpu().numpy(), F=F.cpu().numpy())
        if "particles" in read and scene.material == scenes.SNOW:
            out["alpha"] = sim.read_plastic_state().cpu().numpy()
        if "grid" in read:
            m, p = sim.read_grid()
            out.update(m=m.cpu().numpy(), p=p.cpu().numpy())
        out["status"] = sim.status()
        return out
    finally:
        sim.close()


def oracle_run(scene, steps: int, prec="f64"):
    sim = oracle.OracleSim(scene, prec)
    sim.step(steps)
    return sim


def field_maxrel(gpu, ref):
    """max |gpu - ref| / max |ref| (the grid-parity metric)."""
    ref = np.asarray(ref, np.float64)
    return float(np.abs(np.asarray(gpu, np.float64) - ref).max() / max(np.abs(ref).max(), 1e-300))


def particle_errors(gpu: dict, orc, material: int):
    """Per-field errors normalised by each field's natural scale."""
    vmax = max(np.abs(orc.v).max(), 1e-30)
    cscale = 4 * orc.n * vmax + np.abs(orc.C).max()
    e = dict(
        x=float(np.abs(gpu["x"] - orc.x).max()),
        v=float(np.abs(gpu["v"] - orc.v).max() / vmax),
        C=float(np.abs(gpu["C"] - orc.C).max() / cscale),
    )
    if material == scenes.J_FLUID:
        e["F"] = float(np.abs(gpu["F"] - orc.J).max())
    else:
        e["F"] = float(np.abs(gpu["F"] - orc.F).max())
    return e


def envelope(scene, steps: int):
    """fp32-oracle vs fp64-oracle particle errors: what fp32 arithmetic reaches."""
    a = oracle_run(scene, steps, "f64")
    b = oracle_run(scene, steps, "f32")
    got = dict(x=b.x, v=b.v, C=b.C, F=(b.J if scene.material == scenes.J_FLUID else b.F))
    return a, particle_errors(got, a, scene.material)


def subset_scene(scene, idx):
    """The scene restricted to particles idx (same parameters)."""
    sub = lambda a: None if a is None else np.ascontiguousarray(a[idx])
    return dataclasses.replace(scene, x=sub(scene.x), v=sub(scene.v), E_p=sub(scene.E_p),
                               C=sub(scene.C), F=sub(scene.F), J=sub(scene.J))


def neighbourhood(x: np.ndarray, centres: np.ndarray, n: int, radius_cells: int) -> np.ndarray:
    """Indices of particles whose cell lies within radius_cells (Chebyshev) of
    the cell of any centre."""
    r = int(radius_cells)
    P = n + 2 * r + 2
    def lin(c):
        c = c + r + 1
        return c[..., 0] + P * (c[..., 1] + P * c[..., 2])
    cell = np.floor(x.astype(np.float64) * n).astype(np.int64)
    cc = np.floor(np.asarray(centres, np.float64) * n).astype(np.int64)
    o = np.arange(-r, r + 1)
    offs = np.stack(np.meshgrid(o, o, o, indexing="ij"), -1).reshape(-1, 3)
    near = np.unique(lin(cc[:, None, :] + offs[None, :, :]).ravel())
    return np.nonzero(np.isin(lin(cell), near))[0]
