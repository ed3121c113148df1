"""GPU parity of the sand material (Drucker-Prager plasticity merged into
P2G, and into the fused G2P2G pass): against the oracle, with the per-step
sort, with fused steps, and at the full size of the sand workload on
sampled outputs.  Initial deformation gradients outside the cone, random
affine velocity fields and an expanding field drive every case of the
return mapping (tip, surface, unchanged)."""
import numpy as np
import pytest

from material_point_physics_amd import scenes
import oracle
import parity_util as pu
from test_gpu_parity import assert_grid_parity, assert_particle_parity

pytestmark = pytest.mark.gpu


def sand_scene(seed, N=20000, n=32, **kw):
    kw.setdefault("cscale", 8.0)
    kw.setdefault("fstretch", 0.04)
    return scenes.random_scene(N, n, seed, vscale=1.0, material=scenes.SAND, E=1e4, nu=0.3,
                               friction_deg=30.0, **kw)


def expanding(seed):
    sc = sand_scene(seed, cscale=0.0, fstretch=0.0)
    sc.C = np.tile(30.0 * np.eye(3, dtype=np.float32), (sc.N, 1, 1))
    return sc


def _cases_hit(sc, steps):
    """How many particles the oracle projects to the tip / onto the surface
    in the first step's G2P (to show that the case ran)."""
    o = oracle.Oracle("f64")
    sim = oracle.OracleSim(sc, "f64")
    sim.p2g()
    sim.grid_update()
    F0 = sim.F.copy()
    sim.g2p()
    G = np.eye(3)[None] + sc.params()["dt"] * sim.C
    trial = G @ F0
    alpha = o.sand_alpha(sc.friction_deg)
    kinds = [o.sand_project(trial[p], sc.nu, alpha)[1] for p in range(0, sc.N, max(1, sc.N // 2000))]
    return np.bincount(kinds, minlength=3)


CASES = {
    "strained_5": (lambda: sand_scene(81), 5, None, False),
    "strained_E_p_4": (lambda: sand_scene(82, per_particle_E=True), 4, None, False),
    "expanding_3": (lambda: expanding(83), 3, None, False),
    "strained_fused_never_6": (lambda: sand_scene(84), 6, (1 << 30, 1 << 40), True),
    "strained_fused_every4_9": (lambda: sand_scene(85), 9, (4, 1 << 40), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sand_matches_oracle(name):
    make, steps, policy, fused = CASES[name]
    sc = make()
    hits = _cases_hit(sc, steps)
    pu.log(f"sand {name}: N={sc.N} steps={steps}; first-step cases (unchanged, tip, surface) {hits.tolist()}")
    if name.startswith("expanding"):
        assert hits[1] > 0
    else:
        assert hits[2] > 0
    gpu = pu.gpu_run(sc, steps, sort_policy=policy, fused=fused)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(1e-5, 20 * env["v"]))
    assert gpu["status"][0] & ~np.uint32(0x2) == 0  # no inversion, non-finite or convergence flag


def test_sand_full_size_sampled():
    """The 3.1M-particle sand column, one step: sampled particles (whose F the
    readback projects) and grid nodes against the oracle on their
    neighbourhood, and the total mass."""
    sc = scenes.sand_3m()
    pu.log(f"full-size sand_3m: N={sc.N} n={sc.n}")
    gpu = pu.gpu_run(sc, 1)
    rng = np.random.default_rng(2025)
    sample = rng.choice(sc.N, 48, replace=False)
    idx = pu.neighbourhood(sc.x, sc.x[sample], sc.n, 4)
    sub = pu.subset_scene(sc, idx)
    orc = pu.oracle_run(sub, 1)
    pos = {int(g): k for k, g in enumerate(idx)}
    ks = np.array([pos[int(p)] for p in sample])
    vs = max(np.abs(orc.v[ks]).max(), 1e-30)
    ex = np.abs(gpu["x"][sample] - orc.x[ks]).max()
    ev = np.abs(gpu["v"][sample] - orc.v[ks]).max() / vs
    eF = np.abs(gpu["F"][sample] - orc.F[ks]).max()
    pu.log(f"sand_3m sampled particles: x {ex:.2e} v {ev:.2e} F {eF:.2e}")
    assert ex < 1e-6 and ev < 1e-4 and eF < 1e-6
    m_p = np.float64(sc.params()["rho"]) * sc.params()["p_vol"]
    assert abs(gpu["m"].astype(np.float64).sum() - m_p * sc.N) / (m_p * sc.N) < 1e-6
