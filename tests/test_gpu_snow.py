"""GPU parity of the snow material (non-associative Cam-clay plasticity on
Hencky elasticity, merged into P2G and into the fused G2P2G pass): against
the oracle, with the per-step sort and with fused steps, including each
particle's log plastic volume (the hardening state), and at the full size of
the snow workload on sampled outputs.  Initial deformation gradients and
random affine velocity fields drive every case of the return mapping
(compression tip, tension tip, onto the ellipse, unchanged)."""
import numpy as np
import pytest

from material_point_physics_amd import scenes
import oracle
import parity_util as pu
from test_gpu_parity import assert_grid_parity, assert_particle_parity

pytestmark = pytest.mark.gpu

SNOW = dict(snow_M=0.8, snow_beta=0.9, snow_xi=5.0)


def snow_scene(seed, N=20000, n=32, alpha0=-0.01, **kw):
    kw.setdefault("cscale", 8.0)
    kw.setdefault("fstretch", 0.04)
    return scenes.random_scene(N, n, seed, vscale=1.0, material=scenes.SNOW, E=1e4, nu=0.3,
                               snow=dict(SNOW, snow_alpha0=alpha0), **kw)


def _cases_hit(sc):
    """How many particles (of a sample) the oracle sends to each case of the
    return mapping in the first step's G2P: elastic, compression tip,
    tension tip, onto the ellipse."""
    o = oracle.Oracle("f64")
    P = sc.params()
    mu, lam = o.lame(P["E"], P["nu"])
    sim = oracle.OracleSim(sc, "f64")
    a0 = sim.J.copy()
    sim.p2g()
    sim.grid_update()
    F0 = sim.F.copy()
    sim.g2p()
    trial = (np.eye(3)[None] + P["dt"] * sim.C) @ F0
    kinds = [o.snow_project(trial[p], a0[p], mu, lam, P["snow_M"], P["snow_beta"], P["snow_xi"])[2]
             for p in range(0, sc.N, max(1, sc.N // 3000))]
    return np.bincount(kinds, minlength=4)


def assert_alpha_parity(sc, gpu, orc, steps):
    """The log plastic volume within ten times the fp32 oracle's distance
    from the fp64 oracle (2e-6 at least)."""
    f32 = pu.oracle_run(sc, steps, "f32")
    env = float(np.abs(f32.J.astype(np.float64) - orc.J).max())
    err = float(np.abs(gpu["alpha"].astype(np.float64) - orc.J).max())
    pu.log(f"{sc.name}: log plastic volume err {err:.3e} (fp32 oracle {env:.3e}); "
           f"range [{orc.J.min():.4f}, {orc.J.max():.4f}]")
    assert err <= max(10 * env, 2e-6)


CASES = {
    "strained_5": (lambda: snow_scene(91), 5, None, False),
    "hardened_4": (lambda: snow_scene(92, alpha0=-0.05, fstretch=0.1), 4, None, False),
    "soft_3": (lambda: snow_scene(93, alpha0=0.0, fstretch=0.01, cscale=2.0), 3, None, False),
    "strained_fused_never_6": (lambda: snow_scene(94), 6, (1 << 30, 1 << 40), True),
    "strained_fused_every4_9": (lambda: snow_scene(95), 9, (4, 1 << 40), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_snow_matches_oracle(name):
    make, steps, policy, fused = CASES[name]
    sc = make()
    hits = _cases_hit(sc)
    pu.log(f"snow {name}: N={sc.N} steps={steps}; first-step cases "
           f"(elastic, compression tip, tension tip, ellipse) {hits.tolist()}")
    if name.startswith("strained"):
        assert hits[1] > 0 and hits[2] > 0 and hits[3] > 0
    if name.startswith("hardened"):  # a wide ellipse: mostly elastic, the rest onto its surface
        assert hits[0] > hits[3] > 0
    gpu = pu.gpu_run(sc, steps, sort_policy=policy, fused=fused)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(1e-5, 20 * env["v"]))
    assert_alpha_parity(sc, gpu, orc, steps)
    assert gpu["status"][0] & ~np.uint32(0x2) == 0  # no inversion, non-finite or convergence flag


def test_snow_state_before_any_step_and_arguments():
    """Before any step the log plastic volume reads back as snow_alpha0; a
    per-particle modulus is refused for snow, and the plastic-state readback
    for another material."""
    import torch
    import material_point_physics_amd as mpm
    sc = snow_scene(96, N=3000, alpha0=-0.02)
    sim = mpm.Simulation(sc)
    try:
        a = sim.read_plastic_state().cpu().numpy()
        assert np.all(a == np.float32(-0.02))
    finally:
        sim.close()
    sc_e = snow_scene(97, N=1000)
    sc_e.E_p = np.full(sc_e.N, 1e4, np.float32)
    with pytest.raises(mpm.MpmError) as ei:
        mpm.Simulation(sc_e)
    assert ei.value.code == mpm.MPM_ERR_INVALID_ARG
    el = scenes.random_scene(1000, 16, 98)
    sim = mpm.Simulation(el)
    try:
        out = torch.empty(el.N, dtype=torch.float32, device=sim.device)
        with pytest.raises(mpm.MpmError) as ei:
            mpm.mpm_read_plastic_state(sim.handle, out, sim.stream)
        assert ei.value.code == mpm.MPM_ERR_INVALID_ARG
    finally:
        sim.close()


def test_snow_full_size_sampled():
    """The 1.31M-particle snow block at its full size, here moving down at
    20 m/s (ten times the workload's 2 m/s, so that its bottom layer passes
    the compression tip within three steps), three steps: sampled particles
    (F and log plastic volume after the readback's projection) against the
    oracle on their neighbourhood, including particles of the bottom
    half-cell, and the total mass."""
    import dataclasses
    sc = scenes.snow_1m()
    sc = dataclasses.replace(sc, v=(sc.v * 10).astype(np.float32))
    steps = 3
    pu.log(f"full-size snow_1m at 20 m/s: N={sc.N} n={sc.n} steps={steps}")
    gpu = pu.gpu_run(sc, steps)
    rng = np.random.default_rng(2026)
    bottom = np.nonzero(sc.x[:, 1] < 3.5 / sc.n)[0]
    sample = np.concatenate([rng.choice(sc.N, 32, replace=False), rng.choice(bottom, 16, replace=False)])
    idx = pu.neighbourhood(sc.x, sc.x[sample], sc.n, 6)
    sub = pu.subset_scene(sc, idx)
    orc = pu.oracle_run(sub, steps)
    pos = {int(g): k for k, g in enumerate(idx)}
    ks = np.array([pos[int(p)] for p in sample])
    vs = max(np.abs(orc.v[ks]).max(), 1e-30)
    ex = np.abs(gpu["x"][sample] - orc.x[ks]).max()
    ev = np.abs(gpu["v"][sample] - orc.v[ks]).max() / vs
    eF = np.abs(gpu["F"][sample] - orc.F[ks]).max()
    ea = np.abs(gpu["alpha"][sample] - orc.J[ks]).max()
    moved = int(np.sum(orc.J[ks] != np.float32(-0.01)))
    pu.log(f"snow_1m sampled particles: x {ex:.2e} v {ev:.2e} F {eF:.2e} alpha {ea:.2e}; "
           f"{moved} of {len(ks)} hardened or softened")
    assert moved > 0
    assert ex < 1e-6 and ev < 1e-4 and eF < 1e-5 and ea < 1e-5
    m_p = np.float64(sc.params()["rho"]) * sc.params()["p_vol"]
    assert abs(gpu["m"].astype(np.float64).sum() - m_p * sc.N) / (m_p * sc.N) < 1e-6
