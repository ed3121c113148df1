"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (fp32 path vs fp64 oracle):
  * grid after one step: per field, max|gpu - oracle| / max|oracle| <= 1e-5;
  * particles after k steps: each field's error, normalised by the field's
    scale (x absolute; v by max|v|; C by 4 n max|v| + max|C|; F, J absolute),
    is at most 10x what the fp32 oracle reaches on the same scene, and never
    required below 2e-6 (float atomics sum in another order, so the GPU is an
    fp32 computation with its own rounding, not the oracle's).
"""
import numpy as np
import pytest

import material_point_physics_amd as mpm
from material_point_physics_amd import scenes
import parity_util as pu

pytestmark = pytest.mark.gpu

GRID_TOL = 1e-5


def particle_tolerance(env: dict) -> dict:
    return {k: max(10.0 * v, 2e-6) for k, v in env.items()}


def assert_grid_parity(scene, gpu, orc, tol=GRID_TOL):
    em = pu.field_maxrel(gpu["m"], orc.grid_mass())
    ep = pu.field_maxrel(gpu["p"], orc.grid_momentum())
    pu.log(f"{scene.name}: grid mass err {em:.3e}, momentum err {ep:.3e}")
    assert em <= tol and ep <= tol


def assert_particle_parity(scene, gpu, orc, env):
    err = pu.particle_errors(gpu, orc, scene.material)
    tol = particle_tolerance(env)
    pu.log(f"{scene.name}: particle err {err} tol {tol}")
    for k in err:
        assert err[k] <= tol[k], (k, err[k], tol[k])


def inverted_F(N, seed, gap):
    """F = U diag(s) V^T with a third of them reflected (det F < 0).  With
    gap=True the singular values are a permutation of (0.75, 1.0, 1.25), so
    the sign-corrected rotation is well conditioned; otherwise they are
    random in [0.7, 1.3] and may nearly coincide."""
    rng = np.random.default_rng(seed)
    U = scenes.random_rotation(rng, N)
    V = scenes.random_rotation(rng, N)
    if gap:
        sv = np.array([rng.permutation([0.75, 1.0, 1.25]) for _ in range(N)])
    else:
        sv = rng.uniform(0.7, 1.3, (N, 3))
    F = (U * sv[:, None, :]) @ np.transpose(V, (0, 2, 1))
    F[::3, :, 0] *= -1
    return F.astype(np.float32)


GRID_SCENES = {
    "cube_8k": scenes.cube_8k,
    "jelly3_55k": scenes.jelly3_55k,
    "blocks_1m": scenes.blocks_1m,
    "strained_E_p": lambda: scenes.random_scene(30000, 32, 41, cscale=20.0, fstretch=0.2, vscale=1.0,
                                                per_particle_E=True),
    "inverted_F": lambda: scenes.random_scene(3000, 32, 47, cscale=5.0, vscale=1.0),
    "fluid_J": lambda: scenes.random_scene(20000, 32, 42, cscale=20.0, fstretch=0.1, vscale=1.0,
                                           material=scenes.J_FLUID, E=400.0),
    "ragged_n20": lambda: scenes.random_scene(4099, 20, 43, cscale=3.0, fstretch=0.1),
    "one_cell_3000": lambda: scenes.random_scene(3000, 32, 44, lo=[0.5] * 3, hi=[0.5 + 1 / 32] * 3,
                                                 vscale=0.5, cscale=2.0),
    "clamp_faces": lambda: scenes.random_scene(2048, 32, 45, lo=[2 / 32] * 3, hi=[30 / 32] * 3, vscale=2.0),
}


@pytest.mark.parametrize("name", list(GRID_SCENES))
def test_grid_after_one_step(name):
    sc = GRID_SCENES[name]()
    if name == "inverted_F":
        sc.F = inverted_F(sc.N, 47, gap=True)
    if name == "clamp_faces":
        # put particles exactly on the clamp planes 2dx and (n-2)dx
        x = sc.x.copy()
        x[:100, 0] = np.float32(2 / 32)
        x[100:200, 1] = np.float32(30 / 32)
        sc.x = x
    pu.log(f"grid parity {name}: N={sc.N} n={sc.n}")
    gpu = pu.gpu_run(sc, 1)
    orc = pu.oracle_run(sc, 1)
    assert_grid_parity(sc, gpu, orc)
    assert gpu["status"][3] == 0  # no non-finite values


def test_inverted_near_degenerate_within_fp32_envelope():
    """Reflected F with close singular values: the sign-corrected rotation is
    ill-conditioned (its axis is determined only to about eps / gap), so the
    tolerance is 10x what the fp32 oracle reaches on the same input."""
    sc = scenes.random_scene(3000, 32, 48, cscale=5.0, vscale=1.0)
    sc.F = inverted_F(sc.N, 48, gap=False)
    pu.log("inverted near-degenerate")
    gpu = pu.gpu_run(sc, 1)
    a = pu.oracle_run(sc, 1, "f64")
    b = pu.oracle_run(sc, 1, "f32")
    env = pu.field_maxrel(b.grid_momentum(), a.grid_momentum())
    err = pu.field_maxrel(gpu["p"], a.grid_momentum())
    pu.log(f"near-degenerate inverted: gpu {err:.3e}, fp32 oracle {env:.3e}")
    assert err <= max(GRID_TOL, 10 * env)
    assert gpu["status"][0] & mpm.MPM_STATUS_INVERTED


PARTICLE_CASES = {
    "cube_8k_10": (scenes.cube_8k, 10),
    "strained_E_p_3": (lambda: scenes.random_scene(20000, 32, 51, cscale=20.0, fstretch=0.2, vscale=1.0,
                                                   per_particle_E=True), 3),
    "fluid_J_3": (lambda: scenes.random_scene(20000, 32, 52, cscale=20.0, fstretch=0.1, vscale=1.0,
                                              material=scenes.J_FLUID, E=400.0), 3),
    "jelly3_55k_5": (scenes.jelly3_55k, 5),
}


@pytest.mark.parametrize("name", list(PARTICLE_CASES))
def test_particles_after_steps(name):
    make, steps = PARTICLE_CASES[name]
    sc = make()
    pu.log(f"particle parity {name}: N={sc.N} n={sc.n} steps={steps}")
    gpu = pu.gpu_run(sc, steps)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(GRID_TOL, 20 * env["v"]))


def test_read_back_before_any_step_is_the_input():
    sc = scenes.random_scene(5000, 32, 60, cscale=3.0, fstretch=0.2, per_particle_E=True)
    pu.log("identity readback")
    gpu = pu.gpu_run(sc, 0)
    assert np.array_equal(gpu["x"], sc.x)
    assert np.array_equal(gpu["v"], sc.v)
    assert np.array_equal(gpu["C"], sc.C)
    # The kernels keep F - I: off-diagonal entries come back exactly, and a
    # diagonal entry within one rounding of F - 1 and one of 1 + (F - 1)
    # (exactly for entries in [0.5, 2], where F - 1 is exact).
    diag = np.broadcast_to(np.eye(3, dtype=bool), sc.F.shape)
    d = np.abs(gpu["F"].astype(np.float64) - sc.F.astype(np.float64))
    assert not d[~diag].any()
    assert np.all(d[diag] <= 2.0 ** -22 * np.maximum(1.0, np.abs(sc.F[diag])))
    inner = diag & (sc.F >= 0.5) & (sc.F <= 2.0)
    assert not d[inner].any()
    assert not gpu["m"].any() and not gpu["p"].any()


def test_empty_and_single_particle():
    pu.log("empty scene")
    sc0 = scenes.random_scene(0, 32, 61)
    g0 = pu.gpu_run(sc0, 3)
    assert g0["x"].shape == (0, 3) and not g0["m"].any()
    pu.log("single particle")
    sc1 = scenes.random_scene(1, 32, 62, cscale=4.0, fstretch=0.2)
    g1 = pu.gpu_run(sc1, 2)
    orc, env = pu.envelope(sc1, 2)
    assert_particle_parity(sc1, g1, orc, env)


@pytest.mark.parametrize("N", [63, 64, 65, 1023, 1024, 1025, 4097])
def test_ragged_particle_counts(N):
    sc = scenes.random_scene(N, 24, 70 + N, cscale=5.0, fstretch=0.15, vscale=1.0)
    pu.log(f"ragged N={N}")
    gpu = pu.gpu_run(sc, 2)
    orc, env = pu.envelope(sc, 2)
    assert_particle_parity(sc, gpu, orc, env)


def test_status_clean_run_and_bad_input():
    sc = scenes.cube_8k()
    pu.log("status words")
    g = pu.gpu_run(sc, 10, read=())
    assert g["status"] == [0] * mpm.MPM_STATUS_WORDS
    bad = scenes.random_scene(500, 32, 63)
    x = bad.x.copy()
    x[7] = np.nan
    x[9, 1] = 0.999
    bad.x = x
    g = pu.gpu_run(bad, 1, read=("particles",))
    assert g["status"][0] & mpm.MPM_STATUS_BAD_INPUT
    assert np.all(np.isfinite(g["x"]))
    lo, hi = 2 / 32, 30 / 32
    assert np.all(g["x"] >= lo) and np.all(g["x"] <= hi)


def test_profiled_steps_match_graph_steps():
    """Eager per-kernel-timed steps run the same kernels as the graph."""
    import torch
    sc = scenes.random_scene(20000, 32, 64, cscale=10.0, fstretch=0.2, vscale=1.0)
    pu.log("profiled vs graph")
    a = mpm.Simulation(sc)
    b = mpm.Simulation(sc)
    try:
        a.step(3)
        ms = mpm.mpm_step_profiled(b.handle, 3, b.stream)
        assert set(ms) == {"k_scan_tiles", "k_scan_bins", "k_scatter", "k_p2g", "k_g2p"}
        # (a grid whose bins fit one scan tile skips k_scan_tiles: about 0 ms)
        assert all(v >= 0 for v in ms.values())
        assert all(ms[k] > 0 for k in ("k_scan_bins", "k_scatter", "k_p2g", "k_g2p"))
        assert mpm.mpm_steps_taken(a.handle) == mpm.mpm_steps_taken(b.handle) == 3
        xa, va, Ca, Fa = a.read_particles()
        xb, vb, Cb, Fb = b.read_particles()
        # float atomics sum in another order, so compare against each field's scale
        for u, w in [(xa, xb), (va, vb), (Ca, Cb), (Fa, Fb)]:
            assert float((u - w).abs().max() / w.abs().max()) < 1e-5
    finally:
        a.close()
        b.close()


def test_batched_graphs_match_single_steps():
    """mpm_step(17) (two 8-step graphs and one single step) against 17 calls of
    mpm_step(1): the same steps, and the same step count.  Two runs differ by
    the order of their float atomics (and of the atomic mover slots), as any
    two runs do, so each field's difference is held to the run-to-run bar of
    test_gpu_lifecycle: the fp32 oracle's own distance from fp64, with the
    parity normalisation (C by 4 n max|v| + max|C|)."""
    sc = scenes.random_scene(20000, 32, 66, cscale=10.0, fstretch=0.2, vscale=1.0)
    pu.log("batched vs single-step graphs")
    a = mpm.Simulation(sc)
    b = mpm.Simulation(sc)
    try:
        a.step(17)
        for _ in range(17):
            b.step(1)
        assert mpm.mpm_steps_taken(a.handle) == mpm.mpm_steps_taken(b.handle) == 17
        ra = [t.cpu().numpy() for t in a.read_particles()]
        rb = [t.cpu().numpy() for t in b.read_particles()]
        ma, pa = a.read_grid()
        mb, pb = b.read_grid()
    finally:
        a.close()
        b.close()
    orc, env = pu.envelope(sc, 17)
    vmax = max(np.abs(orc.v).max(), 1e-30)
    scale = dict(x=1.0, v=vmax, C=4 * sc.n * vmax + np.abs(orc.C).max(), F=1.0)
    for k, u, w in zip(("x", "v", "C", "F"), ra, rb):
        d = float(np.abs(u - w).max() / scale[k])
        pu.log(f"batched vs single {k}: {d:.3e} (fp32 envelope {env[k]:.3e})")
        assert d <= max(env[k], 2e-6), (k, d, env[k])
    assert pu.field_maxrel(ma.cpu().numpy(), mb.cpu().numpy()) <= 1e-5
    assert pu.field_maxrel(pa.cpu().numpy(), pb.cpu().numpy()) <= 1e-5


def test_resume_from_read_state():
    """10 steps equal 5 steps, read back, re-create from the read state, 5 steps."""
    sc = scenes.random_scene(20000, 32, 65, cscale=10.0, fstretch=0.2, vscale=1.0, per_particle_E=True)
    pu.log("resume")
    first = pu.gpu_run(sc, 5, read=("particles",))
    sc2 = scenes.Scene(**{**sc.__dict__, "x": first["x"], "v": first["v"], "C": first["C"], "F": first["F"]})
    second = pu.gpu_run(sc2, 5)
    orc, env = pu.envelope(sc, 10)
    assert_particle_parity(sc, second, orc, env)


def test_multiple_chunks_per_block():
    """More than 1024 particles in one 8^3 node-block: several P2G chunks
    accumulate into the same window nodes."""
    sc = scenes.random_scene(6000, 32, 66, lo=[0.40] * 3, hi=[0.40 + 6 / 32] * 3, vscale=1.0, cscale=5.0,
                             fstretch=0.1)
    pu.log("multi-chunk block")
    gpu = pu.gpu_run(sc, 2)
    orc, env = pu.envelope(sc, 2)
    assert_particle_parity(sc, gpu, orc, env)


@pytest.mark.parametrize("mode", ["sorted", "free_zone", "fused_scheduled"])
def test_position_clamp_matches_oracle(mode):
    """Reading S15: positions are clamped to [2dx, (n-2)dx] after advection,
    and status word 1 counts the clamped components.  Three clusters leave
    the box through its faces (walls and gravity off) and are clamped in
    every one of 5 steps; the fourth stays inside.  x, v, C, F and the clamp
    count must match the oracle's, with the clamp taken by G2P (sorting every
    step or under the free-zone policy) or by the fused G2P2G pass."""
    sc = scenes.clamp_scene()
    steps = 5
    pu.log(f"position clamp, {mode}: N={sc.N} n={sc.n} steps={steps}")
    policy = {"sorted": None, "free_zone": (4, 1 << 40), "fused_scheduled": (4, 1 << 40)}[mode]
    gpu = pu.gpu_run(sc, steps, sort_policy=policy, fused=mode == "fused_scheduled")
    orc, env = pu.envelope(sc, steps)
    assert orc.clamped == steps * sc.extra["clamped_per_step"]
    n = sc.n
    lo, hi = np.float32(2.0 / n), np.float32((n - 2.0) / n)
    cl = sc.extra["cluster"]
    # the crossing components sit exactly on their planes
    assert np.all(gpu["x"][cl == 0, 0] == lo) and np.all(gpu["x"][cl == 1, 1] == hi)
    assert np.all(gpu["x"][cl == 2, :2] == lo) and np.all(gpu["x"][cl == 2, 2] == hi)
    assert_particle_parity(sc, gpu, orc, env)
    pu.log(f"clamp counts: gpu {gpu['status'][1]}, oracle {orc.clamped}")
    assert gpu["status"][1] == orc.clamped
    assert gpu["status"][0] == mpm.MPM_STATUS_CLAMPED
