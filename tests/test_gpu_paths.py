"""GPU parity on every launch configuration the scene size selects.

The scene's size picks, at creation, the particles per chunk (64, 128, 256),
the P2G windows per wavefront (8 for small scenes, else 2) and the sort's
kernels (one kernel for small scenes of at most 4096 bins; else a scan in one
workgroup for at most 8192 bins, or in tiles, and the scatter).  Each case
below asserts the configuration it is meant to cover (mpm_launch_config),
then compares every particle after three steps with the fp64 oracle, within
10x the fp32 oracle's own distance from it (the bar of test_gpu_parity), and
the grid.  Dense boxes put several full chunks in a bin, so the scatter's
block transpose runs.  The 256-particle chunks are covered at 1.1M particles
in test_gpu_fullfield.
"""
import pytest

from material_point_physics_amd import scenes
import material_point_physics_amd as mpm
import parity_util as pu
from test_gpu_parity import assert_grid_parity, assert_particle_parity, GRID_TOL

pytestmark = pytest.mark.gpu

CASES = {
    # (scene, expected (chunk, windows, sort kernels))
    "small_one_kernel_sort": (lambda: scenes.random_scene(20000, 32, 81, cscale=10.0, fstretch=0.2, vscale=1.0,
                                                          per_particle_E=True), (64, 8, 1)),
    "small_dense_bins": (lambda: scenes.random_scene(24000, 32, 82, lo=[0.3] * 3, hi=[0.55] * 3, cscale=10.0,
                                                     fstretch=0.2, vscale=1.0), (64, 8, 1)),
    "eight_windows_tiled_scan": (lambda: scenes.random_scene(30000, 128, 83, lo=[0.4] * 3, hi=[0.6] * 3,
                                                             cscale=20.0, fstretch=0.2, vscale=1.0, dt=2e-5),
                                 (64, 8, 3)),
    "two_windows_chunk64": (lambda: scenes.random_scene(200000, 64, 84, cscale=10.0, fstretch=0.2, vscale=1.0,
                                                        dt=5e-5), (64, 2, 2)),
    "two_windows_chunk64_dense": (lambda: scenes.random_scene(200000, 64, 85, lo=[0.25] * 3, hi=[0.75] * 3,
                                                              cscale=10.0, fstretch=0.2, vscale=1.0, dt=5e-5),
                                  (64, 2, 2)),
    "two_windows_chunk128": (lambda: scenes.random_scene(600000, 64, 86, lo=[0.2] * 3, hi=[0.8] * 3, cscale=10.0,
                                                         fstretch=0.2, vscale=1.0, dt=5e-5), (128, 2, 2)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_launch_configuration_parity(name):
    make, expect = CASES[name]
    sc = make()
    sim = mpm.Simulation(sc)
    try:
        cfg = sim.launch_config()
    finally:
        sim.close()
    pu.log(f"{name}: N={sc.N} n={sc.n} launch {cfg}")
    assert (cfg["chunk"], cfg["p2g_windows"], cfg["sort_kernels"]) == expect
    steps = 3
    gpu = pu.gpu_run(sc, steps)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(GRID_TOL, 20 * env["v"]))
    assert (gpu["status"][0] & mpm.MPM_STATUS_NONFINITE) == 0
