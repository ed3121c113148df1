"""GPU parity of the free-zone sort policy (mpm_set_sort_policy): between
sorts each chunk keeps its particles, and a particle that left its chunk's bin
is deposited and gathered through the grid directly.  The physics is the same
as sorting every step, so the oracle and the tolerances of the per-step-sort
parity tests apply unchanged.

The policy's decision is taken on the device; these cases pin it from the
host side: with a max interval longer than the run, no step after creation
sorts, and the oracle trajectory shows particles leaving their creation bins,
so the mover paths run."""
import numpy as np
import pytest

from material_point_physics_amd import scenes
import parity_util as pu
from test_gpu_parity import assert_grid_parity, assert_particle_parity

pytestmark = pytest.mark.gpu

NEVER = (1 << 30, 1 << 40)  # no sort after creation


def bins_of(x, n):
    return np.floor(x * n - 0.5).astype(np.int64) >> 2


def swirl(seed, **kw):
    """Random particles carried by a coherent velocity field (a translation
    plus a rotation about the box's vertical axis, up to ~0.1 cell per step),
    so that many of them cross bin boundaries within a few steps.  (Random
    per-particle velocities would cancel on the grid after one transfer.)"""
    sc = scenes.random_scene(20000, 32, seed, **kw)
    x = sc.x.astype(np.float64)
    v = np.stack([15.0 - 50.0 * (x[:, 2] - 0.5), np.full(len(x), 5.0), 50.0 * (x[:, 0] - 0.5)], axis=1)
    sc.v = v.astype(np.float32)
    return sc


CASES = {
    # no sort after creation: many particles leave their bins
    "swirl_never": (lambda: swirl(61, cscale=2.0), 8, NEVER),
    # the three jelly spheres, sorted every 4 steps
    "jelly3_every4": (scenes.jelly3_55k, 10, (4, 1 << 40)),
    # fluid, sorted whenever more than 50 particles have left their bins
    "swirl_fluid_budget50": (lambda: swirl(62, material=scenes.J_FLUID, E=400.0), 8, (1 << 30, 50)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_free_zone_particles_match_oracle(name):
    make, steps, policy = CASES[name]
    sc = make()
    pu.log(f"free zone {name}: N={sc.N} n={sc.n} steps={steps} policy={policy}")
    gpu = pu.gpu_run(sc, steps, sort_policy=policy)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(1e-5, 20 * env["v"]))
    if policy == NEVER:
        moved = (bins_of(orc.x, sc.n) != bins_of(sc.x, sc.n)).any(axis=1).sum()
        pu.log(f"{name}: {moved} particles left their creation bin")
        assert moved > 100  # the direct deposit and gather paths ran


def test_free_zone_equals_per_step_sort():
    """Same scene, per-step sort vs never re-sorting: equal up to the order of
    float additions (relative to each field's scale)."""
    sc = swirl(63, cscale=2.0)
    a = pu.gpu_run(sc, 6)
    b = pu.gpu_run(sc, 6, sort_policy=NEVER)
    for k in ("x", "v", "C", "F", "m", "p"):
        scale = max(np.abs(a[k]).max(), 1e-30)
        err = np.abs(a[k] - b[k]).max() / scale
        pu.log(f"per-step vs free zone {k}: {err:.2e}")
        assert err < 1e-5, (k, err)
