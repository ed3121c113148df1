"""GPU parity of the fused G2P2G steps (mpm_set_fused_steps): between sorts
the G2P of a step and the P2G of the next run in one kernel, and the state
is read back from wherever that kernel left it.  The physics is the same as
separate kernels, so the oracle and the tolerances of the per-step-sort
parity tests apply unchanged.

Cases: the free-zone scenes (no sort after creation, a sort every 3 steps,
a mover budget), the equality with per-step sorting, batched graphs against
single steps, readback between launches that end on a fused pass, switching
fusion off and on, and the default policy (every step sorts, so no step is
fused); then the host-scheduled sorts (a power-of-two interval and no mover
budget), where a step after a fused pass launches the fused kernel alone."""
import numpy as np
import pytest

import material_point_physics_amd as mpm
from material_point_physics_amd import scenes
import parity_util as pu
from test_gpu_parity import assert_grid_parity, assert_particle_parity
from test_gpu_free_zone import NEVER, bins_of, swirl

pytestmark = pytest.mark.gpu

CASES = {
    # no sort after creation: every step after the first is fused, and many
    # particles leave their bins (direct deposits and gathers)
    "swirl_never": (lambda: swirl(71, cscale=2.0), 8, NEVER),
    # the three jelly spheres, sorted every 3 steps (plain G2P before each sort;
    # 3 is not a power of two, so the device decides)
    "jelly3_every3": (scenes.jelly3_55k, 10, (3, 1 << 40)),
    # fluid with per-particle modulus, sorted when more than 50 particles left their bins
    "swirl_fluid_budget50": (lambda: swirl(72, material=scenes.J_FLUID, E=400.0, per_particle_E=True), 8,
                             (1 << 30, 50)),
    # elastic with per-particle modulus, no sort after creation
    "swirl_E_never": (lambda: swirl(73, cscale=2.0, per_particle_E=True), 7, NEVER),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_particles_match_oracle(name):
    make, steps, policy = CASES[name]
    sc = make()
    pu.log(f"fused {name}: N={sc.N} n={sc.n} steps={steps} policy={policy}")
    gpu = pu.gpu_run(sc, steps, sort_policy=policy, fused=True)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(1e-5, 20 * env["v"]))
    assert gpu["status"][0] == 0
    if policy == NEVER:
        moved = (bins_of(orc.x, sc.n) != bins_of(sc.x, sc.n)).any(axis=1).sum()
        pu.log(f"{name}: {moved} particles left their creation bin")
        assert moved > 100


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(a).max(), 1e-30)


@pytest.mark.parametrize("policy", [None, NEVER, (3, 1 << 40)], ids=["every_step", "never", "every3"])
def test_fused_equals_separate_kernels(policy):
    """Same scene and policy, fused vs separate kernels: equal up to the
    order of float additions."""
    sc = swirl(74, cscale=2.0)
    a = pu.gpu_run(sc, 9, sort_policy=policy)
    b = pu.gpu_run(sc, 9, sort_policy=policy, fused=True)
    for k in ("x", "v", "C", "F", "m", "p"):
        err = _rel(a[k], b[k])
        pu.log(f"separate vs fused ({policy}) {k}: {err:.2e}")
        assert err < 1e-5, (k, err)


def _read(sim):
    x, v, C, F = sim.read_particles()
    m, p = sim.read_grid()
    return dict(x=x.cpu().numpy(), v=v.cpu().numpy(), C=C.cpu().numpy(), F=F.cpu().numpy(), m=m.cpu().numpy(),
                p=p.cpu().numpy())


def test_fused_batched_graphs_and_mid_run_readback():
    """17 steps as one call (two 8-step graphs and a single step) against
    17 single-step calls with a readback after each, both fused and never
    re-sorting: every call ends on a fused pass, whose state (v, C stored,
    F current, the grid of the last step) the readback must find.  Then the
    run is checked against the oracle."""
    sc = swirl(75, cscale=2.0)
    steps = 17
    a = pu.gpu_run(sc, steps, sort_policy=NEVER, fused=True)
    sim = mpm.Simulation(sc)
    try:
        sim.set_sort_policy(*NEVER)
        sim.set_fused_steps(True)
        for k in range(steps):
            sim.step(1)
            if k in (0, 5, 11):
                mid = _read(sim)
                orc, env = pu.envelope(sc, k + 1)
                pu.log(f"after {k + 1} single steps")
                assert_particle_parity(sc, mid, orc, env)
                assert_grid_parity(sc, mid, orc, tol=max(1e-5, 20 * env["v"]))
        b = _read(sim)
    finally:
        sim.close()
    for f in ("x", "v", "C", "F", "m", "p"):
        err = _rel(a[f], b[f])
        pu.log(f"17 steps batched vs single: {f} {err:.2e}")
        assert err < 1e-5, (f, err)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, a, orc, env)


def test_switch_fusion_off_and_on():
    """Fused steps, then separate kernels, then fused again (the separate
    P2G must see that the fused pass already ran it): equal to the oracle."""
    sc = swirl(76, cscale=2.0)
    sim = mpm.Simulation(sc)
    try:
        sim.set_sort_policy(5, 1 << 40)
        sim.set_fused_steps(True)
        sim.step(3)
        sim.set_fused_steps(False)
        sim.step(4)
        sim.set_fused_steps(True)
        sim.step(3)
        got = _read(sim)
        got["status"] = sim.status()
    finally:
        sim.close()
    orc, env = pu.envelope(sc, 10)
    assert_particle_parity(sc, got, orc, env)
    assert_grid_parity(sc, got, orc, tol=max(1e-5, 20 * env["v"]))


# A fixed power-of-two interval with no mover budget: the host schedules the
# sorts, and a step after a fused pass launches the fused kernel alone.
SCHED_CASES = {
    "swirl_every4": (lambda: swirl(77, cscale=2.0), 13, (4, 1 << 40)),
    "swirl_fluid_every2": (lambda: swirl(78, material=scenes.J_FLUID, E=400.0), 9, (2, 1 << 40)),
    "swirl_E_every8": (lambda: swirl(79, cscale=2.0, per_particle_E=True), 19, (8, 1 << 40)),
    "jelly3_every16": (scenes.jelly3_55k, 21, (16, 1 << 40)),
}


@pytest.mark.parametrize("name", list(SCHED_CASES))
def test_scheduled_fused_steps_match_oracle(name):
    make, steps, policy = SCHED_CASES[name]
    sc = make()
    pu.log(f"scheduled fused {name}: N={sc.N} n={sc.n} steps={steps} policy={policy}")
    gpu = pu.gpu_run(sc, steps, sort_policy=policy, fused=True)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, gpu, orc, env)
    assert_grid_parity(sc, gpu, orc, tol=max(1e-5, 20 * env["v"]))
    assert gpu["status"][0] == 0


def test_scheduled_batches_single_steps_and_mode_changes():
    """K = 4 without a budget: 21 steps as one call against single-step calls
    with readbacks (lean graphs of every phase, the first full step under the
    schedule), then the modes in turn (scheduled, device-decided, separate,
    scheduled again), all against the oracle."""
    sc = swirl(80, cscale=2.0)
    steps = 21
    a = pu.gpu_run(sc, steps, sort_policy=(4, 1 << 40), fused=True)
    sim = mpm.Simulation(sc)
    try:
        sim.set_sort_policy(4, 1 << 40)
        sim.set_fused_steps(True)
        for k in range(steps):
            sim.step(1)
            if k in (2, 9):
                mid = _read(sim)
                orc, env = pu.envelope(sc, k + 1)
                pu.log(f"scheduled: after {k + 1} single steps")
                assert_particle_parity(sc, mid, orc, env)
        b = _read(sim)
    finally:
        sim.close()
    for f in ("x", "v", "C", "F", "m", "p"):
        err = _rel(a[f], b[f])
        pu.log(f"scheduled, {steps} steps batched vs single: {f} {err:.2e}")
        assert err < 1e-5, (f, err)
    orc, env = pu.envelope(sc, steps)
    assert_particle_parity(sc, a, orc, env)

    sim = mpm.Simulation(sc)
    try:
        sim.set_fused_steps(True)
        sim.set_sort_policy(4, 1 << 40)  # scheduled
        sim.step(6)
        sim.set_sort_policy(3, 1 << 40)  # device-decided (3 is not a power of two)
        sim.step(5)
        sim.set_fused_steps(False)       # separate kernels
        sim.step(3)
        sim.set_fused_steps(True)
        sim.set_sort_policy(2, 1 << 40)  # scheduled again, other interval
        sim.step(9)
        got = _read(sim)
        got["status"] = sim.status()
    finally:
        sim.close()
    orc, env = pu.envelope(sc, 23)
    assert_particle_parity(sc, got, orc, env)
    assert_grid_parity(sc, got, orc, tol=max(1e-5, 20 * env["v"]))


@pytest.mark.parametrize("policy", [(1 << 30, 1 << 40), (4, 1 << 40)], ids=["device_decided", "scheduled"])
def test_fused_profiled_steps_match_graph_steps(policy):
    """Eager per-kernel-timed steps (the benchmark's timing path) run the same
    kernels as the fused graphs: 11 steps either way, then particles and grid
    compared; in the scheduled mode the kernels a step does not launch take
    no time."""
    sc = swirl(86, cscale=2.0)
    pu.log(f"fused profiled vs graph, policy {policy}")
    a = mpm.Simulation(sc)
    b = mpm.Simulation(sc)
    try:
        for s in (a, b):
            s.set_sort_policy(*policy)
            s.set_fused_steps(True)
        a.step(11)
        ms = mpm.mpm_step_profiled(b.handle, 11, b.stream)
        assert all(v >= 0 for v in ms.values()) and ms["k_g2p"] > 0
        assert mpm.mpm_steps_taken(a.handle) == mpm.mpm_steps_taken(b.handle) == 11
        ra, rb = _read(a), _read(b)
    finally:
        a.close()
        b.close()
    for f in ("x", "v", "C", "F", "m", "p"):
        err = _rel(ra[f], rb[f])
        pu.log(f"profiled vs graph {f}: {err:.2e}")
        assert err < 1e-5, (f, err)
