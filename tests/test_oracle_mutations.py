"""The oracle's pins must catch plausible mistakes.

Each case plants one slip in a private copy of the oracle's C source (a
dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
constant), builds it with gcc into a temporary library, points the oracle
binding at it and runs the pin tests.  At least one pin must fail for every
mutant.  Everything here runs on the CPU; the GPU library is not involved.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = open(oracle.SRC).read()

MUTANTS = [
    ("weights mirrored", "w[o] = bspline2(f - (real)o);", "w[o] = bspline2(f + (real)o - 2);"),
    ("base without half shift", "return (int64_t)floor(xn - (real)0.5);", "return (int64_t)floor(xn);"),
    ("spline inner piece", "return (real)0.75 - d * d;", "return (real)0.75 - d;"),
    ("no SVD sign fix on V", "if (dot3(v3x, v[2]) < 0)", "if (0)"),
    ("rotation transposed", "mat_mul_bt(U, V, R);", "mat_mul_bt(V, U, R);"),
    ("stress F^T F order", "mat_mul_bt(D, F, tau);", "for (int r_ = 0; r_ < 3; ++r_) for (int c_ = 0; c_ < 3; ++c_) "
     "{ real s_ = 0; for (int k_ = 0; k_ < 3; ++k_) s_ += F[k_ * 3 + r_] * D[k_ * 3 + c_]; tau[r_ * 3 + c_] = s_; }"),
    ("stress drops lambda term", "tau[a * 4] += lam * (J - 1) * J;", "tau[a * 4] += 0;"),
    ("stress lambda term without J", "tau[a * 4] += lam * (J - 1) * J;", "tau[a * 4] += lam * (J - 1);"),
    ("lame swapped", "*mu = E / (2 * (1 + nu));", "*mu = E * nu / ((1 + nu) * (1 - 2 * nu)) + 0 * E / (2 * (1 + nu));"),
    ("fluid stress sign", "return K * J * (J - 1);", "return K * J * (1 - J);"),
    ("D^-1 = 2/dx^2 in P2G", "const real inv_dx2x4 = 4 * (real)P->n * (real)P->n; /* D^{-1}",
     "const real inv_dx2x4 = 2 * (real)P->n * (real)P->n; /* D^{-1}"),
    ("stress term sign in P2G", "A[i] = mass * C[9 * p + i] - dt * vol", "A[i] = mass * C[9 * p + i] + dt * vol"),
    ("mass without density", "mass = (real)P->rho * (real)P->p_vol;", "mass = (real)P->p_vol;"),
    ("A transposed in P2G", "real ad = A[a * 3] * d[0] + A[a * 3 + 1] * d[1] + A[a * 3 + 2] * d[2];",
     "real ad = A[a] * d[0] + A[3 + a] * d[1] + A[6 + a] * d[2];"),
    ("P2G offset sign", "real d[3] = {(real)i * dx - x[3 * p], (real)j * dx - x[3 * p + 1], (real)k * dx - x[3 * p + 2]};\n"
     "          int64_t id = node_index(n, i, j, k);\n          gm[id]",
     "real d[3] = {x[3 * p] - (real)i * dx, x[3 * p + 1] - (real)j * dx, x[3 * p + 2] - (real)k * dx};\n"
     "          int64_t id = node_index(n, i, j, k);\n          gm[id]"),
    ("P2G axis swap in index", "int64_t id = node_index(n, i, j, k);\n          gm[id]", "int64_t id = node_index(n, j, i, k);\n          gm[id]"),
    ("grid update without gravity", "va = gp[3 * id + a] / gm[id] + dt * (real)P->gravity[a];", "va = gp[3 * id + a] / gm[id];"),
    ("wall one layer too thick", "int in_wall = i < wall ||", "int in_wall = i <= wall ||"),
    ("wall only on low side", "|| i >= n - wall || j >= n - wall || k >= n - wall;", ";"),
    ("G2P C without D^-1", "for (int i = 0; i < 9; ++i) Cn[i] = inv_dx2x4 * B[i];", "for (int i = 0; i < 9; ++i) Cn[i] = B[i];"),
    ("G2P C transposed", "for (int c = 0; c < 3; ++c) B[a * 3 + c] += wt * vi[a] * d[c];",
     "for (int c = 0; c < 3; ++c) B[c * 3 + a] += wt * vi[a] * d[c];"),
    ("G2P F update right-multiplied", "mat_mul(G, F + 9 * p, F + 9 * p);", "mat_mul(F + 9 * p, G, F + 9 * p);"),
    ("G2P fluid J additive", "J[p] = J[p] * mat_det(G);", "J[p] = J[p] + mat_det(G) - 1 + dt * 0;"),
    ("G2P advects with pre-gravity velocity", "real xa = x[3 * p + a] + dt * vn[a];",
     "real xa = x[3 * p + a] + dt * (vn[a] - dt * (real)P->gravity[a]);"),
    ("G2P velocity of neighbour axis", "vn[a] += wt * vi[a];", "vn[a] += wt * vi[(a + 1) % 3];"),
    ("G2P without the position clamp", "if (xa < lo) { xa = lo; ++clamped; }\n      if (xa > hi) { xa = hi; ++clamped; }",
     ""),
    ("G2P clamp box [dx, (n-1)dx]", "const real lo = 2 * dx, hi = (real)(n - 2) * dx;",
     "const real lo = dx, hi = (real)(n - 1) * dx;"),
    ("G2P clamp counts the x component only", "if (xa < lo) { xa = lo; ++clamped; }\n      if (xa > hi) { xa = hi; ++clamped; }",
     "if (xa < lo) { xa = lo; clamped += a == 0; }\n      if (xa > hi) { xa = hi; clamped += a == 0; }"),
    ("sand tip on compression", "  if (t > 0) {\n    kind = 1;", "  if (t < 0) {\n    kind = 1;"),
    ("sand cone factor doubled", "const real g = nd + (1 + nu) / (1 - 2 * nu) * t * alpha;",
     "const real g = nd + 2 * (1 + nu) / (1 - 2 * nu) * t * alpha;"),
    ("sand strain without the half", "e[i] = (real)0.5 * log(l[i]);", "e[i] = log(l[i]);"),
    ("sand stress drops lambda", "m[i] = (2 * mu * e[i] + lam * t) / l[i];", "m[i] = (2 * mu * e[i]) / l[i];"),
    ("sand alpha with cos", "const real sp = sin(friction_deg", "const real sp = cos(friction_deg"),
    ("sand projection moves the trace", "h[i] = e[i] - g * d[i] / nd;", "h[i] = e[i] - g * e[i] / nd;"),
    ("sand no projection in G2P", "if (P->material == 2) orc_sand_project(", "if (0) orc_sand_project("),
    ("sand stress of the fixed-corotated model", "orc_kirchhoff_sand(F + 9 * p, mu, lam, tau);",
     "orc_kirchhoff_fc(F + 9 * p, mu, lam, tau);"),
    ("sand stretch scaled inversely", "m[i] = exp(h[i] - e[i]);", "m[i] = exp(e[i] - h[i]);"),
    ("snow hardens on expansion", "real x = xi * (a < 0 ? -a : 0);", "real x = xi * (a > 0 ? a : 0);"),
    ("snow hardening uncapped", "if (x > (real)ORC_SNOW_XCAP) x = (real)ORC_SNOW_XCAP;", ""),
    ("snow hardening cosh", "return kappa * sinh(x);", "return kappa * (cosh(x) - 1);"),
    ("snow bulk modulus is lambda", "const real kappa = lam + 2 * mu / 3;", "const real kappa = lam;"),
    ("snow q without sqrt(3/2)", "const real q2 = 6 * mu * mu * nd2;", "const real q2 = 4 * mu * mu * nd2;"),
    ("snow tension tip without beta", "t_new = beta * p0 / kappa;", "t_new = p0 / kappa;"),
    ("snow tension test without beta", "} else if (p < -beta * p0) {", "} else if (p < -p0) {"),
    ("snow plastic volume sign", "*a += t - t_new;", "*a += t_new - t;"),
    ("snow yield with M unsquared", "const real y = (1 + 2 * beta) * q2 + M * M * (p + beta * p0) * (p - p0);",
     "const real y = (1 + 2 * beta) * q2 + M * (p + beta * p0) * (p - p0);"),
    ("snow surface without the cohesion factor", "((1 + 2 * beta) * q2));", "(q2));"),
    ("snow surface moves the trace", "m[i] = exp(t_new / 3 + k * d[i] - e[i]);", "m[i] = exp(k * e[i] - e[i]);"),
    ("snow compression tip sign", "t_new = -p0 / kappa;", "t_new = p0 / kappa;"),
    ("snow no projection in G2P", "if (P->material == 3) {", "if (0) {"),
    ("snow stress of the fixed-corotated model", "} else if (P->material == 2 || P->material == 3) {",
     "} else if (P->material == 2) {"),
]


def _all_pins():
    rng = np.random.default_rng(0)
    out = [
        lambda o: [pins.test_weights_moments(o, f) for f in [0.5, 0.77, 1.0, 1.31, 1.49]],
        pins.test_weights_support_and_base,
        pins.test_weights_are_c1_continuous,
        lambda o: [pins.test_svd_against_numpy(o, s) for s in range(6)],
        lambda o: [pins.test_rotation_is_polar_factor(o, s) for s in range(4)],
        pins.test_lame_closed_forms,
        pins.test_stress_closed_forms,
        lambda o: [pins.test_stress_is_energy_derivative(o, s) for s in range(3)],
        pins.test_fluid_stress,
        pins.test_p2g_single_particle_table,
        lambda o: pins.test_p2g_mass_momentum_angular_momentum(),
        lambda o: pins.test_affine_reproduction_translation_and_rotation(),
        lambda o: pins.test_free_fall(),
        lambda o: pins.test_step_momentum_conservation(),
        lambda o: pins.test_walls_zero_velocity(),
        lambda o: pins.test_position_clamp(),
        lambda o: pins.test_stress_force_is_energy_gradient(),
        lambda o: pins.test_fluid_J_matches_det_F(),
        pins.test_sand_alpha_is_the_mohr_coulomb_fit,
        pins.test_sand_stress_closed_form_and_energy,
        pins.test_sand_projection_cases,
        pins.test_sand_projection_is_objective,
        lambda o: pins.test_sand_step_projects_in_g2p(),
        lambda o: pins.test_sand_stress_force_is_energy_gradient(),
        pins.test_snow_hardening_closed_form,
        pins.test_snow_projection_cases,
        pins.test_snow_projection_without_hardening,
        pins.test_snow_projection_is_objective,
        lambda o: pins.test_snow_step_projects_in_g2p(),
        lambda o: pins.test_snow_p2g_uses_hencky_stress(),
    ]
    del rng
    return out


def _build(src_text, out):
    with tempfile.NamedTemporaryFile("w", suffix=".c", delete=False) as f:
        f.write(src_text)
        cpath = f.name
    try:
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                        "-DORC_REAL=double", cpath, "-o", out, "-lm"], check=True,
                       capture_output=True)
    finally:
        os.unlink(cpath)


def _failing_pins(libpath):
    saved_path, saved_lib = oracle.LIBS["f64"], oracle._loaded.pop("f64", None)
    oracle.LIBS["f64"] = libpath
    failed = []
    try:
        o = oracle.Oracle("f64")
        with np.errstate(all="ignore"):
            for k, pin in enumerate(_all_pins()):
                try:
                    pin(o)
                except (AssertionError, RuntimeError, np.linalg.LinAlgError, FloatingPointError):
                    failed.append(k)
    finally:
        oracle.LIBS["f64"] = saved_path
        oracle._loaded.pop("f64", None)
        if saved_lib is not None:
            oracle._loaded["f64"] = saved_lib
    return failed


def test_unmutated_source_passes_all_pins(tmp_path):
    lib = str(tmp_path / "orig.so")
    _build(SRC, lib)
    assert _failing_pins(lib) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    lib = str(tmp_path / "mut.so")
    _build(SRC.replace(old, new), lib)
    assert _failing_pins(lib), f"no pin catches mutant '{name}'"
