"""ctypes binding of the serial CPU MLS-MPM oracle (``mpm_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never imports, links or calls it, and it never calls the GPU library.

Two builds of the same C source exist: ``f64`` (the reference) and ``f32``
(used only to measure the rounding envelope that fp32 arithmetic can reach).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mpm_oracle.c")
LIBS = {"f64": os.path.join(HERE, "libmpm_oracle_f64.so"),
        "f32": os.path.join(HERE, "libmpm_oracle_f32.so")}
CTYPES_REAL = {"f64": ctypes.c_double, "f32": ctypes.c_float}
NP_REAL = {"f64": np.float64, "f32": np.float32}


def build(force: bool = True) -> None:
    """Compile both precisions with gcc (no fast-math, no FP contraction)."""
    for prec, out in LIBS.items():
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        real = "double" if prec == "f64" else "float"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", f"-DORC_REAL={real}", SRC, "-o", out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


class OrcParams(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("wall", ctypes.c_int32), ("material", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("dt", ctypes.c_double),
                ("gravity", ctypes.c_double * 3), ("E", ctypes.c_double),
                ("nu", ctypes.c_double), ("rho", ctypes.c_double), ("p_vol", ctypes.c_double),
                ("friction_deg", ctypes.c_double), ("snow_M", ctypes.c_double),
                ("snow_beta", ctypes.c_double), ("snow_xi", ctypes.c_double)]


_loaded = {}


def lib(prec: str = "f64") -> ctypes.CDLL:
    if prec in _loaded:
        return _loaded[prec]
    path = LIBS[prec]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(force=False)
    L = ctypes.CDLL(path)
    R = CTYPES_REAL[prec]
    P = ctypes.POINTER(R)
    L.orc_real_bytes.restype = ctypes.c_int
    L.orc_base.argtypes = [R]
    L.orc_base.restype = ctypes.c_int64
    L.orc_weights.argtypes = [R, P]
    L.orc_svd3.argtypes = [P, P, P, P]
    L.orc_rotation.argtypes = [P, P]
    L.orc_lame.argtypes = [R, R, P, P]
    L.orc_kirchhoff_fc.argtypes = [P, R, R, P]
    L.orc_kirchhoff_fluid.argtypes = [R, R]
    L.orc_kirchhoff_fluid.restype = R
    L.orc_sand_alpha.argtypes = [R]
    L.orc_sand_alpha.restype = R
    L.orc_sand_project.argtypes = [P, R, R]
    L.orc_sand_project.restype = ctypes.c_int
    L.orc_kirchhoff_sand.argtypes = [P, R, R, P]
    L.orc_snow_p0.argtypes = [R, R, R]
    L.orc_snow_p0.restype = R
    L.orc_snow_project.argtypes = [P, P, R, R, R, R, R]
    L.orc_snow_project.restype = ctypes.c_int
    pp = ctypes.POINTER(OrcParams)
    L.orc_grid_clear.argtypes = [pp, P, P]
    L.orc_p2g.argtypes = [pp, ctypes.c_int64, P, P, P, P, P, P, P, P]
    L.orc_p2g.restype = ctypes.c_int64
    L.orc_grid_update.argtypes = [pp, P, P, P]
    L.orc_g2p.argtypes = [pp, ctypes.c_int64, P, P, P, P, P, P]
    L.orc_g2p.restype = ctypes.c_int64
    L.orc_step.argtypes = [pp, ctypes.c_int64, P, P, P, P, P, P, P, P, P]
    L.orc_step.restype = ctypes.c_int64
    assert L.orc_real_bytes() == ctypes.sizeof(R)
    _loaded[prec] = L
    return L


def make_params(n, dt, gravity, wall, material, E, nu, rho, p_vol, friction_deg=30.0,
                snow_M=0.8, snow_beta=0.9, snow_xi=5.0, snow_alpha0=0.0) -> OrcParams:
    """snow_alpha0 is part of the initial state (the log plastic volume every
    particle starts with), not of the step: OracleSim puts it in J."""
    P = OrcParams()
    P.n, P.wall, P.material, P.pad = int(n), int(wall), int(material), 0
    P.dt = float(dt)
    for a in range(3):
        P.gravity[a] = float(gravity[a])
    P.E, P.nu, P.rho, P.p_vol = float(E), float(nu), float(rho), float(p_vol)
    P.friction_deg = float(friction_deg)
    P.snow_M, P.snow_beta, P.snow_xi = float(snow_M), float(snow_beta), float(snow_xi)
    return P


def _ptr(a, prec):
    if a is None:
        return None
    assert a.dtype == NP_REAL[prec] and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(CTYPES_REAL[prec]))


class Oracle:
    """Thin wrapper over the oracle's entry points at one precision."""

    def __init__(self, prec: str = "f64"):
        self.prec = prec
        self.L = lib(prec)
        self.dtype = NP_REAL[prec]

    def arr(self, a, shape=None):
        out = np.ascontiguousarray(np.asarray(a, dtype=self.dtype))
        return out if shape is None else out.reshape(shape)

    def base(self, xn: float) -> int:
        return int(self.L.orc_base(xn))

    def weights(self, f: float) -> np.ndarray:
        w = np.zeros(3, self.dtype)
        self.L.orc_weights(f, _ptr(w, self.prec))
        return w

    def svd3(self, F):
        F = self.arr(F, (3, 3))
        U = np.zeros((3, 3), self.dtype)
        s = np.zeros(3, self.dtype)
        V = np.zeros((3, 3), self.dtype)
        self.L.orc_svd3(_ptr(F, self.prec), _ptr(U, self.prec), _ptr(s, self.prec), _ptr(V, self.prec))
        return U, s, V

    def rotation(self, F):
        F = self.arr(F, (3, 3))
        R = np.zeros((3, 3), self.dtype)
        self.L.orc_rotation(_ptr(F, self.prec), _ptr(R, self.prec))
        return R

    def lame(self, E, nu):
        R = CTYPES_REAL[self.prec]
        mu, lam = R(), R()
        self.L.orc_lame(E, nu, ctypes.byref(mu), ctypes.byref(lam))
        return mu.value, lam.value

    def kirchhoff_fc(self, F, mu, lam):
        F = self.arr(F, (3, 3))
        tau = np.zeros((3, 3), self.dtype)
        self.L.orc_kirchhoff_fc(_ptr(F, self.prec), mu, lam, _ptr(tau, self.prec))
        return tau

    def kirchhoff_fluid(self, J, K):
        return float(self.L.orc_kirchhoff_fluid(J, K))

    def sand_alpha(self, friction_deg):
        return float(self.L.orc_sand_alpha(friction_deg))

    def sand_project(self, F, nu, alpha):
        """Returns (projected F, case: 0 unchanged, 1 tip, 2 cone surface)."""
        F = self.arr(F, (3, 3)).copy()
        kind = int(self.L.orc_sand_project(_ptr(F, self.prec), nu, alpha))
        return F, kind

    def snow_p0(self, a, kappa, xi):
        return float(self.L.orc_snow_p0(a, kappa, xi))

    def snow_project(self, F, a, mu, lam, M, beta, xi):
        """Returns (projected F, new log plastic volume, case: 0 elastic,
        1 compression tip, 2 tension tip, 3 onto the ellipse)."""
        F = self.arr(F, (3, 3)).copy()
        av = np.array([a], dtype=self.dtype)
        kind = int(self.L.orc_snow_project(_ptr(F, self.prec), _ptr(av, self.prec), mu, lam, M, beta, xi))
        return F, float(av[0]), kind

    def kirchhoff_sand(self, F, mu, lam):
        F = self.arr(F, (3, 3))
        tau = np.zeros((3, 3), self.dtype)
        self.L.orc_kirchhoff_sand(_ptr(F, self.prec), mu, lam, _ptr(tau, self.prec))
        return tau


class OracleSim:
    """Particle state plus a dense grid, stepped by the oracle.

    Arrays are AoS in the oracle's precision: x, v (N,3); C, F (N,3,3);
    J (N,) (for snow: the log plastic volume a = ln J_P, starting at the
    scene's snow_alpha0); E_p (N,) or None.  The grid after the last step is kept in
    gm (n^3), gp (n^3,3) (P2G momentum) and gv (n^3,3) (updated velocity),
    indexed [k, j, i] = node (i, j, k).
    """

    def __init__(self, scene, prec: str = "f64", x=None, v=None, C=None, F=None, J=None):
        self.orc = Oracle(prec)
        self.prec = prec
        dt = self.orc.dtype
        p = scene.params()
        self.params = make_params(**p)
        self.n = p["n"]
        N = scene.N if x is None else len(x)
        # Own copies: the state is advanced in place, and the inputs (the
        # scene's arrays) must stay as they were.
        own = lambda a, shape: np.array(np.reshape(a, shape), dtype=dt, order="C", copy=True)
        self.x = own(scene.x if x is None else x, (N, 3))
        self.v = own(scene.v if v is None else v, (N, 3))
        C0 = C if C is not None else scene.C
        self.C = np.zeros((N, 3, 3), dt) if C0 is None else own(C0, (N, 3, 3))
        F0 = F if F is not None else scene.F
        self.F = np.tile(np.eye(3, dtype=dt), (N, 1, 1)) if F0 is None else own(F0, (N, 3, 3))
        J0 = J if J is not None else scene.J
        if J0 is not None:
            self.J = own(J0, (N,))
        elif p["material"] == 3:
            self.J = np.full(N, p["snow_alpha0"], dt)
        else:
            self.J = np.ones(N, dt)
        self.E_p = None if scene.E_p is None else own(scene.E_p, (N,))
        nn = self.n ** 3
        self.gm = np.zeros(nn, dt)
        self.gp = np.zeros((nn, 3), dt)
        self.gv = np.zeros((nn, 3), dt)
        self.clamped = 0

    @property
    def N(self):
        return self.x.shape[0]

    def _P(self, a):
        return _ptr(a, self.prec)

    def step(self, k: int = 1) -> None:
        for _ in range(k):
            r = self.orc.L.orc_step(ctypes.byref(self.params), self.N, self._P(self.x), self._P(self.v),
                                    self._P(self.C), self._P(self.F), self._P(self.J), self._P(self.E_p),
                                    self._P(self.gm), self._P(self.gp), self._P(self.gv))
            if r < 0:
                raise RuntimeError("oracle: a particle stencil left the grid")
            self.clamped += int(r)

    def p2g(self):
        """P2G alone from the current state into freshly cleared gm, gp."""
        self.orc.L.orc_grid_clear(ctypes.byref(self.params), self._P(self.gm), self._P(self.gp))
        r = self.orc.L.orc_p2g(ctypes.byref(self.params), self.N, self._P(self.x), self._P(self.v),
                               self._P(self.C), self._P(self.F), self._P(self.J), self._P(self.E_p),
                               self._P(self.gm), self._P(self.gp))
        if r != 0:
            raise RuntimeError("oracle: a particle stencil left the grid")

    def grid_update(self):
        self.orc.L.orc_grid_update(ctypes.byref(self.params), self._P(self.gm), self._P(self.gp),
                                   self._P(self.gv))

    def g2p(self):
        r = self.orc.L.orc_g2p(ctypes.byref(self.params), self.N, self._P(self.x), self._P(self.v),
                               self._P(self.C), self._P(self.F), self._P(self.J), self._P(self.gv))
        self.clamped += int(r)

    def grid_mass(self):
        n = self.n
        return self.gm.reshape(n, n, n)

    def grid_momentum(self):
        """m_i * v_i after gravity and walls, shape (n,n,n,3) indexed [k,j,i]."""
        n = self.n
        return (self.gv * self.gm[:, None]).reshape(n, n, n, 3)
