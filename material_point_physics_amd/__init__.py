"""Python binding of libmpm.so (one explicit MLS-MPM step on MI355X).

The functions below carry the names of the C ABI in ``include/mpm.h`` and only
marshal arguments: every step of the path runs in the library's HIP kernels.
Device arrays may be passed as integers (device addresses) or as torch
tensors (their ``data_ptr()``); streams as integers or ``torch.cuda.Stream``.

The library is loaded on first use; if it has not been built the call fails
with an error that says how to build it (there is no CPU fallback).

``Simulation`` is a convenience wrapper that allocates the workspace and the
readback buffers with torch (PyTorch is used only for device memory and
streams).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmpm.so")

MPM_OK = 0
MPM_ERR_INVALID_ARG = -1
MPM_ERR_WORKSPACE = -2
MPM_ERR_HIP = -3
MPM_ERR_STATE = -4
MPM_ERR_TOO_LARGE = -5
MPM_NOALLOC_SCRATCH_BYTES = 64 << 20

MPM_FIXED_COROTATED = 0
MPM_J_FLUID = 1
MPM_SAND = 2
MPM_SNOW = 3

MPM_STATUS_NONFINITE = 0x1
MPM_STATUS_CLAMPED = 0x2
MPM_STATUS_INVERTED = 0x4
MPM_STATUS_BAD_INPUT = 0x8
MPM_STATUS_NO_CONVERGE = 0x10
MPM_STATUS_WORDS = 8

# Every symbol include/mpm.h declares.
EXPORTS = ("mpm_workspace_bytes", "mpm_create", "mpm_step", "mpm_set_sort_policy", "mpm_set_fused_steps",
           "mpm_read_particles", "mpm_run_noalloc", "mpm_read_plastic_state",
           "mpm_read_grid",
           "mpm_status", "mpm_steps_taken", "mpm_num_kernels", "mpm_kernel_name", "mpm_launch_config",
           "mpm_step_profiled",
           "mpm_destroy", "mpm_error_string")


class MpmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {mpm_error_string(code)} ({code})")
        self.code = code


class mpm_params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("grid_n", ctypes.c_int32), ("dt", ctypes.c_float),
                ("gravity", ctypes.c_float * 3), ("wall_nodes", ctypes.c_int32), ("material", ctypes.c_int32),
                ("E", ctypes.c_float), ("nu", ctypes.c_float), ("rho", ctypes.c_float), ("p_vol", ctypes.c_float),
                ("friction_deg", ctypes.c_float), ("snow_M", ctypes.c_float), ("snow_beta", ctypes.c_float),
                ("snow_xi", ctypes.c_float), ("snow_alpha0", ctypes.c_float)]


def make_params(n, dt, gravity, wall, material, E, nu, rho, p_vol, friction_deg=30.0,
                snow_M=0.8, snow_beta=0.9, snow_xi=5.0, snow_alpha0=-0.01) -> mpm_params:
    p = mpm_params()
    p.struct_size = ctypes.sizeof(mpm_params)
    p.grid_n, p.dt = int(n), float(dt)
    for a in range(3):
        p.gravity[a] = float(gravity[a])
    p.wall_nodes, p.material = int(wall), int(material)
    p.E, p.nu, p.rho, p.p_vol = float(E), float(nu), float(rho), float(p_vol)
    p.friction_deg = float(friction_deg)
    p.snow_M, p.snow_beta, p.snow_xi, p.snow_alpha0 = float(snow_M), float(snow_beta), float(snow_xi), float(snow_alpha0)
    return p


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmpm.so (built in-tree by ``__graft_entry__.build()`` or
    ``python material_point_physics_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python material_point_physics_amd/build.py` "
                          "(hipcc, gfx950). There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    pp = ctypes.POINTER(mpm_params)
    L.mpm_workspace_bytes.argtypes = [pp, i64]
    L.mpm_workspace_bytes.restype = sz
    L.mpm_create.argtypes = [pp, i64, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]
    L.mpm_create.restype = ctypes.c_int
    L.mpm_step.argtypes = [vp, i32, vp]
    L.mpm_step.restype = ctypes.c_int
    L.mpm_set_sort_policy.argtypes = [vp, i32, i64, vp]
    L.mpm_set_sort_policy.restype = ctypes.c_int
    L.mpm_set_fused_steps.argtypes = [vp, i32]
    L.mpm_set_fused_steps.restype = ctypes.c_int
    L.mpm_read_particles.argtypes = [vp, vp, vp, vp, vp, vp]
    L.mpm_run_noalloc.argtypes = [pp, i64, vp, vp, vp, vp, vp, i32, vp, vp]
    L.mpm_run_noalloc.restype = ctypes.c_int
    L.mpm_read_plastic_state.argtypes = [vp, vp, vp]
    L.mpm_read_plastic_state.restype = ctypes.c_int
    L.mpm_read_particles.restype = ctypes.c_int
    L.mpm_read_grid.argtypes = [vp, vp, vp, vp]
    L.mpm_read_grid.restype = ctypes.c_int
    L.mpm_status.argtypes = [vp, vp, vp]
    L.mpm_status.restype = ctypes.c_int
    L.mpm_steps_taken.argtypes = [vp]
    L.mpm_steps_taken.restype = i64
    L.mpm_num_kernels.argtypes = []
    L.mpm_num_kernels.restype = i32
    L.mpm_kernel_name.argtypes = [i32]
    L.mpm_kernel_name.restype = ctypes.c_char_p
    L.mpm_launch_config.argtypes = [vp, ctypes.POINTER(i32)]
    L.mpm_launch_config.restype = ctypes.c_int
    L.mpm_step_profiled.argtypes = [vp, i32, vp, ctypes.POINTER(ctypes.c_float)]
    L.mpm_step_profiled.restype = ctypes.c_int
    L.mpm_destroy.argtypes = [vp]
    L.mpm_destroy.restype = None
    L.mpm_error_string.argtypes = [ctypes.c_int]
    L.mpm_error_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _addr(a):
    """Device address of a torch tensor / int / None (no copies)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int, what: str):
    if rc != MPM_OK:
        raise MpmError(rc, what)


# ------------------------------------------------------- C-ABI functions

def mpm_error_string(code: int) -> str:
    return lib().mpm_error_string(int(code)).decode()


def mpm_workspace_bytes(params: mpm_params, n_particles: int) -> int:
    return int(lib().mpm_workspace_bytes(ctypes.byref(params), int(n_particles)))


def mpm_create(params: mpm_params, n_particles: int, x0, v0=None, C0=None, F0=None, E_p=None,
               workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    out = ctypes.c_void_p()
    rc = lib().mpm_create(ctypes.byref(params), int(n_particles), _addr(x0), _addr(v0), _addr(C0), _addr(F0),
                          _addr(E_p), _addr(workspace), int(workspace_bytes), _stream(stream), ctypes.byref(out))
    _check(rc, "mpm_create")
    return out.value


def mpm_step(sim: int, n_steps: int, stream=None) -> None:
    _check(lib().mpm_step(sim, int(n_steps), _stream(stream)), "mpm_step")


def mpm_set_sort_policy(sim: int, max_interval: int, mover_budget: int, stream=None) -> None:
    _check(lib().mpm_set_sort_policy(sim, int(max_interval), int(mover_budget), _stream(stream)),
           "mpm_set_sort_policy")


def mpm_set_fused_steps(sim: int, enable: int) -> None:
    _check(lib().mpm_set_fused_steps(sim, int(enable)), "mpm_set_fused_steps")


def mpm_read_particles(sim: int, x=None, v=None, C=None, F_or_J=None, stream=None) -> None:
    _check(lib().mpm_read_particles(sim, _addr(x), _addr(v), _addr(C), _addr(F_or_J), _stream(stream)),
           "mpm_read_particles")


def mpm_run_noalloc(params: mpm_params, n_particles: int, x, v=None, C=None, F_or_J=None, E_p=None,
                    n_steps: int = 1, status=None, stream=None) -> None:
    _check(lib().mpm_run_noalloc(ctypes.byref(params), int(n_particles), _addr(x), _addr(v), _addr(C),
                                 _addr(F_or_J), _addr(E_p), int(n_steps), _addr(status), _stream(stream)),
           "mpm_run_noalloc")


def mpm_read_plastic_state(sim: int, alpha, stream=None) -> None:
    _check(lib().mpm_read_plastic_state(sim, _addr(alpha), _stream(stream)), "mpm_read_plastic_state")


def mpm_read_grid(sim: int, mass=None, momentum=None, stream=None) -> None:
    _check(lib().mpm_read_grid(sim, _addr(mass), _addr(momentum), _stream(stream)), "mpm_read_grid")


def mpm_status(sim: int, status_device, stream=None) -> None:
    _check(lib().mpm_status(sim, _addr(status_device), _stream(stream)), "mpm_status")


def mpm_steps_taken(sim: int) -> int:
    return int(lib().mpm_steps_taken(sim))


def mpm_num_kernels() -> int:
    return int(lib().mpm_num_kernels())


def mpm_kernel_name(k: int) -> str:
    r = lib().mpm_kernel_name(int(k))
    return r.decode() if r else None


def mpm_launch_config(sim: int) -> dict:
    """The launch configuration chosen at creation: particles per chunk, P2G
    windows per wavefront, kernels of the step's sort."""
    buf = (ctypes.c_int32 * 3)()
    _check(lib().mpm_launch_config(sim, buf), "mpm_launch_config")
    return {"chunk": int(buf[0]), "p2g_windows": int(buf[1]), "sort_kernels": int(buf[2])}


def mpm_step_profiled(sim: int, n_steps: int, stream=None):
    """Returns the per-kernel elapsed milliseconds summed over n_steps."""
    nk = mpm_num_kernels()
    buf = (ctypes.c_float * nk)()
    _check(lib().mpm_step_profiled(sim, int(n_steps), _stream(stream), buf), "mpm_step_profiled")
    return {mpm_kernel_name(k): float(buf[k]) for k in range(nk)}


def mpm_destroy(sim: int) -> None:
    if sim:
        lib().mpm_destroy(sim)


# ----------------------------------------------------- torch convenience

class Simulation:
    """Owns a workspace (torch uint8 tensor on the device) and a handle.

    ``scene`` is a :class:`material_point_physics_amd.scenes.Scene` or any
    object with the same fields.  Inputs are uploaded from numpy once.
    """

    def __init__(self, scene, device="cuda", stream=None):
        import numpy as np
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        p = scene.params()
        self.params = make_params(**p)
        self.n = p["n"]
        self.material = p["material"]
        self.N = scene.N
        nbytes = mpm_workspace_bytes(self.params, self.N)
        if nbytes == 0:
            raise MpmError(MPM_ERR_INVALID_ARG, "mpm_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self._ws_addr = (base + 255) // 256 * 256
        self._ws_bytes = nbytes
        dev = lambda a, shape: (None if a is None else
                                torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32)).reshape(shape))
                                .to(self.device))
        x0 = dev(scene.x, (self.N, 3))
        v0 = dev(scene.v, (self.N, 3))
        C0 = dev(getattr(scene, "C", None), (self.N, 3, 3))
        if self.material == MPM_J_FLUID:
            F0 = dev(getattr(scene, "J", None), (self.N,))
        else:
            F0 = dev(getattr(scene, "F", None), (self.N, 3, 3))
        E0 = dev(scene.E_p, (self.N,))
        with torch.cuda.stream(self.stream):
            self.handle = mpm_create(self.params, self.N, x0, v0, C0, F0, E0, self._ws_addr, self._ws_bytes,
                                     self.stream)
        self.stream.synchronize()  # inputs may be released after this
        del x0, v0, C0, F0, E0

    def launch_config(self) -> dict:
        return mpm_launch_config(self.handle)

    def step(self, k: int = 1):
        mpm_step(self.handle, k, self.stream)

    def set_sort_policy(self, max_interval: int, mover_budget: int):
        mpm_set_sort_policy(self.handle, max_interval, mover_budget, self.stream)

    def set_fused_steps(self, enable: bool):
        mpm_set_fused_steps(self.handle, 1 if enable else 0)

    def read_particles(self):
        torch = self.torch
        N = self.N
        x = torch.empty((N, 3), dtype=torch.float32, device=self.device)
        v = torch.empty((N, 3), dtype=torch.float32, device=self.device)
        C = torch.empty((N, 3, 3), dtype=torch.float32, device=self.device)
        F = torch.empty((N,) if self.material == MPM_J_FLUID else (N, 3, 3), dtype=torch.float32,
                        device=self.device)
        mpm_read_particles(self.handle, x, v, C, F, self.stream)
        self.stream.synchronize()
        return x, v, C, F

    def read_plastic_state(self):
        """Snow: each particle's log plastic volume ln J_P, (N,)."""
        a = self.torch.empty((self.N,), dtype=self.torch.float32, device=self.device)
        mpm_read_plastic_state(self.handle, a, self.stream)
        self.stream.synchronize()
        return a

    def read_grid(self):
        torch = self.torch
        n = self.n
        m = torch.empty((n, n, n), dtype=torch.float32, device=self.device)
        p = torch.empty((n, n, n, 3), dtype=torch.float32, device=self.device)
        mpm_read_grid(self.handle, m, p, self.stream)
        self.stream.synchronize()
        return m, p

    def status(self):
        torch = self.torch
        st = torch.zeros(MPM_STATUS_WORDS, dtype=torch.int32, device=self.device)
        mpm_status(self.handle, st, self.stream)
        self.stream.synchronize()
        return [int(v) & 0xFFFFFFFF for v in st.cpu().tolist()]

    def close(self):
        if getattr(self, "handle", None):
            self.stream.synchronize()
            mpm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
