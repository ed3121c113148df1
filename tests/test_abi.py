"""The C-ABI library loads on the CPU, exports every symbol include/mpm.h
declares, and rejects invalid arguments on the host before any GPU work.
No compute call is made here."""
import ctypes
import os
import re

import pytest

import material_point_physics_amd as mpm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mpm.EXPORTS)


def declaration_comments():
    """Each function declaration of the header with the comment block right
    before it (a declaration may share the comment of the one before it
    when they are adjacent, as mpm_num_kernels and mpm_kernel_name do)."""
    text = open(HEADER).read()
    out = {}
    last_comment = ""
    pos = 0
    for m in re.finditer(r"/\*.*?\*/|\b(mpm_[a-z_]+)\s*\(", text, flags=re.S):
        if m.group(0).startswith("/*"):
            last_comment = m.group(0)
            pos = m.end()
            continue
        name = m.group(1)
        between = text[pos:m.start()]
        # the comment belongs to this declaration if only code of the
        # declarations since it lies in between
        if ";" in between and not re.search(r"mpm_[a-z_]+\s*\(", between):
            last_comment = ""
        out.setdefault(name, last_comment)
    return out


def test_every_declaration_cites_the_page():
    """Each entry point's comment names the passage of the MPM page it
    follows (its problem statement, a single-GPU principle, a figure, the
    free zone, the fused kernel, a scene or a section)."""
    cites = declaration_comments()
    assert set(cites) == set(declared_functions())
    for name, comment in cites.items():
        if name == "mpm_run_noalloc":
            # not a step of the page's method: its comment names the callers it serves
            assert "cannot allocate" in comment, comment[:120]
            continue
        assert re.search(r"\bpage'?s?\b", comment), (name, comment[:120])
        assert re.search(r"principle|problem statement|Fig\.|§|free zone|fused|scene|discussion|study",
                         comment), (name, comment[:120])


def test_library_exports_every_declared_symbol():
    L = mpm.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {mpm.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_library_is_gfx950_only():
    """The embedded offload bundle names gfx950 and no other GPU target."""
    data = open(mpm.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[a-z-]*(gfx[0-9a-f]+)", data))
    assert targets == {b"gfx950"}, targets


def good_params(**kw):
    d = dict(n=32, dt=1e-4, gravity=(0, -9.8, 0), wall=3, material=0, E=1e4, nu=0.2, rho=1.0, p_vol=1e-6)
    d.update(kw)
    return mpm.make_params(**d)


def test_workspace_bytes_scales_and_rejects_bad_params():
    a = mpm.mpm_workspace_bytes(good_params(), 1000)
    b = mpm.mpm_workspace_bytes(good_params(), 2000)
    c = mpm.mpm_workspace_bytes(good_params(n=64), 1000)
    assert 0 < a < b and a < c
    assert mpm.mpm_workspace_bytes(good_params(), 0) > 0
    for bad in [dict(n=4), dict(n=2048), dict(dt=0.0), dict(dt=float("nan")), dict(wall=-1), dict(wall=20),
                dict(material=7), dict(E=-1.0), dict(nu=0.5), dict(rho=0.0), dict(p_vol=0.0),
                dict(gravity=(0, float("inf"), 0))]:
        assert mpm.mpm_workspace_bytes(good_params(**bad), 1000) == 0, bad
    # snow: a positive modulus and M, non-negative beta and xi, a finite initial log plastic volume
    assert mpm.mpm_workspace_bytes(good_params(material=3), 1000) > 0
    assert mpm.mpm_workspace_bytes(good_params(material=3, snow_beta=0.0, snow_xi=0.0, snow_alpha0=0.3), 1000) > 0
    for bad in [dict(E=0.0), dict(snow_M=0.0), dict(snow_M=float("inf")), dict(snow_beta=-0.1),
                dict(snow_xi=-1.0), dict(snow_xi=float("nan")), dict(snow_alpha0=float("inf"))]:
        assert mpm.mpm_workspace_bytes(good_params(material=3, **bad), 1000) == 0, bad
    assert mpm.mpm_workspace_bytes(good_params(material=0, E=0.0, snow_M=0.0), 1000) > 0  # read only for snow
    assert mpm.mpm_workspace_bytes(good_params(), -1) == 0
    assert mpm.mpm_workspace_bytes(good_params(), 1 << 31) == 0
    assert mpm.mpm_workspace_bytes(good_params(), 1 << 28) == 0  # 32-bit element offsets
    assert mpm.mpm_workspace_bytes(good_params(), (1 << 28) - 1) > 0
    p = good_params()
    p.struct_size = 8
    assert mpm.mpm_workspace_bytes(p, 10) == 0


def test_create_rejects_bad_arguments_before_any_launch():
    L = mpm.lib()
    p = good_params()
    need = mpm.mpm_workspace_bytes(p, 100)
    out = ctypes.c_void_p(123)
    fake = 1 << 40  # never dereferenced: every case below fails host validation
    # NULL out pointer
    assert L.mpm_create(ctypes.byref(p), 100, fake, None, None, None, None, fake, need, None, None) == mpm.MPM_ERR_INVALID_ARG
    # invalid params
    bad = good_params(n=3)
    assert L.mpm_create(ctypes.byref(bad), 100, fake, None, None, None, None, fake, need, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_INVALID_ARG
    assert out.value is None
    # negative N, missing positions
    assert L.mpm_create(ctypes.byref(p), -5, fake, None, None, None, None, fake, need, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_create(ctypes.byref(p), 100, None, None, None, None, None, fake, need, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_INVALID_ARG
    # workspace: missing, misaligned, too small
    assert L.mpm_create(ctypes.byref(p), 100, fake, None, None, None, None, None, need, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_WORKSPACE
    assert L.mpm_create(ctypes.byref(p), 100, fake, None, None, None, None, fake + 4, need, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_WORKSPACE
    assert L.mpm_create(ctypes.byref(p), 100, fake, None, None, None, None, fake, need - 1, None,
                        ctypes.byref(out)) == mpm.MPM_ERR_WORKSPACE
    assert out.value is None


def test_null_handle_calls_are_rejected():
    L = mpm.lib()
    assert L.mpm_step(None, 1, None) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_set_sort_policy(None, 8, 1000, None) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_set_fused_steps(None, 1) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_read_particles(None, None, None, None, None, None) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_read_grid(None, None, None, None) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_status(None, None, None) == mpm.MPM_ERR_INVALID_ARG
    assert L.mpm_steps_taken(None) == -1
    buf = (ctypes.c_float * 8)()
    assert L.mpm_step_profiled(None, 1, None, buf) == mpm.MPM_ERR_INVALID_ARG
    L.mpm_destroy(None)  # no-op


def test_error_strings_and_kernel_names():
    for code in [0, -1, -2, -3, -4]:
        assert mpm.mpm_error_string(code) != "unknown error"
    assert mpm.mpm_error_string(-99) == "unknown error"
    nk = mpm.mpm_num_kernels()
    assert nk == 5
    names = [mpm.mpm_kernel_name(k) for k in range(nk)]
    assert names == ["k_scan_tiles", "k_scan_bins", "k_scatter", "k_p2g", "k_g2p"]
    assert mpm.mpm_kernel_name(nk) is None and mpm.mpm_kernel_name(-1) is None


def test_params_struct_matches_header():
    # the binding's fields are the header's, in order, with the same C types
    import re
    hdr = open(os.path.join(ROOT, "include", "mpm.h")).read()
    body = re.search(r"typedef struct \{(.*?)\} mpm_params;", hdr, re.S).group(1)
    decl = [re.match(r"\s*(\w+)\s+(\w+)(\[\d+\])?;", l).groups() for l in body.strip().splitlines()]
    ctype = {"uint32_t": ctypes.c_uint32, "int32_t": ctypes.c_int32, "float": ctypes.c_float}
    assert [f[0] for f in mpm.mpm_params._fields_] == [d[1] for d in decl]
    for (name, ct), (ty, _, arr) in zip(mpm.mpm_params._fields_, decl):
        want = ctype[ty] * int(arr[1:-1]) if arr else ctype[ty]
        assert ctypes.sizeof(ct) == ctypes.sizeof(want), name
    # uint32 + int32 + float + float[3] + int32 + int32 + 9 floats = 68 bytes
    assert ctypes.sizeof(mpm.mpm_params) == 68


def test_run_noalloc_rejects_on_the_host():
    """mpm_run_noalloc checks its arguments and its size limit before any HIP
    call (so these run without a GPU): a problem whose workspace exceeds the
    static scratch, the snow material, negative counts, a missing x."""
    big = good_params(n=128)
    assert mpm.mpm_workspace_bytes(big, 100000) > mpm.MPM_NOALLOC_SCRATCH_BYTES
    L = mpm.lib()

    def run(prm, n, x=1 << 20, steps=1):
        return L.mpm_run_noalloc(ctypes.byref(prm), n, x, None, None, None, None, steps, None, None)

    assert run(big, 100000) == mpm.MPM_ERR_TOO_LARGE
    assert run(good_params(material=3), 1000) == mpm.MPM_ERR_INVALID_ARG
    assert run(good_params(), -1) == mpm.MPM_ERR_INVALID_ARG
    assert run(good_params(), 1000, steps=-1) == mpm.MPM_ERR_INVALID_ARG
    assert run(good_params(), 1000, x=None) == mpm.MPM_ERR_INVALID_ARG
    assert run(good_params(n=4), 1000) == mpm.MPM_ERR_INVALID_ARG
    assert "scratch" in mpm.mpm_error_string(mpm.MPM_ERR_TOO_LARGE)


def test_committed_api_trace_shows_no_sync_or_allocation_between_steps():
    """The committed HIP API trace of bench.py's timed region (rocprofv3
    --hip-trace, delimited by a ROCTx range): the steps are graph launches,
    and no synchronisation, device-to-host copy or allocation occurs between
    them (the page's CPU-GPU synchronisation and memory-reallocation
    principles, Figs. 3 and 4)."""
    path = os.path.join(ROOT, "profiles", "jelly3_55k_timed_steps_hip_api.txt")
    calls = {}
    forbidden_line = None
    for line in open(path):
        m = re.match(r"^(hip[A-Za-z0-9_]+)\s+(\d+)\s*$", line)
        if m:
            calls[m.group(1)] = int(m.group(2))
        if line.startswith("forbidden calls"):
            forbidden_line = line
    assert forbidden_line is not None and forbidden_line.strip().endswith(": none")
    assert calls.get("hipGraphLaunch", 0) == 50 // 8 + 50 % 8
    for name in calls:
        for bad in ("Synchronize", "hipMemcpy", "hipMalloc", "hipFree", "hipMemset", "Query"):
            assert bad not in name, name
