#!/usr/bin/env python3
"""Throughput of one explicit MLS-MPM step on one MI355X.

A "step" is one pass of the whole hot path (bucket sort by block, P2G with
fused stress, grid update, G2P) over the resident particle set, replayed as a
HIP graph through the C ABI.  The default workload is the 12M-particle
heterogeneous slab on a 256^3 grid.

Printed JSON line (rank 0, N=1):
  value          particle-steps/s over K timed steps (inputs resident in HBM)
  roofline       dominant kernel: algorithmic bytes per launch / its average
                 launch time (HIP events around each kernel on the stream it
                 runs on, measured in eager profiled steps), vs 8 TB/s
  cpu_baseline   the serial fp64 oracle timed on this host on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "particle-steps/sec at 12M particles (256^3 grid) + achieved HBM GB/s"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_bytes(N: int, active_nodes: int, nbins: int, material: int, has_E: bool, sorted_steps=True,
                 fused=False) -> dict:
    """Algorithmic HBM bytes per launch of each kernel (what the method must
    move through that kernel; see the byte model in the design notes).
    fp32 everywhere; F is 9 floats (elastic, sand) or 1 (fluid J).  With
    sorted_steps=False (free-zone steps without a sort) the scatter moves
    nothing and P2G reads the key word (4 B) instead of perm and the cell
    byte (5 B).  With fused=True (fused steps without a sort) the separate
    P2G moves nothing and the G2P2G kernel reads x, F, E and writes x and F
    back (ids and moduli stay at their slots between sorts), plus v and C (stored on the last step of each launch, and on every
    profiled step), and per active node reads the window once, writes the
    next accumulator and clears the one of two steps before."""
    f = 4 if material == 1 else 36  # fluid J, else F (elastic, sand, snow)
    e = 4 if has_E else 0
    if fused:
        kb = kernel_bytes(N, active_nodes, nbins, material, has_E, sorted_steps=False)
        kb["k_p2g"] = 0
        # x, F (and E) read; x and F written (snow also its log plastic volume);
        # the ids and moduli stay in place between sorts
        kb["k_g2p2g"] = N * (12 + f + e) + N * (12 + f + (e if material == 3 else 0)) + N * (12 + 36) + 48 * active_nodes
        del kb["k_g2p"]
        return kb
    if not sorted_steps:
        kb = kernel_bytes(N, active_nodes, nbins, material, has_E)
        kb["k_scatter"] = 0
        kb["k_p2g"] -= N
        return kb
    return {
        # bin counts read twice, cursors written, counts zeroed
        "k_scan_tiles": 4 * nbins,
        "k_scan_bins": 12 * nbins,
        # reads the key word, writes perm and the cell byte
        "k_scatter": 9 * N,
        # reads perm, cell byte, x, v, C, F(, E), id; writes F(, E), x, id in
        # the new order; accumulator write per active node, and the clear of
        # the previous step's accumulator (one float4 per active node)
        "k_p2g": N * (4 + 1 + 12 + 12 + 36 + f + e + 4 + f + e + 12 + 4) + 32 * active_nodes,
        # reads x; writes v, C, key (the new x is formed again by the next
        # P2G from x and v); reads the accumulator (m, p) once per active node
        # and applies the grid update to it
        "k_g2p": N * (12 + 12 + 36 + 4) + 16 * active_nodes,
    }


def roctx():
    """ROCTx range push/pop (the profiler SDK's marker library), so that a
    `rocprofv3 --marker-trace` run can delimit the timed region; None when
    the library is absent (the markers are then skipped)."""
    import ctypes
    for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
        try:
            L = ctypes.CDLL(name)
        except OSError:
            continue
        L.roctxRangePushA.argtypes = [ctypes.c_char_p]
        L.roctxRangePushA.restype = ctypes.c_int
        L.roctxRangePop.restype = ctypes.c_int
        return L
    return None


def source_sha1() -> str:
    """sha1 of the kernel code: every file of csrc/ in name order, with
    comments and whitespace removed (a comment edit does not change a kernel)."""
    import hashlib
    import re
    d = os.path.join(ROOT, "material_point_physics_amd", "csrc")
    h = hashlib.sha1()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def committed_traffic(workload: str, kernel: str, mode: str = ""):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary
    profiles/<workload><mode>_all_kernels_traffic.txt (FETCH_SIZE and WRITE_SIZE runs,
    each scaled by the calibration copy; mode "_fused" for the fused steps),
    or None when that summary is missing or was taken from a different
    kernel source."""
    path = os.path.join(ROOT, "profiles", f"{workload}{mode}_all_kernels_traffic.txt")
    if not os.path.exists(path):
        return None
    sha, val = None, None
    for line in open(path):
        if line.startswith("source_sha1:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith(f"traffic {kernel}"):
            for tok in line.split():
                if tok.startswith("total_bytes="):
                    val = float(tok.split("=", 1)[1])
    if sha != source_sha1() or val is None:
        return None
    return val


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="slab_12m")
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--cpu-steps", type=int, default=1, help="oracle steps for the CPU baseline (0 = skip)")
    ap.add_argument("--sort-interval", type=int, default=0,
                    help="free-zone sort policy: sort at least every K steps (0 = sort every step, the default)")
    ap.add_argument("--fused", action="store_true",
                    help="fused G2P2G steps between sorts (mpm_set_fused_steps; use with --sort-interval)")
    ap.add_argument("--alt-fused-interval", type=int, default=32,
                    help="also time the same workload with fused steps and host-scheduled sorts every K steps "
                         "(reported as fused_steps; 0 = skip)")
    ap.add_argument("--mover-budget", type=int, default=-1,
                    help="free-zone sort policy: also sort when more particles than this left their bins "
                         "(default: N/1000)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import material_point_physics_amd as mpm
    from material_point_physics_amd import scenes

    torch.cuda.set_device(0)
    t0 = time.time()
    sc = scenes.SCENES[args.workload]()
    log(f"scene {sc.name}: N={sc.N} n={sc.n} generated in {time.time() - t0:.1f}s")
    sim = mpm.Simulation(sc)
    stream = sim.stream
    free_zone = args.sort_interval > 1
    budget = args.mover_budget if args.mover_budget >= 0 else sc.N // 1000
    if free_zone:
        sim.set_sort_policy(args.sort_interval, budget)
        log(f"free-zone sort policy: at least every {args.sort_interval} steps, or more than {budget} movers")
    if args.fused:
        sim.set_fused_steps(True)
        log("fused G2P2G steps between sorts")
    log("created; warmup")
    sim.step(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: K graph-replayed steps, synchronised on both sides
    # (a ROCTx range "mpm_timed_steps" marks it for the API-trace audit)
    rtx = roctx()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    if rtx:
        rtx.roctxRangePushA(b"mpm_timed_steps")
    ev0.record(stream)
    sim.step(args.steps)
    ev1.record(stream)
    if rtx:
        rtx.roctxRangePop()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    dev_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * t_wall / args.steps
    value = sc.N * args.steps / t_wall
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {dev_ms / args.steps:.4f} ms/step device")

    # ---- per-kernel launch times (HIP events around each kernel, same stream)
    kms = mpm.mpm_step_profiled(sim.handle, args.profile_steps, stream)
    kavg = {("k_g2p2g" if (args.fused and k == "k_g2p") else k): v / args.profile_steps for k, v in kms.items()}
    m, _ = sim.read_grid()
    mass = m.cpu().numpy()
    active_nodes = int((mass > 0).sum())
    n = sc.n
    nb = (n + 7) // 8
    pad = np.zeros((nb * 8,) * 3, bool)
    pad[:n, :n, :n] = mass > 0
    active_blocks = int(pad.reshape(nb, 8, nb, 8, nb, 8).any(axis=(1, 3, 5)).sum())
    status = sim.status()
    sim.close()
    del sim
    # The same workload with fused G2P2G steps between host-scheduled sorts
    # (a sort every K steps, no mover budget), timed the same way: reported
    # beside the headline value, which sorts every step.
    alt = None
    if args.alt_fused_interval > 0 and not args.fused and not free_zone:
        K = args.alt_fused_interval
        sim2 = mpm.Simulation(sc)
        sim2.set_sort_policy(K, 1 << 40)
        sim2.set_fused_steps(True)
        sim2.step(max(args.warmup, 8))
        torch.cuda.synchronize()
        n_alt = max(args.steps, 2 * K)
        t_a = time.perf_counter()
        sim2.step(n_alt)
        torch.cuda.synchronize()
        t_alt = time.perf_counter() - t_a
        st2 = sim2.status()
        sim2.close()
        del sim2
        alt = {"value": round(sc.N * n_alt / t_alt, 1), "unit": "particle-steps/s",
               "ms_per_step": round(1e3 * t_alt / n_alt, 5), "steps": n_alt,
               "sort": f"every {K} steps, scheduled by the host; between sorts one fused G2P2G launch per step",
               "status_clean": bool(st2[0] == 0)}
        log(f"fused steps (sort every {K}): {alt['ms_per_step']:.4f} ms/step")
    # The practical HBM ceiling on this device: a plain 1 GiB device copy
    # (read 1 GiB, write 1 GiB), median of 5, outside the timed region.  The
    # same copy calibrates the HBM-byte counters of a rocprofv3 run.
    cp_src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    cp_ms = []
    for _ in range(6):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        cp_dst.copy_(cp_src)
        e1.record()
        torch.cuda.synchronize()
        cp_ms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * cp_src.numel() * 4 / (float(np.median(cp_ms[1:])) * 1e-3) / 1e9
    del cp_src, cp_dst
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "memory_GB": round(props.total_memory / 1e9, 1)}
    log(f"device {device}; plain 1 GiB copy {copy_gbps:.0f} GB/s")
    # (snow's per-particle slot carries its log plastic volume, read and written like E_p)
    kb = kernel_bytes(sc.N, active_nodes, ((n + 3) // 4) ** 3, sc.material, sc.E_p is not None or sc.material == 3,
                      sorted_steps=not free_zone, fused=args.fused)
    kernels = {k: {"avg_ms": round(kavg[k], 5), "alg_bytes": kb[k],
                   "GBps": round(kb[k] / (kavg[k] * 1e-3) / 1e9, 1)} for k in kavg}
    dom = max(kavg, key=kavg.get)
    achieved = kb[dom] / (kavg[dom] * 1e-3) / 1e9
    traffic = committed_traffic(sc.name, dom, "_fused" if args.fused else "")
    step_bytes = sum(kb.values())
    if args.fused:
        step_bytes -= sc.N * (12 + 36) * 7 // 8  # graph-replayed steps store v and C once per 8-step launch
    log(f"kernels: {kernels}")
    log(f"active nodes {active_nodes}, active blocks {active_blocks}, status {status[:4]}")

    # ---- CPU baseline: the serial oracle on a bounded sample of the workload
    cpu = None
    if args.cpu_steps > 0:
        import oracle
        log(f"oracle: {args.cpu_steps} step(s) of the full workload on one core")
        orc = oracle.OracleSim(sc, "f64")
        t1 = time.perf_counter()
        orc.step(args.cpu_steps)
        t_cpu = time.perf_counter() - t1
        cpu_model = ""
        try:
            cpu_model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
        cpu = {"value": round(sc.N * args.cpu_steps / t_cpu, 1), "unit": "particle-steps/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{args.cpu_steps} full step(s) of {sc.name} ({sc.N} particles, {n}^3 grid), "
                         f"serial fp64 oracle, {t_cpu:.1f} s; host {cpu_model}, {os.cpu_count()} logical CPUs"}
        log(f"oracle: {t_cpu:.1f} s")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "particle-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{sc.name}: {sc.description}", "particles": sc.N, "grid": f"{n}^3",
                   "dt": sc.dt, "material": {0: "fixed-corotated", 1: "J-fluid", 2: "Drucker-Prager sand", 3: "NACC snow"}[sc.material],
                   "sort": (f"free zone: at least every {args.sort_interval} steps or above {budget} movers "
                            "(byte model assumes no sort in the timed steps)") if free_zone else "every step",
                   "fused_g2p2g": bool(args.fused)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "step_hbm": {"alg_bytes_per_step": step_bytes,
                     "GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "copy_GBps": round(copy_gbps, 1),
                     "frac_of_copy": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / copy_gbps, 4)},
        "device": device,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "fused_steps": alt,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
