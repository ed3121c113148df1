"""Summaries of rocprofv3 results (the rocpd SQLite database it writes).

Usage:
    python -m material_point_physics_amd.profiling <results.db> [--kernels k_] [--title TEXT]
    python -m material_point_physics_amd.profiling <fetch.db> --write-db <write.db>
    python -m material_point_physics_amd.profiling <rdreq.db> --request-write-db <wrreq.db>
    python -m material_point_physics_amd.profiling <trace.db> --api-audit

Prints, per kernel: number of dispatches, average / median / total duration
(from the kernel trace), and the per-dispatch median of every collected
hardware counter.  Medians keep one-off dispatches (such as a first step
from an unsorted initial state) from skewing the steady-state figures.
Used to produce the text summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import collections
import sqlite3


def short_name(full: str) -> str:
    s = full.replace("(anonymous namespace)::", "").replace("void ", "")
    return s.split("(")[0].strip()


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def kernel_times(db: str):
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select name, duration from kernels").fetchall()
    acc = collections.defaultdict(list)
    for name, dur in rows:
        acc[short_name(name)].append(float(dur))
    return {k: (len(v), sum(v) / len(v), median(v), sum(v)) for k, v in acc.items()}


def kernel_counters(db: str):
    cur = sqlite3.connect(db).cursor()
    try:
        rows = cur.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
    except sqlite3.OperationalError:
        return {}
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    kname = {}
    for did, kn, cn, val in rows:
        per[did][cn] += float(val)
        kname[did] = short_name(kn)
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for did, cs in per.items():
        for cn, v in cs.items():
            acc[kname[did]][cn].append(v)
    return {k: {c: median(v) for c, v in d.items()} for k, d in acc.items()}


def summarize(db: str, kernels: str = "", title: str = "") -> str:
    out = []
    if title:
        out.append(title)
    times = kernel_times(db)
    ctrs = kernel_counters(db)
    out.append(f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'total_us':>12s}")
    for k in sorted(times, key=lambda k: -times[k][3]):
        if kernels and kernels not in k:
            continue
        n, avg, med, tot = times[k]
        out.append(f"{k:40s} {n:6d} {avg / 1e3:10.2f} {med / 1e3:10.2f} {tot / 1e3:12.1f}")
    if ctrs:
        out.append("")
        out.append("counters (median per dispatch)")
        for k in sorted(ctrs):
            if kernels and kernels not in k:
                continue
            cs = ", ".join(f"{c}={v:.6g}" for c, v in sorted(ctrs[k].items()))
            out.append(f"  {k}: {cs}")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--kernels", default="")
    ap.add_argument("--title", default="")
    ap.add_argument("--write-db", default="", help="with a FETCH_SIZE db: print copy-calibrated traffic")
    ap.add_argument("--request-write-db", default="",
                    help="with a TCC_EA0_RDREQ/RDREQ_32B/BUBBLE db: print the request-size traffic range, "
                         "the writes from this TCC_EA0_WRREQ/WRREQ_64B db")
    ap.add_argument("--api-audit", action="store_true",
                    help="with a --hip-trace --marker-trace db: HIP calls inside the timed range")
    a = ap.parse_args()
    if a.api_audit:
        print(api_audit_text(a.db, a.title))
        return
    if a.request_write_db:
        for k, v in request_traffic(a.db, a.request_write_db, a.kernels or "k_").items():
            print(f"requests {k} read_bytes=[{v['read_lo']:.6g}, {v['read_hi']:.6g}] write_bytes={v['write']:.6g} "
                  f"total_bytes=[{v['total_lo']:.6g}, {v['total_hi']:.6g}] ea_atomics={v['atomics']:.6g}")
        return
    if a.write_db:
        t = traffic(a.db, a.write_db, a.kernels or "k_")
        print(f"copy calibration: FETCH_SIZE x {t['fetch_factor']:.4f}, WRITE_SIZE x {t['write_factor']:.4f}")
        for k, v in t["kernels"].items():
            print(f"traffic {k} fetch_bytes={v['fetch_bytes']:.6g} write_bytes={v['write_bytes']:.6g} "
                  f"total_bytes={v['total_bytes']:.6g}")
    else:
        print(summarize(a.db, a.kernels, a.title))



# ------------------------------------------------------------ HBM traffic

COPY_KIB = 1048576  # the benchmark's plain device copy: 1 GiB read, 1 GiB written


def copy_calibration(db: str, counter: str, known_kib: float = COPY_KIB) -> float:
    """Scale factor for `counter` (FETCH_SIZE or WRITE_SIZE, KiB per dispatch):
    known bytes of the benchmark's plain 1 GiB device copy divided by what
    the counter reads for that copy (the copy dispatch with the largest value:
    no other copy in the benchmark moves as much)."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select dispatch_id, kernel_name, value from counters_collection where counter_name = ?",
                       (counter,)).fetchall()
    per = collections.defaultdict(float)
    for did, kn, val in rows:
        if "copy" in kn.lower():
            per[did] += float(val)
    if not per:
        raise ValueError(f"no copy dispatch with {counter} in {db}")
    return known_kib / max(per.values())


def traffic(fetch_db: str, write_db: str, kernels: str = "k_"):
    """Per-kernel HBM bytes per dispatch (median), each counter scaled by its
    copy calibration factor."""
    fk = copy_calibration(fetch_db, "FETCH_SIZE")
    wk = copy_calibration(write_db, "WRITE_SIZE")
    fc = kernel_counters(fetch_db)
    wc = kernel_counters(write_db)
    out = {}
    for k in sorted(set(fc) | set(wc)):
        if kernels and kernels not in k:
            continue
        f = fc.get(k, {}).get("FETCH_SIZE", 0.0) * fk * 1024
        w = wc.get(k, {}).get("WRITE_SIZE", 0.0) * wk * 1024
        out[k] = {"fetch_bytes": f, "write_bytes": w, "total_bytes": f + w}
    return {"fetch_factor": fk, "write_factor": wk, "kernels": out}


def request_traffic(read_db: str, write_db: str, kernels: str = "k_"):
    """Per-kernel HBM bytes per dispatch (median) from the request counters
    of the L2-to-fabric interface, without a calibration factor:
      reads: TCC_EA0_RDREQ_sum requests, of which TCC_EA0_RDREQ_32B_sum carry
             32 B and TCC_BUBBLE_sum 128 B; the rest carry 64 or 128 B (no
             counter tells them apart), so the read bytes lie in
             [32 R32 + 64 (R - R32 - B128) + 128 B128,  32 R32 + 128 (R - R32)]
             -- the lower end is rocprofv3's FETCH_SIZE;
      writes: TCC_EA0_WRREQ_sum transactions of 32 or 64 B, of which
             TCC_EA0_WRREQ_64B_sum carry 64 B (WRITE_SIZE), atomics included.
    A streaming copy's reads sit at the upper end (one request per 128-byte
    line), which is why a FETCH_SIZE calibrated on the copy is this range's
    upper end."""
    rc = kernel_counters(read_db)
    wc = kernel_counters(write_db)
    out = {}
    for k in sorted(set(rc) | set(wc)):
        if kernels and kernels not in k:
            continue
        r = rc.get(k, {})
        R, R32, B = r.get("TCC_EA0_RDREQ_sum", 0.0), r.get("TCC_EA0_RDREQ_32B_sum", 0.0), r.get("TCC_BUBBLE_sum", 0.0)
        w = wc.get(k, {})
        W, W64 = w.get("TCC_EA0_WRREQ_sum", 0.0), w.get("TCC_EA0_WRREQ_64B_sum", 0.0)
        lo = 32 * R32 + 64 * (R - R32 - B) + 128 * B
        hi = 32 * R32 + 128 * (R - R32)
        wb = 32 * (W - W64) + 64 * W64
        out[k] = {"read_lo": lo, "read_hi": hi, "write": wb, "total_lo": lo + wb, "total_hi": hi + wb,
                  "atomics": w.get("TCC_EA0_ATOMIC_sum", 0.0)}
    return out


# ------------------------------------------------------- host-API audit

# HIP calls that would stall the host on the device, copy device data back,
# or allocate: none may occur between two steps.
FORBIDDEN_API = ("Synchronize", "hipMemcpy", "hipMalloc", "hipFree", "hipHostMalloc", "hipHostFree",
                 "hipMemset", "hipStreamQuery", "hipEventQuery", "hipDeviceReset")


def api_audit(db: str, marker: str = "mpm_timed_steps"):
    """HIP runtime calls made on the thread of the ROCTx range `marker`
    while it was open (a `rocprofv3 --hip-trace --marker-trace` database):
    returns (calls by name, the range's duration in ns, forbidden names seen)."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select category, name, tid, start, end, id from regions").fetchall()
    # rocprofv3 records a ROCTx range under the API name (roctxThreadRangeA)
    # with the message among the region's arguments
    msgs = collections.defaultdict(list)
    try:
        for rid, val in cur.execute("select id, value from region_args"):
            msgs[rid].append(str(val))
    except sqlite3.OperationalError:
        pass
    rng = [r for r in rows if r[1] == marker or ("MARKER" in str(r[0]).upper() and marker in msgs.get(r[5], []))]
    if not rng:
        # (the message is not always stored: then the run's only ROCTx range,
        # which bench.py opens around its timed steps and nowhere else)
        rng = [r for r in rows if "MARKER" in str(r[0]).upper() and "RANGE" in str(r[0]).upper()]
    if len(rng) != 1:
        raise ValueError(f"expected one '{marker}' range in {db}, found {len(rng)}")
    _, _, tid, t0, t1, _ = rng[0]
    calls = collections.Counter(r[1] for r in rows
                                if r[2] == tid and t0 <= r[3] <= t1 and r[1] != marker
                                and "MARKER" not in str(r[0]).upper())
    bad = sorted(n for n in calls if any(f in n for f in FORBIDDEN_API))
    return calls, t1 - t0, bad


def api_audit_text(db: str, title: str = "") -> str:
    calls, dur, bad = api_audit(db)
    out = [title] if title else []
    out.append(f"timed range: {dur / 1e6:.3f} ms")
    out.append(f"{'HIP call inside the timed range':40s} {'count':>8s}")
    for n, k in sorted(calls.items(), key=lambda kv: (-kv[1], kv[0])):
        out.append(f"{n:40s} {k:8d}")
    out.append(f"forbidden calls (synchronisation, copies, allocation): {', '.join(bad) if bad else 'none'}")
    return "\n".join(out)


if __name__ == "__main__":
    main()
