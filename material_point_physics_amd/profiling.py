"""Summaries of rocprofv3 results (the rocpd SQLite database it writes).

Usage:
    python -m material_point_physics_amd.profiling <results.db> [--kernels k_] [--title TEXT]

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
    a = ap.parse_args()
    print(summarize(a.db, a.kernels, a.title))


if __name__ == "__main__":
    main()
