"""Summaries of rocprofv3 output (rocpd SQLite databases) for libmoe's kernels.

    python -m combine_topk_ids_amd.rocprof_summary trace DB [--title T] [--phases]
        per-kernel launch count and average / min / max duration (markdown);
        with --phases, per phase of the run: launches separated from the
        previous libmoe launch by more than --gap-ms (default 300) start a
        new phase, so the workloads bench.py measures one after another
        (with seconds of input generation between them) get tables of their
        own even where two of them launch the same kernel on the same grid

    python -m combine_topk_ids_amd.rocprof_summary counters \\
        --fetch FETCH_DB --write WRITE_DB --workload NAME [--json OUT]
        HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs, each scaled by
        what the same counter reads for a streaming kernel of known size
        (bench.py's reference kernel: 1 GiB read + 1 GiB written, a negation
        of a bf16 tensor), plus the source hash of the kernels measured.
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
GIB = 1 << 30
REF_KERNEL = "neg_kernel"  # bench.py's 1 GiB read + 1 GiB write reference


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"\(.*", "", name)
    return name.replace("void ", "")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def trace_table(db: str, only_moe: bool = True) -> list[dict]:
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), "
        "grid_x, workgroup_x from kernels group by name, grid_x order by sum(duration) desc"
    ).fetchall()
    out = []
    for n, c, a, mi, ma, gx, wx in rows:
        if only_moe and "moe::" not in n:
            continue
        out.append(dict(kernel=short_name(n), calls=c, avg_us=a / 1e3, min_us=mi / 1e3,
                        max_us=ma / 1e3, grid=f"{gx // max(wx, 1)}x{wx}"))
    return out


def trace_phases(db: str, gap_ms: float = 300.0) -> list[list[dict]]:
    """trace_table split into phases of the run (see the module docstring)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end, duration, grid_x, workgroup_x from kernels "
                       "order by start").fetchall()
    phases, cur, last_end = [], [], None
    for n, st, en, d, gx, wx in rows:
        if "moe::" not in n:
            continue
        if last_end is not None and st - last_end > gap_ms * 1e6:
            phases.append(cur)
            cur = []
        cur.append((n, d, gx, wx))
        last_end = en if last_end is None else max(last_end, en)
    if cur:
        phases.append(cur)
    out = []
    for ph in phases:
        groups = collections.OrderedDict()
        for n, d, gx, wx in ph:
            groups.setdefault((n, gx, wx), []).append(d)
        tab = []
        for (n, gx, wx), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            tab.append(dict(kernel=short_name(n), calls=len(ds), avg_us=sum(ds) / len(ds) / 1e3,
                            min_us=min(ds) / 1e3, max_us=max(ds) / 1e3,
                            grid=f"{gx // max(wx, 1)}x{wx}"))
        out.append(tab)
    return out


def counter_table(db: str, counter: str) -> dict:
    con = sqlite3.connect(db)
    rows = con.execute(
        "select kernel_name, grid_size, count(*), avg(value) from counters_collection "
        "where counter_name = ? group by kernel_name, grid_size", (counter,)).fetchall()
    out = collections.defaultdict(list)
    for n, g, c, kib in rows:
        out[short_name(n)].append(dict(grid=g, calls=c, kib=kib))
    return out


def _ref_factor(table: dict) -> float:
    ref = [r for n, rs in table.items() if REF_KERNEL in n for r in rs]
    if not ref:
        raise SystemExit(f"no {REF_KERNEL} dispatch found for calibration")
    kib = max(r["kib"] for r in ref)
    return GIB / (kib * 1024.0)


def counters(fetch_db: str, write_db: str, workload: str) -> dict:
    ft, wt = counter_table(fetch_db, "FETCH_SIZE"), counter_table(write_db, "WRITE_SIZE")
    f_fetch, f_write = _ref_factor(ft), _ref_factor(wt)
    kernels = {}
    for name in sorted(set(ft) | set(wt)):
        if "moe::" not in name:
            continue
        fr, wr = ft.get(name, []), wt.get(name, [])
        calls = sum(r["calls"] for r in fr)
        fkib = sum(r["kib"] * r["calls"] for r in fr) / max(calls, 1)
        wcalls = sum(r["calls"] for r in wr)
        wkib = sum(r["kib"] * r["calls"] for r in wr) / max(wcalls, 1)
        base = re.sub(r"<.*", "", name.split("::")[-1])
        kernels[base] = dict(
            name=name, launches=calls, fetch_kib_raw=round(fkib, 2), write_kib_raw=round(wkib, 2),
            hbm_read_bytes=int(fkib * 1024 * f_fetch), hbm_write_bytes=int(wkib * 1024 * f_write),
            hbm_bytes_per_launch=int(fkib * 1024 * f_fetch + wkib * 1024 * f_write))
    return dict(workload=workload, source_hash=kernel_source_hash(),
                calibration=dict(kernel=REF_KERNEL, bytes_read=GIB, bytes_written=GIB,
                                 fetch_factor=round(f_fetch, 4), write_factor=round(f_write, 4)),
                kernels=kernels)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--title", default="")
    t.add_argument("--phases", action="store_true")
    t.add_argument("--gap-ms", type=float, default=300.0)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--json")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        tables = trace_phases(a.db, a.gap_ms) if a.phases else [trace_table(a.db)]
        if a.title:
            print(f"### {a.title}\n")
        for i, rows in enumerate(tables):
            if a.phases:
                print(f"Phase {i + 1}\n")
            print("| kernel | grid (blocks x threads) | launches | avg us | min us | max us |")
            print("|---|---|---|---|---|---|")
            for r in rows:
                print(f"| {r['kernel']} | {r['grid']} | {r['calls']} | {r['avg_us']:.2f} | "
                      f"{r['min_us']:.2f} | {r['max_us']:.2f} |")
            print()
    else:
        rec = counters(a.fetch, a.write, a.workload)
        text = json.dumps(rec, indent=1)
        if a.json:
            with open(a.json, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    main()
