"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m ternary_weight_decode_amd.rocprof_summary trace DIR [--kernel RE] [--window A:B]
    python -m ternary_weight_decode_amd.rocprof_summary pmc DIR [--kernel RE] [--window A:B]

``trace`` reads the kernel-trace CSV under DIR (``--kernel-trace -f csv``) and
prints, per kernel and grid size, the dispatch count and the mean / median /
min / max device duration.  ``pmc`` reads the counter-collection CSV
(``--pmc ... -f csv``) and prints, per kernel and grid size, the median and
mean of every counter per dispatch.  ``--kernel`` keeps kernels whose name
matches the regular expression; ``--window A:B`` keeps the matching
dispatches with ordinal A <= i < B (in dispatch order over every kernel the
expression keeps), e.g. the launches of a benchmark's timed region.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[-1]


def _col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def short_name(name: str) -> str:
    """Kernel name without namespaces and argument lists, template arguments kept."""
    name = re.sub(r"^void\s+", "", name.strip())
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        out.append(ch)
    return re.sub(r"\btern::", "", "".join(out)).strip()


def _window(rows, spec):
    if not spec:
        return rows
    a, b = spec.split(":")
    return rows[int(a or 0):int(b) if b else None]


def load_trace(d: str, kernel: str | None, window: str | None):
    rows = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    out = []
    for r in rows:
        name = short_name(_col(r, "Kernel_Name"))
        if kernel and not re.search(kernel, name):
            continue
        grid = int(_col(r, "Grid_Size_X", "Grid_Size")) * int(r.get("Grid_Size_Y", 1) or 1) * \
            int(r.get("Grid_Size_Z", 1) or 1)
        wg = int(_col(r, "Workgroup_Size_X", "Workgroup_Size"))
        ns = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
        out.append((int(_col(r, "Dispatch_Id")), name, grid, wg, ns))
    out.sort()
    return _window(out, window)


def cmd_trace(args):
    rows = load_trace(args.dir, args.kernel, args.window)
    groups = {}
    for (_, name, grid, wg, ns) in rows:
        groups.setdefault((name, grid, wg), []).append(ns)
    print(f"{'kernel':60s} {'grid':>9s} {'wg':>5s} {'calls':>6s} {'mean_us':>9s} {'median_us':>9s} "
          f"{'min_us':>8s} {'max_us':>8s}")
    for (name, grid, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name[:60]:60s} {grid:9d} {wg:5d} {len(v):6d} {statistics.mean(v) / 1e3:9.3f} "
              f"{statistics.median(v) / 1e3:9.3f} {min(v) / 1e3:8.3f} {max(v) / 1e3:8.3f}")
    allv = [r[4] for r in rows]
    if allv:
        print(f"all kept dispatches: {len(allv)}, mean {statistics.mean(allv) / 1e3:.3f} us, "
              f"median {statistics.median(allv) / 1e3:.3f} us")


def cmd_pmc(args):
    rows = list(csv.DictReader(open(_find(args.dir, "counter_collection.csv"))))
    per = {}
    for r in rows:
        name = short_name(_col(r, "Kernel_Name"))
        if args.kernel and not re.search(args.kernel, name):
            continue
        did = int(_col(r, "Dispatch_Id"))
        grid = int(_col(r, "Grid_Size"))
        wg = int(_col(r, "Workgroup_Size"))
        d = per.setdefault(did, {"name": name, "grid": grid, "wg": wg, "c": {}})
        cn = _col(r, "Counter_Name")
        d["c"][cn] = d["c"].get(cn, 0.0) + float(_col(r, "Counter_Value"))
    disp = _window([per[k] for k in sorted(per)], args.window)
    groups = {}
    for d in disp:
        g = groups.setdefault((d["name"], d["grid"], d["wg"]), {})
        for cn, v in d["c"].items():
            g.setdefault(cn, []).append(v)
    for (name, grid, wg), cs in groups.items():
        n = max(len(v) for v in cs.values())
        print(f"{name}  grid={grid} wg={wg} dispatches={n}")
        for cn in sorted(cs):
            v = cs[cn]
            print(f"  {cn:32s} median {statistics.median(v):16.1f}   mean {statistics.mean(v):16.1f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("trace", "pmc"):
        p = sub.add_parser(name)
        p.add_argument("dir")
        p.add_argument("--kernel", default=None)
        p.add_argument("--window", default=None)
    args = ap.parse_args(argv)
    (cmd_trace if args.cmd == "trace" else cmd_pmc)(args)


if __name__ == "__main__":
    main()
