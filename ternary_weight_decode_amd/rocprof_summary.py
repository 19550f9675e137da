"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m ternary_weight_decode_amd.rocprof_summary trace DIR [--kernel RE] [--window A:B]
    python -m ternary_weight_decode_amd.rocprof_summary pmc DIR [--kernel RE] [--window A:B]
    python -m ternary_weight_decode_amd.rocprof_summary runs DIR [DIR ...] --bench OUT [--kernel RE] [--passes P]
                                                             [--scale COUNTER=F ...]

``trace`` reads the kernel-trace CSV under DIR (``--kernel-trace -f csv``) and
prints, per kernel and grid size, the dispatch count and the mean / median /
min / max device duration.  ``pmc`` reads the counter-collection CSV
(``--pmc ... -f csv``) and prints, per kernel and grid size, the median and
mean of every counter per dispatch.  ``--kernel`` keeps kernels whose name
matches the regular expression; ``--window A:B`` keeps the matching
dispatches with ordinal A <= i < B (in dispatch order over every kernel the
expression keeps), e.g. the launches of a benchmark's timed region.

``runs`` splits a sweep into its cases: consecutive kept dispatches of the
same kernel and grid form one run, and the runs are matched in order with
the ``rows`` of the sweep's JSON line (the last line of OUT holding one).
Each run is P equal passes (an eager warm-up, then graph replays); the first
is dropped and the median of the rest is printed.  Where a run has k times
the dispatches of the smallest run of its unit, every call was k launches
and k consecutive dispatches are summed.  DIR holds a kernel trace or a
counter collection; for counters, ``--scale`` turns a counter's KiB into
bytes (the factor from a copy of known size) and, with a row's ``bytes``,
the ratio of measured to algorithmic bytes is printed; counters taken in
separate runs of the same sweep (one directory each) are merged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
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
        vgpr = r.get("Arch_VGPR_Count") or r.get("VGPR_Count") or "0"
        out.append((int(_col(r, "Dispatch_Id")), name, grid, wg, ns, int(vgpr)))
    out.sort()
    return _window(out, window)


def cmd_trace(args):
    rows = load_trace(args.dir, args.kernel, args.window)
    groups = {}
    for (_, name, grid, wg, ns, _) in rows:
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


def load_pmc(d: str, kernel: str | None):
    """Per dispatch (in dispatch order): name, grid, workgroup size, {counter: value}."""
    per = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        name = short_name(_col(r, "Kernel_Name"))
        if kernel and not re.search(kernel, name):
            continue
        did = int(_col(r, "Dispatch_Id"))
        e = per.setdefault(did, [name, int(_col(r, "Grid_Size")), int(_col(r, "Workgroup_Size")), {}])
        cn = _col(r, "Counter_Name")
        e[3][cn] = e[3].get(cn, 0.0) + float(_col(r, "Counter_Value"))
    return [tuple(per[k]) for k in sorted(per)]


def split_runs(disp):
    """Consecutive dispatches with the same (name, grid, workgroup size): [(key, [payload, ...])]."""
    runs = []
    for name, grid, wg, payload in disp:
        key = (name, grid, wg)
        if runs and runs[-1][0] == key:
            runs[-1][1].append(payload)
        else:
            runs.append((key, [payload]))
    return runs


def bench_rows(path: str):
    rows = None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            try:
                d = json.loads(line)
            except ValueError:
                continue
            if isinstance(d.get("rows"), list):
                rows = d["rows"]
    if rows is None:
        sys.exit(f"no JSON line with rows in {path}")
    return rows


def row_label(r: dict) -> str:
    unit = r.get("proj", r.get("unit", "?"))
    fmt = r.get("format", "")
    return f"{unit:7s}{fmt:8s}{r.get('act', ''):5s} M={r.get('M', '?'):>2}"


def _calls(vals, k, combine):
    """Sum (combine) every k consecutive dispatches into one call."""
    return [combine(vals[i:i + k]) for i in range(0, len(vals) - k + 1, k)]


def simds_per_sq(d: str):
    """SIMDs served by one SQ_BUSY_CYCLES instance (one per shader engine): Simd_Count / Num_Shader_Banks
    of the GPU agent in the run's agent-info CSV, or None."""
    hits = sorted(glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True))
    for path in hits:
        for r in csv.DictReader(open(path)):
            try:
                simds, ses = int(r.get("Simd_Count") or 0), int(r.get("Num_Shader_Banks") or 0)
            except ValueError:
                continue
            if simds > 0 and ses > 0 and "gfx" in (r.get("Name") or ""):
                return simds / ses
    return None


def sq_text(med: dict, per_sq) -> str:
    """SQ counters of one case: instructions per wave, the share of wave time spent waiting, and, with the
    SIMDs per shader engine (SQ_BUSY_CYCLES is summed over the engines, so per engine it is about the
    kernel's duration in cycles), the matrix cores' busy share per SIMD (SQ_VALU_MFMA_BUSY_CYCLES) and
    the VALU issue share per SIMD (4 cycles per wave64 VALU instruction)."""
    waves = med["SQ_WAVES"]
    out = [f"waves {waves:7.0f}"]
    for c, lab in (("SQ_INSTS_VALU", "valu"), ("SQ_INSTS_MFMA", "mfma"), ("SQ_INSTS_LDS", "lds"),
                   ("SQ_INSTS_SALU", "salu")):
        if c in med:
            out.append(f"{lab}/wave {med[c] / waves:7.1f}")
    if "SQ_WAIT_INST_ANY" in med and med.get("SQ_WAVE_CYCLES"):
        out.append(f"wait {100 * med['SQ_WAIT_INST_ANY'] / med['SQ_WAVE_CYCLES']:5.1f}%")
    if per_sq and med.get("SQ_BUSY_CYCLES"):
        simd_cycles = med["SQ_BUSY_CYCLES"] * per_sq
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            out.append(f"mfma busy {100 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:5.1f}%")
        if "SQ_INSTS_VALU" in med:
            out.append(f"valu issue {100 * 4 * med['SQ_INSTS_VALU'] / simd_cycles:5.1f}%")
    return "  ".join(out)


def cmd_runs(args):
    rows = bench_rows(args.bench)
    counters = glob.glob(os.path.join(args.dir[0], "**", "*counter_collection.csv"), recursive=True)
    if counters:
        # one counter per run of the sweep: the runs' dispatches are merged position by position
        per_dir = [split_runs(load_pmc(d, args.kernel)) for d in args.dir]
        runs = per_dir[0]
        for other in per_dir[1:]:
            if [(k, len(v)) for k, v in other] != [(k, len(v)) for k, v in runs]:
                sys.exit("the counter runs do not hold the same sequence of dispatches")
            runs = [(k, [{**a, **b} for a, b in zip(v, w)]) for (k, v), (_, w) in zip(runs, other)]
    else:
        if len(args.dir) != 1:
            sys.exit("one kernel-trace directory at a time")
        disp = [(n, g, w, (ns, vg)) for (_, n, g, w, ns, vg) in load_trace(args.dir[0], args.kernel, None)]
        runs = split_runs(disp)
    if len(runs) != len(rows):
        sys.exit(f"{len(runs)} runs of dispatches but {len(rows)} rows in {args.bench}: the kernel filter or "
                 f"the sweep does not match")
    # the rows of one unit and weight format share their copies, hence their launches per pass
    unit_of = lambda r: (r.get("proj", r.get("unit")), r.get("format"))
    base = {}
    for (key, v), r in zip(runs, rows):
        base[unit_of(r)] = min(base.get(unit_of(r), len(v)), len(v))
    scale = dict(s.split("=") for s in args.scale)
    per_sq = simds_per_sq(args.dir[0]) if counters else None
    for (key, v), r in zip(runs, rows):
        name, grid, wg = key
        k = max(1, round(len(v) / base[unit_of(r)]))
        v = v[len(v) // args.passes:]
        kname = (name.split("<")[0] + (f" x{k}" if k > 1 else ""))[:26]
        head = f"  {row_label(r)}  {kname:26s} {grid // wg:5d} x {wg:4d}"
        if counters:
            calls = _calls(v, k, lambda g: {c: sum(d[c] for d in g) for c in g[0]})
            med = {c: statistics.median(d[c] for d in calls) for c in sorted(calls[0])}
            if "SQ_WAVES" in med:
                text = sq_text(med, per_sq)
            else:
                text = "  ".join(f"{c} {m:10.1f} KiB" for c, m in med.items())
            if all(c in scale for c in med) and "bytes" in r:
                meas = sum(m * 1024 * float(scale[c]) for c, m in med.items())
                text += f"  -> {meas / 1e6:8.3f} MB  algorithmic {r['bytes'] / 1e6:8.3f} MB  " \
                        f"ratio {meas / r['bytes']:.3f}"
            print(f"{head}  {text}")
        else:
            calls = _calls([ns for ns, _ in v], k, sum)
            print(f"{head}  launches={len(v) * args.passes // (args.passes - 1):6d}  "
                  f"median_us={statistics.median(calls) / 1e3:7.2f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("trace", "pmc"):
        p = sub.add_parser(name)
        p.add_argument("dir")
        p.add_argument("--kernel", default=None)
        p.add_argument("--window", default=None)
    p = sub.add_parser("runs")
    p.add_argument("dir", nargs="+", help="a kernel-trace directory, or counter directories of the same sweep")
    p.add_argument("--bench", required=True, help="the sweep's output (its JSON line with rows)")
    p.add_argument("--kernel", default=None)
    p.add_argument("--passes", type=int, default=7, help="equal passes per run; the first is dropped")
    p.add_argument("--scale", action="append", default=[], help="COUNTER=F: bytes per counted KiB / 1024")
    args = ap.parse_args(argv)
    {"trace": cmd_trace, "pmc": cmd_pmc, "runs": cmd_runs}[args.cmd](args)


if __name__ == "__main__":
    main()
