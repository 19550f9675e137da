"""Benchmark of the ternary decode hot path on one MI355X.

One step = one token-equivalent of single-stream decode at the Qwen3-8B
shapes: the 252 ternary linears of 36 layers (q, k, v, o, gate, up, down;
M = 1, bf16 activations, fp32 outputs) followed by the untied int8 output
head 151936 x 4096.  Every linear has its own packed weights and its own
activation vector, all resident in HBM before timing (2.47 GB per step, ten
times the 256 MB last-level cache, so every step streams from HBM).

Prints one JSON line: whole-step throughput in GB/s of algorithmic bytes
(packed weights + scales + activations + outputs), the token-equivalent time,
the roofline of the dominant kernel (the M=1 ternary GEMV) from HIP events
around each of its launches, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--engine graph|chain] [--compose separate|fused] [--no-graph]

Engines: "chain" runs the step's ternary linears as one persistent launch of
tern_gemv_chain, each linear reading an earlier one's output and waiting only
for it, the next weights streaming meanwhile, and then the head; "graph"
replays a hipGraph of one tern_gemv launch per linear (each with its own
input vector) and the head.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
METRIC = "ternary GEMV GB/s and % HBM peak, 8B shapes M=1; us/token-equiv"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2], help="1 = 0.6B shapes, 2 = 8B shapes")
    ap.add_argument("--compose", default="fused", choices=["separate", "fused"],
                    help="separate: one launch per linear (252 + head); fused: q|k|v and gate|up share a launch")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of replaying a hipGraph")
    ap.add_argument("--engine", default="graph", choices=["graph", "chain"],
                    help="chain: one persistent tern_gemv_chain launch per step; graph: one launch per linear")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="token mode: skip the config-0 single linear and the 0.6B token-equivalent")
    ap.add_argument("--prefill-case", default=None, metavar="PROJ:M",
                    help="--mode prefill: run only this shape and M (e.g. gate:2048)")
    ap.add_argument("--mode", default="token",
                    choices=["token", "smallm", "prefill", "head", "fv5", "sweep", "copy", "peak", "floor"],
                    help="token: the headline step; smallm: speculative-verify M sweep on the 8B shapes; "
                         "prefill: int8-MFMA contraction at M in {64, 512, 2048}; "
                         "copy: plain 256 MiB device copies (reference for memory-counter scaling); "
                         "peak: the matrix-core throughput probe (int8 16x16x64 and bf16 16x16x32); "
                         "floor: per-launch cost of near-empty dependent launches and the streaming read rate")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Step:
    """Device-resident inputs of one token-equivalent and the launch list."""

    def __init__(self, tw, synth, config: int, compose: str, quiet: bool = False):
        import torch
        self.torch = torch
        self.tw = tw
        lins = synth.model_linears(config)
        log_ = (lambda msg: None) if quiet else log
        self.launches = []          # (kind, packed/W, n, k, x, y, bytes, label)
        t0 = time.time()

        def gen(lin):
            return synth.linear_inputs(lin)

        # generate on host threads a layer at a time, pack on the GPU
        per_layer = 7
        groups = [lins[i:i + per_layer] for i in range(0, len(lins), per_layer)]
        for gi, group in enumerate(groups):
            data = synth.parallel_map(gen, group)
            by = {lin.proj: (lin, d) for lin, d in zip(group, data)}
            if compose == "fused":
                units = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
            else:
                units = [(p, [p]) for p in synth.PROJ]
            for label, projs in units:
                ts = np.concatenate([by[p][1][0] for p in projs], axis=0)
                ss = np.concatenate([by[p][1][1] for p in projs], axis=0)
                x = by[projs[0]][1][2]
                n, k = ts.shape
                t_dev = torch.from_numpy(ts).cuda()
                s_dev = torch.from_numpy(ss.view(np.int16)).cuda()
                packed = tw.tern_pack(t_dev, s_dev)
                del t_dev, s_dev
                x_dev = torch.from_numpy(x.view(np.int16)).cuda()
                y_dev = torch.empty((1, n), dtype=torch.float32, device="cuda")
                nbytes = tw.tern_packed_bytes(n, k) + 2 * k + 4 * n
                self.launches.append(("tern", packed, n, k, x_dev, y_dev, nbytes, label))
            if gi % 6 == 5:
                log_(f"generated and packed {gi + 1}/{len(groups)} layers ({time.time() - t0:.1f}s)")
        w, rs, xh = synth.head_inputs(config)
        v, k = w.shape
        # the head is stored in its packed layout (row groups of 64, read workgroup-contiguously);
        # the logits are those of the row-major head bit for bit
        w_dev = torch.from_numpy(w).cuda()
        self.head = (tw.i8_head_pack(w_dev), torch.from_numpy(rs).cuda(),
                     torch.from_numpy(xh.view(np.int16)).cuda(), torch.empty((1, v), dtype=torch.float32,
                                                                             device="cuda"))
        del w_dev
        self.head_vk = (v, k)
        self.head_bytes = v * k + 4 * v + 2 * k + 4 * v
        self.tern_bytes = sum(l[6] for l in self.launches)
        self.bytes = self.tern_bytes + self.head_bytes
        torch.cuda.synchronize()
        log_(f"inputs resident: {self.bytes / 1e9:.3f} GB algorithmic per step, "
             f"{len(self.launches)} ternary launches + head ({time.time() - t0:.1f}s)")

    def clone(self):
        """A second copy of every device buffer (same values, distinct memory)."""
        c = object.__new__(Step)
        c.torch, c.tw = self.torch, self.tw
        c.launches = [(kind, p.clone(), n, k, x.clone(), y.clone(), b, lab)
                      for (kind, p, n, k, x, y, b, lab) in self.launches]
        c.head = tuple(t.clone() for t in self.head)
        c.head_vk = self.head_vk
        c.head_bytes, c.tern_bytes, c.bytes = self.head_bytes, self.tern_bytes, self.bytes
        return c

    def run_tern(self, label=None):
        tw = self.tw
        for (_, p, n, k, x, y, _, lab) in self.launches:
            if label is None or lab == label:
                tw.tern_gemv(p, n, k, x, y=y)

    def run_head(self):
        wp, rs, xh, yh = self.head
        self.tw.i8_head_gemv_packed(wp, rs, *self.head_vk, xh, y=yh)

    def run(self):
        self.run_tern()
        self.run_head()

    # ---- persistent-chain engine: the same linears, in order, as one launch.
    # Each linear after the first reads the output of the nearest earlier one
    # with at least K outputs (its first K values, rounded to bf16), the way
    # decode feeds one linear into the next (attention and the gated
    # activation, which sit between them in the model, are not part of this
    # path), so every step truly waits for its input.
    def plan_chain(self):
        tw = self.tw
        specs = []
        for i, (_, p, n, k, x, y, _, _) in enumerate(self.launches):
            src = next((j for j in range(i - 1, -1, -1) if self.launches[j][2] >= k), -1)
            specs.append((p, n, k, x.view(-1) if src < 0 else None, src, y.view(-1)))
        ws = tw.tern_chain_workspace(specs)
        tw.tern_chain_plan(specs, ws)
        return ws, len(specs)

    def run_chain(self, ws, n):
        self.tw.tern_gemv_chain(ws, n)


def capture(torch, fn):
    """Capture fn's launches (on a side stream, as torch requires) into a hipGraph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


class ProfilerRegion:
    """roctx profiler resume / pause around a region: under `rocprofv3 --selected-regions`
    only the launches inside such regions are traced or counted; otherwise these calls do
    nothing.  The roctx library ships with ROCm; without it the region is a no-op."""

    def __init__(self):
        import ctypes
        self.lib = None
        root = os.environ.get("ROCM_PATH", "/opt/rocm")
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                self.lib = ctypes.CDLL(os.path.join(root, "lib", name))
                break
            except OSError:
                continue

    def resume(self):
        if self.lib is not None:
            self.lib.roctxProfilerResume(0)

    def pause(self):
        if self.lib is not None:
            self.lib.roctxProfilerPause(0)


def time_replays(torch, g, reps: int, region: ProfilerRegion | None = None, warm_ms: float = 20.0) -> float:
    """Mean milliseconds per replay from HIP events on the replay stream, after untimed
    replays for at least warm_ms (at least one): a case timed right after its inputs were
    generated ran up to 10% slower with a single warm-up replay (8B gate prefill at
    M = 2048: 178.7 vs 165.6 us for the same kernel timed later).  With a region, exactly
    the timed replays run inside it."""
    t0 = time.perf_counter()
    for i in range(1000):
        g.replay()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= warm_ms:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if region is not None:
        region.resume()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    if region is not None:
        region.pause()
    return e0.elapsed_time(e1) / reps


TRAFFIC_PROFILE = "profiles/tern_gemv_m1_8b_token_fused_hbm_traffic.txt"


GEMV_SOURCES = ("tern_gemv.hip", "tern_oneshot.h", "tern_tile.h", "tern_device.h")   # the M = 1 GEMV's sources


def measured_traffic(root: str, compose: str, config: int = 2):
    """HBM bytes per ternary-GEMV launch from the committed memory-counter
    summary, or None when it does not apply: other shapes (the summary covers
    the 8B shapes), other composition, or the GEMV kernel source changed since
    the counters were taken."""
    import hashlib
    import re
    if compose != "fused" or config != 2:
        return None
    try:
        text = open(os.path.join(root, TRAFFIC_PROFILE)).read()
        src = b"".join(open(os.path.join(root, "ternary_weight_decode_amd", "csrc", f), "rb").read()
                       for f in GEMV_SOURCES)
    except OSError:
        return None
    m = re.search(r"ternary GEMV per launch .*?: HBM ([0-9.]+) MB", text)
    h = re.search(r"sha256 \(" + ", ".join(GEMV_SOURCES) + r"\) at measurement: ([0-9a-f]{64})", text)
    if not m or not h or h.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(float(m.group(1)) * 1e6)


TRACE_PROFILE = "profiles/tern_gemv_m1_8b_token_fused_kernel_trace.txt"


def measured_trace(root: str, compose: str, config: int = 2):
    """The dominant kernel's mean device duration per launch from the committed rocprofv3
    trace summary (the roofline replays' dispatch window), and the roofline fraction it
    gives, or None when it does not apply: other shapes or composition, or the GEMV kernel
    source changed since the trace was taken.  Under the tracer every dispatch is timed on
    its own and runs longer than between graph replays, so this fraction is the lower one."""
    import hashlib
    import re
    if compose != "fused" or config != 2:
        return None
    try:
        text = open(os.path.join(root, TRACE_PROFILE)).read()
        src = b"".join(open(os.path.join(root, "ternary_weight_decode_amd", "csrc", f), "rb").read()
                       for f in GEMV_SOURCES)
    except OSError:
        return None
    m = re.search(r"/ ([0-9.]+) us \(roofline replays\) = [0-9.]+ TB/s = ([0-9.]+) of 8 TB/s", text)
    h = re.search(r"kernel sources sha256 \(" + ", ".join(GEMV_SOURCES) + r"\): ([0-9a-f]{64})", text)
    if not m or not h or h.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return {"avg_launch_us": float(m.group(1)), "frac": float(m.group(2)), "source": TRACE_PROFILE}


def time_calls(torch, fn, reps: int) -> float:
    """Mean milliseconds per call of fn (launches only) from HIP events on the current stream."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def roofline(root, args, achieved, tern_ms, n_tern, step):
    base = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}
    if args.engine == "chain":
        base.update({"traffic": measured_chain_traffic(root, args.compose) if args.config == 2 else None,
                     "kernel": f"chain_kernel (tern_gemv_chain, M=1, {n_tern} dependent steps per launch)",
                     "avg_launch_us": round(tern_ms * 1e3, 3),
                     "avg_bytes_per_launch": int(step.tern_bytes),
                     "launches_per_step": 1,
                     "us_per_linear_step": round(tern_ms / n_tern * 1e3, 3),
                     "timing": "HIP events around back-to-back launches of the step's ternary chain"})
    else:
        base.update({"traffic": measured_traffic(root, args.compose, args.config),
                     "traced": measured_trace(root, args.compose, args.config),
                     "kernel": "gemv_m1_kernel<U> (tern_gemv, M=1)",
                     "avg_launch_us": round(tern_ms / n_tern * 1e3, 3),
                     "avg_bytes_per_launch": int(step.tern_bytes / n_tern),
                     "launches_per_step": n_tern,
                     "timing": "HIP events around hipGraph replays of the step's ternary GEMV launches"})
    return base


CHAIN_TRAFFIC_PROFILE = "profiles/tern_chain_8b_token_fused_hbm_traffic.txt"


def measured_chain_traffic(root: str, compose: str):
    """HBM bytes per chain launch from the committed memory-counter summary, or
    None when the chain kernel source changed since the counters were taken."""
    import hashlib
    import re
    if compose != "fused":
        return None
    try:
        text = open(os.path.join(root, CHAIN_TRAFFIC_PROFILE)).read()
        src = open(os.path.join(root, "ternary_weight_decode_amd", "csrc", "tern_chain.hip"), "rb").read()
    except OSError:
        return None
    m = re.search(r"chain per launch .*?: HBM ([0-9.]+) MB", text)
    h = re.search(r"sha256 \(tern_chain.hip\) at measurement: ([0-9a-f]{64})", text)
    if not m or not h or h.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(float(m.group(1)) * 1e6)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, oracle, target_s: float):
    """The fp64 oracle (a correctness reference, not a tuned CPU kernel) on
    the host cores in this process's affinity mask: its bf16 GEMV over the
    seven linears of one 8B layer (the same generated inputs as the GPU step's
    layer 0, packed by the oracle), repeated until target_s of CPU time is
    spent; per linear the median of 3 timed calls; and the single 3072 x 1024
    linear of the smallest configuration on one core."""
    cores = len(os.sched_getaffinity(0))
    used = oracle.set_threads(cores)
    lins = [l for l in synth.model_linears(2) if l.layer == 0]
    work = []
    for lin in lins:
        t, s, x = synth.linear_inputs(lin)
        work.append((lin.proj, oracle.pack(t, s), lin.n, lin.k, x))
    per_linear = {}
    done_bytes, t_used, reps = 0, 0.0, 0
    times = {proj: [] for (proj, *_rest) in work}
    while t_used < target_s or reps < 3:
        for (proj, p, n, k, x) in work:
            t0 = time.perf_counter()
            oracle.gemv_bf16(p, n, k, x)
            dt = time.perf_counter() - t0
            t_used += dt
            times[proj].append(dt)
            done_bytes += p.size + 2 * k + 4 * n
        reps += 1
    for (proj, p, n, k, x) in work:
        med = float(np.median(times[proj][:3]))
        per_linear[proj] = {"n_k": [n, k], "ms_median3": round(med * 1e3, 2),
                            "GB/s": round((p.size + 2 * k + 4 * n) / med / 1e9, 4)}
    layer_ms = sum(v["ms_median3"] for v in per_linear.values())
    # config 0 on one core
    t0_, s0_, x0_ = synth.config0_inputs()
    p0 = oracle.pack(t0_, s0_)
    oracle.set_threads(1)
    c0 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemv_bf16(p0, 3072, 1024, x0_)
        c0.append(time.perf_counter() - t0)
    oracle.set_threads(used)
    c0_ms = float(np.median(c0)) * 1e3
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"fp64 oracle bf16 GEMV over the 7 linears of one 8B layer, {reps} pass(es), "
                      f"{done_bytes / 1e6:.1f} MB algorithmic in {t_used:.1f} s",
            "seconds": round(t_used, 2),
            "affinity_cores": cores, "cpu_model": cpu_model(),
            "per_linear_median3": per_linear,
            "layer_ms_median3": round(layer_ms, 2),
            "token_equiv_ternary_ms_estimate": round(36 * layer_ms, 1),
            "c0_single_core_ms_median3": round(c0_ms, 2),
            "c0_single_core_GB/s": round(849_920 / (c0_ms * 1e-3) / 1e9, 4),
            "note": "correctness reference (naive bit-by-bit unpack, fp64 accumulation), not a tuned CPU kernel"}


INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s


def shape_inputs(tw, synth, torch, proj, m, seed=7):
    """Packed weights of one 8B-shape linear (layer 0) and m bf16 activation rows."""
    n, k = synth.SHAPES_8B[proj]
    lin = synth.Linear(2, 0, proj, n, k, synth.P_ZERO, synth.P_PLUS)
    t, s, _ = synth.linear_inputs(lin)
    x = synth.gen_x_bf16(np.random.default_rng(seed), m, k)
    packed = tw.tern_pack(torch.from_numpy(t).cuda(), torch.from_numpy(s.view(np.int16)).cuda())
    return n, k, packed, torch.from_numpy(x.view(np.int16)).cuda()


def rotate_copies(torch, packed, total_bytes=1 << 30):
    """Distinct copies of a packed matrix so consecutive launches stream from HBM."""
    reps = max(1, min(256, total_bytes // max(1, packed.numel())))
    return [packed] + [packed.clone() for _ in range(reps - 1)]


def measure_c0(tw, synth, torch, reps: int):
    """The smallest configuration: one 3072 x 1024 ternary linear (seed 0), M = 1, as a
    hipGraph over distinct packed copies totalling >= 1 GB, so every launch reads HBM."""
    t, s, x = synth.config0_inputs()
    n, k = t.shape
    packed = tw.tern_pack(torch.from_numpy(t).cuda(), torch.from_numpy(s.view(np.int16)).cuda())
    copies = [packed] + [packed.clone() for _ in range(max(1, (1 << 30) // packed.numel()))]
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: [tw.tern_gemv(c, n, k, xd, y=y) for c in copies])
    ms = time_replays(torch, g, reps) / len(copies)
    nbytes = tw.tern_packed_bytes(n, k) + 2 * k + 4 * n
    del g, copies
    return {"workload": "config 0: one 3072x1024 ternary linear (0.6B gate shape), M=1, seed 0, bf16",
            "copies_rotated": int((1 << 30) // packed.numel()) + 1, "us_per_launch": round(ms * 1e3, 3),
            "bytes_per_launch": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


def measure_c1(tw, synth, torch, compose: str, reps: int):
    """The 0.6B shapes: 196 ternary linears (fused: 112 launches) and the tied int8 head
    151936 x 1024, M = 1, one token-equivalent per step; two copies of the model (distinct
    memory, 2 x 274 MB, beyond the 256 MB last-level cache) are replayed alternately."""
    steps = [Step(tw, synth, 1, compose, quiet=True)]
    steps.append(steps[0].clone())
    graphs = [capture(torch, st.run) for st in steps]
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for g in graphs:
            g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (2 * reps) * 1e3
    tern_graphs = [capture(torch, st.run_tern) for st in steps]
    e0.record()
    for _ in range(reps):
        for g in tern_graphs:
            g.replay()
    e1.record()
    torch.cuda.synchronize()
    tern_us = e0.elapsed_time(e1) / (2 * reps) * 1e3
    st = steps[0]
    out = {"workload": "qwen3-0.6b-shapes token-equivalent: 196 ternary GEMVs (28 layers x q,k,v,o,gate,up,down) "
                       "+ tied int8 head 151936x1024, M=1, two model copies alternated",
           "compose": compose, "launches_per_step": len(st.launches) + 1, "bytes_per_step": int(st.bytes),
           "us_per_token_equiv": round(us, 2), "GB/s": round(st.bytes / (us * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100 * st.bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
           "ternary_us_per_token_equiv": round(tern_us, 2),
           "ternary_us_per_launch": round(tern_us / len(st.launches), 3)}
    del graphs, tern_graphs, steps
    return out


def measure_floor(tw, torch, reps: int, n_tern: int = 0, tern_bytes: int = 0, tern_us: float = 0.0):
    """What a GEMV launch at M = 1 sits on: the cost per launch of dependent launches in a hipGraph (an
    empty kernel; 256 workgroups x 512 threads storing one float each; the same after one 16-byte load
    per thread from a distinct, cold 2 MiB buffer) and the rate of a plain streaming read of 1 GiB.  With
    the step's launch count and ternary bytes: the floor-plus-read model of the ternary part of a step
    (launches x cold-load floor + bytes at the read rate) beside its measured time."""
    launches = 256
    bufs = [torch.zeros(256 * 512 * 16, dtype=torch.uint8, device="cuda") for _ in range(launches)]
    sink = torch.zeros(1 << 14, dtype=torch.float32, device="cuda")
    out = {}
    for name, kind, grid in (("empty_us", "empty", 1), ("store_256x512_us", "store", 256),
                             ("cold_load_256x512_us", "load", 256)):
        g = capture(torch, lambda: [tw.tern_launch_probe(kind, grid, src=b if kind == "load" else None, sink=sink)
                                    for b in bufs])
        out[name] = round(time_replays(torch, g, reps) / launches * 1e3, 3)
        del g
    del bufs
    big = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    ms = time_calls(torch, lambda: tw.tern_launch_probe("read", 4096, src=big, sink=sink), reps)
    read_gbs = big.numel() / (ms * 1e-3) / 1e9
    out["read_1GiB_GB/s"] = round(read_gbs, 1)
    del big
    if n_tern:
        model = n_tern * out["cold_load_256x512_us"] + tern_bytes / (read_gbs * 1e9) * 1e6
        out["ternary_model_us"] = round(model, 1)
        out["ternary_measured_us"] = round(tern_us, 1)
        out["model_over_measured"] = round(model / tern_us, 3)
    return out


def mode_smallm(args, tw, synth, torch):
    """Speculative-verify sweep: every 8B shape at M in {1,2,4,7,8} (and 16, the largest batch a call
    takes), bf16 and int8 activations; weights rotate over >= 1 GB of copies so each launch reads HBM."""
    out = []
    for proj in synth.PROJ:
        n, k, packed, x16 = shape_inputs(tw, synth, torch, proj, 16)
        copies = rotate_copies(torch, packed)
        for m in (1, 2, 4, 7, 8, 16):
            x = x16[:m].contiguous()
            q, sx = tw.tern_quantize_i8(x)
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            for variant in ("bf16", "int8"):
                def run():
                    for p in copies:
                        if variant == "bf16":
                            tw.tern_gemv(p, n, k, x, y=y)
                        else:
                            tw.tern_gemv_i8(p, n, k, q, sx, y=y)
                g = capture(torch, run)
                ms = time_replays(torch, g, 5) / len(copies)
                act = m * (2 * k if variant == "bf16" else k + 4)
                nbytes = tw.tern_packed_bytes(n, k) + act + 4 * m * n
                out.append({"proj": proj, "n_k": [n, k], "M": m, "act": variant, "us": round(ms * 1e3, 2),
                            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes})
                print(f"smallm {proj} M={m} {variant}: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
                del g
        del copies
    print(json.dumps({"mode": "smallm", "unit": "GB/s of weights+activations+outputs per launch, cold HBM",
                      "rows": out}), flush=True)


def mode_prefill(args, tw, synth, torch):
    """int8-MFMA prefill at M in {64, 512, 2048} on the 8B gate/up/down shapes: TOP/s counting
    2*M*N*K dense operations (the matrix cores execute the zero weights too)."""
    out = []
    cases = [(p, m) for p in ("gate", "up", "down") for m in (64, 512, 2048)]
    if args.prefill_case:
        proj, m = args.prefill_case.split(":")
        cases = [(proj, int(m))]
    for proj in dict.fromkeys(p for p, _ in cases):
        n, k, packed, _ = shape_inputs(tw, synth, torch, proj, 1)
        copies = rotate_copies(torch, packed)   # >= 1 GB of copies: well beyond the 256 MB last-level cache
        n_copies = len(copies)
        for m in [m for p, m in cases if p == proj]:
            x = torch.from_numpy(synth.gen_x_bf16(np.random.default_rng(m), m, k).view(np.int16)).cuda()
            q, sx = tw.tern_quantize_i8(x)
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            g = capture(torch, lambda: [tw.tern_gemm_prefill(c, n, k, q, sx, y=y) for c in copies])
            ms = time_replays(torch, g, 5) / len(copies)
            ops = 2.0 * m * n * k
            tops = ops / (ms * 1e-3) / 1e12
            nbytes = tw.tern_packed_bytes(n, k) + m * (k + 4) + 4 * m * n
            out.append({"proj": proj, "n_k": [n, k], "M": m, "us": round(ms * 1e3, 2), "TOP/s": round(tops, 1),
                        "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 1),
                        "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
            del g
        del copies
    print(json.dumps({"mode": "prefill", "peak_tops": INT8_PEAK_TOPS,
                      "weights": f"{n_copies} distinct packed copies per shape (>= 1 GB), replayed in turn",
                      "rows": out}), flush=True)


def mode_peak(args, tw, synth, torch):
    """What the matrix cores sustain: the probe's independent MFMA chains on registers (no
    memory traffic), 2048 workgroups of 4 waves, timed with HIP events over repeated launches;
    the median of 5 timings against the published dense peaks."""
    out = []
    grid = 2048
    sink = torch.empty(tw.lib().tern_mfma_peak_sink_bytes(grid) // 4, dtype=torch.int32, device="cuda")
    for kind, iters, peak in (("int8", 20000, INT8_PEAK_TOPS), ("bf16", 20000, 2500.0)):
        ops = tw.tern_mfma_peak(kind, iters, grid, sink)        # warm-up launch
        torch.cuda.synchronize()
        rates = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                tw.tern_mfma_peak(kind, iters, grid, sink)
            e1.record()
            torch.cuda.synchronize()
            rates.append(4 * ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        med = float(np.median(rates))
        out.append({"mfma": "v_mfma_i32_16x16x64_i8" if kind == "int8" else "v_mfma_f32_16x16x32_bf16",
                    "T_ops_per_s_median": round(med, 1), "T_ops_per_s_runs": [round(r, 1) for r in rates],
                    "published_dense_peak": peak, "pct_of_published": round(100 * med / peak, 1),
                    "grid": grid, "iters": iters})
        log(f"peak {kind}: {med:.0f} T/s ({100 * med / peak:.1f}% of {peak:.0f})")
    print(json.dumps({"mode": "peak", "rows": out}), flush=True)


def mode_head(args, tw, synth, torch):
    """The int8 head (151936 x 4096 at --config 2, x 1024 at --config 1) alone and fused with
    the greedy argmax, bf16 and int8 activations, M = 1, with a per-row scale and with a scale per
    256-weight block (FV5B-style); then the embedding-row gather of 1 and 512 tokens: us per call
    and GB/s of the bytes each call must move."""
    w, rs, xh = synth.head_inputs(args.config)
    v, k = w.shape
    W, RS = torch.from_numpy(w).cuda(), torch.from_numpy(rs).cuda()
    copies = [W] + [W.clone() for _ in range(2)]          # 3 x 622 MB: every call streams from HBM
    x = torch.from_numpy(xh.view(np.int16)).cuda()
    q, sx = tw.tern_quantize_i8(x)
    y = torch.empty((1, v), dtype=torch.float32, device="cuda")
    ws = tw.i8_head_argmax_workspace(v, 1)
    # block-scaled (FV5B-style) scales of the same rows: one fp32 per 256 weights
    S = torch.from_numpy(np.random.default_rng(11).uniform(0.002, 0.02, (v, k // 256)).astype(np.float32)).cuda()
    row_bytes, blk_bytes = v * k + 4 * v, v * k + 4 * v * (k // 256)
    packed = [tw.i8_head_pack(c) for c in copies]
    pk = {id(c): p for c, p in zip(copies, packed)}
    runs = {
        "head_bf16": (lambda c: tw.i8_head_gemv(c, RS, x, y=y), row_bytes),
        "head_int8": (lambda c: tw.i8_head_gemv_i8(c, RS, q, sx, y=y), row_bytes),
        "head_bf16_packed": (lambda c: tw.i8_head_gemv_packed(pk[id(c)], RS, v, k, x, y=y), row_bytes),
        "head_int8_packed": (lambda c: tw.i8_head_gemv_packed_i8(pk[id(c)], RS, v, k, q, sx, y=y), row_bytes),
        "head_argmax_bf16": (lambda c: tw.i8_head_argmax(c, RS, x, workspace=ws), row_bytes),
        "head_argmax_bf16_with_logits": (lambda c: tw.i8_head_argmax(c, RS, x, workspace=ws, logits=y), row_bytes),
        "head_argmax_int8": (lambda c: tw.i8_head_argmax_i8(c, RS, q, sx, workspace=ws), row_bytes),
        "head_argmax_bf16_packed": (lambda c: tw.i8_head_argmax_packed(pk[id(c)], RS, v, k, x, workspace=ws),
                                    row_bytes),
        "head_argmax_int8_packed": (lambda c: tw.i8_head_argmax_packed_i8(pk[id(c)], RS, v, k, q, sx, workspace=ws),
                                    row_bytes),
        "fv5b_head_bf16": (lambda c: tw.fv5b_head_gemv(c, S, x, y=y), blk_bytes),
        "fv5b_head_int8": (lambda c: tw.fv5b_head_gemv_i8(c, S, q, sx, y=y), blk_bytes),
        "fv5b_head_argmax_bf16": (lambda c: tw.fv5b_head_argmax(c, S, x, workspace=ws), blk_bytes),
        "fv5b_head_argmax_int8": (lambda c: tw.fv5b_head_argmax_i8(c, S, q, sx, workspace=ws), blk_bytes),
        "fv5b_head_bf16_packed": (lambda c: tw.fv5b_head_gemv_packed(pk[id(c)], S, v, k, x, y=y), blk_bytes),
        "fv5b_head_argmax_bf16_packed": (lambda c: tw.fv5b_head_argmax_packed(pk[id(c)], S, v, k, x, workspace=ws),
                                         blk_bytes),
    }
    out = []
    for name, (fn, nbytes) in runs.items():
        g = capture(torch, lambda: [fn(c) for c in copies])
        ms = time_replays(torch, g, 5) / len(copies)
        out.append({"call": name, "V": v, "K": k, "us": round(ms * 1e3, 2),
                    "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del g
    # the argmax fused with the next token's embedding row (a 151936 x hidden table), against the two calls
    E = torch.from_numpy(np.random.default_rng(12).integers(-127, 128, (v, k), dtype=np.int8)).cuda()
    ES = torch.from_numpy(np.random.default_rng(13).uniform(0.002, 0.02, (v, k // 256)).astype(np.float32)).cuda()
    eb = torch.empty((1, k), dtype=torch.bfloat16, device="cuda")
    idx1 = torch.empty(1, dtype=torch.int32, device="cuda")
    pair = {
        "fv5b_head_argmax_then_embed": lambda c: (idx1.copy_(tw.fv5b_head_argmax(c, S, x, workspace=ws)[0]),
                                                  tw.fv5b_embed(E, ES, idx1, f32=False, out_bf16=eb)),
        "fv5b_head_argmax_embed": lambda c: tw.fv5b_head_argmax_embed(c, S, x, E, ES, workspace=ws, f32=False,
                                                                      out_bf16=eb),
    }
    for name, fn in pair.items():
        g = capture(torch, lambda: [fn(c) for c in copies])
        ms = time_replays(torch, g, 5) / len(copies)
        out.append({"call": name, "V": v, "K": k, "us": round(ms * 1e3, 2),
                    "GB/s": round(blk_bytes / (ms * 1e-3) / 1e9, 1)})
        del g
    # embedding rows (the step before the first linear): 1 token, and a 512-token prefill batch
    for m in (1, 512):
        ids = torch.from_numpy(np.random.default_rng(m).integers(0, v, m).astype(np.int32)).cuda()
        outs = (torch.empty((m, k), dtype=torch.float32, device="cuda"),
                torch.empty((m, k), dtype=torch.bfloat16, device="cuda"))
        g = capture(torch, lambda: [tw.fv5b_embed(c, S, ids, out=outs[0], out_bf16=outs[1]) for c in copies])
        ms = time_replays(torch, g, 5) / len(copies)
        nbytes = m * (k + 4 * (k // 256) + 4 + 6 * k)
        out.append({"call": f"fv5b_embed_m{m}", "V": v, "K": k, "us": round(ms * 1e3, 2),
                    "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del g
    print(json.dumps({"mode": "head", "rows": out}), flush=True)


def mode_sweep(args, tw, synth, torch):
    """The M = 1 ternary GEMV (bf16 activations) at K = 4096 over N from 1024 to 196608 rows: how the
    per-launch latency gives way to streaming as the matrix grows.  Weights rotate over >= 1 GB of
    copies so each launch reads HBM; us per launch from hipGraph replays."""
    out = []
    k = 4096
    rng = np.random.default_rng(17)
    x = torch.from_numpy(synth.gen_x_bf16(rng, 1, k).view(np.int16)).cuda()
    for n in (1024, 4096, 12288, 24576, 49152, 98304, 196608):
        t = torch.from_numpy(synth.gen_ternary(rng, n, k)).cuda()
        sc = torch.from_numpy(synth.gen_scales(rng, n, k // 128).view(np.int16)).cuda()
        packed = tw.tern_pack(t, sc)
        del t, sc
        copies = rotate_copies(torch, packed)
        y = torch.empty((1, n), dtype=torch.float32, device="cuda")
        g = capture(torch, lambda: [tw.tern_gemv(c, n, k, x, y=y) for c in copies])
        ms = time_replays(torch, g, 5) / len(copies)
        nbytes = tw.tern_packed_bytes(n, k) + 2 * k + 4 * n
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append({"n_k": [n, k], "MB": round(nbytes / 1e6, 2), "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                    "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)})
        log(f"sweep N={n}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")
        del g, copies, packed
    print(json.dumps({"mode": "sweep", "rows": out}), flush=True)


FV5_UNITS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",)))


def mode_fv5(args, tw, synth, torch):
    """Five-level (FV5-style, 3.25 bits per weight) GEMV on the fused 8B linears of one layer
    at M in {1, 4, 8, 16}, bf16 and int8 activations, with the ternary GEMV of the same shapes
    beside it; weights rotate
    over >= 1 GB of copies so each launch reads HBM.  Also the bytes-weighted M = 1 layer
    aggregate (one layer = the four fused launches)."""
    out = []
    layer = {f"{f}_{a}": [0.0, 0] for f in ("fv5", "ternary") for a in ("bf16", "int8")}
    for label, projs in FV5_UNITS:
        lins = [synth.Linear(2, 0, p, *synth.SHAPES_8B[p], synth.P_ZERO, synth.P_PLUS) for p in projs]
        parts = [synth.linear5_inputs(lin) for lin in lins]
        lv = np.concatenate([d[0] for d in parts], axis=0)
        lo = np.concatenate([d[1] for d in parts], axis=0)
        hi = np.concatenate([d[2] for d in parts], axis=0)
        n, k = lv.shape
        p5 = tw.tern5_pack(torch.from_numpy(lv).cuda(), torch.from_numpy(lo).cuda(), torch.from_numpy(hi).cuda())
        t = np.clip(lv, -1, 1)
        s16 = np.repeat(lo, 2, axis=1).astype(np.float16).view(np.int16)
        p3 = tw.tern_pack(torch.from_numpy(t).cuda(), torch.from_numpy(s16).cuda())
        del lv, lo, hi, parts, t
        x16 = torch.from_numpy(synth.gen_x_bf16(np.random.default_rng(5), 16, k).view(np.int16)).cuda()
        q16, sx16 = tw.tern_quantize_i8(x16)
        for fmt, packed, nbytes_w, call, call_i8 in (
                ("fv5", p5, tw.tern5_packed_bytes(n, k), tw.tern5_gemv, tw.tern5_gemv_i8),
                ("ternary", p3, tw.tern_packed_bytes(n, k), tw.tern_gemv, tw.tern_gemv_i8)):
            copies = rotate_copies(torch, packed)
            for m in (1, 4, 8, 16):
                x = x16[:m].contiguous()
                q, sx = q16[:m].contiguous(), sx16[:m].contiguous()
                y = torch.empty((m, n), dtype=torch.float32, device="cuda")
                for act in ("bf16", "int8"):
                    if act == "bf16":
                        g = capture(torch, lambda: [call(c, n, k, x, y=y) for c in copies])
                    else:
                        g = capture(torch, lambda: [call_i8(c, n, k, q, sx, y=y) for c in copies])
                    ms = time_replays(torch, g, 5) / len(copies)
                    nbytes = nbytes_w + m * (2 * k if act == "bf16" else k + 4) + 4 * m * n
                    gbs = nbytes / (ms * 1e-3) / 1e9
                    out.append({"unit": label, "format": fmt, "act": act, "n_k": [n, k], "M": m,
                                "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "bytes": nbytes})
                    print(f"fv5 {label} {fmt} M={m} {act}: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
                    if m == 1:
                        layer[f"{fmt}_{act}"][0] += ms * 1e3
                        layer[f"{fmt}_{act}"][1] += nbytes
                    del g
            del copies
        del p5, p3
    agg = {fmt: {"us_per_layer": round(us, 2), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                 "pct_hbm_peak": round(100 * b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
           for fmt, (us, b) in layer.items()}
    print(json.dumps({"mode": "fv5", "rows": out, "layer_m1": agg}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on a single "
              f"MI355X; across GPUs it would shard every linear by output rows, each GPU holding and computing "
              f"its rows, with an all-gather of y where the next linear needs the whole vector)", file=sys.stderr)
        sys.exit(2)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import torch
    import ternary_weight_decode_amd as tw
    from ternary_weight_decode_amd import synth
    assert torch.cuda.is_available(), "no GPU"
    tw.lib()
    if args.mode == "smallm":
        return mode_smallm(args, tw, synth, torch)
    if args.mode == "prefill":
        return mode_prefill(args, tw, synth, torch)
    if args.mode == "head":
        return mode_head(args, tw, synth, torch)
    if args.mode == "fv5":
        return mode_fv5(args, tw, synth, torch)
    if args.mode == "sweep":
        return mode_sweep(args, tw, synth, torch)
    if args.mode == "peak":
        return mode_peak(args, tw, synth, torch)
    if args.mode == "floor":
        print(json.dumps({"mode": "floor", **measure_floor(tw, torch, 10)}), flush=True)
        return
    if args.mode == "copy":
        src = torch.ones(1 << 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_copy": src.numel(), "bytes_written_per_copy": dst.numel(),
                          "copies": 4}), flush=True)
        return

    step = Step(tw, synth, args.config, args.compose)
    chain = args.engine == "chain"
    if chain:
        ws, n_chain = step.plan_chain()

    # ---- timed region: exactly K whole steps
    graph = None
    if not chain and not args.no_graph:
        graph = capture(torch, step.run)

    def one():
        if chain:
            step.run_chain(ws, n_chain)
            step.run_head()
        elif graph is not None:
            graph.replay()
        else:
            step.run()

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    if graph is not None:
        # every launch of the step ran once eagerly before capture, then W warmup replays
        nt = len(step.launches)
        log(f"dispatch window of the timed region: ternary GEMV launches [{nt * (1 + args.warmup)}, "
            f"{nt * (1 + args.warmup + args.steps)}) of this process ({nt} per step)")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = step.bytes * args.steps / wall / 1e9
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {value:.1f} GB/s")
    if chain:
        errs = tw.tern_chain_errors(ws)
        assert errs == 0, f"chain workspace recorded {errs} aborted waits"

    # ---- dominant kernel: HIP events on the stream it runs on.  Graph engine:
    # graph replays of only the ternary GEMV launches (the per-launch time
    # includes the in-graph gap, an upper bound on the kernel's duration).
    # Chain engine: back-to-back launches of the whole chain.
    reps = max(5, min(args.steps, 20))
    n_tern = len(step.launches)
    if chain:
        tern_ms = time_calls(torch, lambda: step.run_chain(ws, n_chain), reps)
    else:
        # the only profiler region of the run: rocprofv3 --selected-regions traces exactly these
        # reps x n_tern launches, the ones the roofline's average is taken over
        g_tern = capture(torch, step.run_tern)
        # one warm replay (the step's W warmup replays ran just before): the dispatch
        # windows the committed trace summaries average over stay fixed
        tern_ms = time_replays(torch, g_tern, reps, ProfilerRegion(), warm_ms=0.0)
    achieved = step.tern_bytes / (tern_ms * 1e-3) / 1e9
    g_head = capture(torch, step.run_head)
    head_ms = time_replays(torch, g_head, reps, warm_ms=0.0)
    # per launch kind (graph engine only: inside the chain the kinds overlap)
    shapes = None
    if not chain:
        shapes = {}
        for label in dict.fromkeys(l[7] for l in step.launches):
            ls = [l for l in step.launches if l[7] == label]
            gl = capture(torch, lambda lab=label: step.run_tern(lab))
            ms = time_replays(torch, gl, reps, warm_ms=0.0) / len(ls)
            del gl
            b = ls[0][6]
            shapes[label] = {"n_k": [ls[0][2], ls[0][3]], "launches": len(ls), "us": round(ms * 1e3, 2),
                             "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                             "pct_peak": round(100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    layer_us = tern_ms / (n_tern / (4 if args.compose == "fused" else 7)) * 1e3
    roof = roofline(root, args, achieved, tern_ms, n_tern, step)
    bytes_step, tern_bytes, head_bytes = step.bytes, step.tern_bytes, step.head_bytes

    used_graph = graph is not None
    extra = {}
    if args.config == 2 and not chain and not args.no_extra_configs:
        del g_tern, g_head, graph, step
        torch.cuda.empty_cache()
        log("config 0 (one 3072x1024 linear, weights rotated over >= 1 GB) ...")
        extra["config0"] = measure_c0(tw, synth, torch, reps)
        log("config 1 (0.6B token-equivalent, two model copies alternated) ...")
        extra["config1"] = measure_c1(tw, synth, torch, args.compose, reps)
        log("launch floor and read ceiling ...")
        extra["launch_floor"] = measure_floor(tw, torch, reps, n_tern, tern_bytes, tern_ms * 1e3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(synth, oracle, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("qwen3-8b-shapes token-equivalent: 252 ternary GEMVs (36 layers x q,k,v,o,gate,up,"
                                "down) + int8 head 151936x4096, M=1" if args.config == 2 else
                                "qwen3-0.6b-shapes token-equivalent: 196 ternary GEMVs + tied int8 head "
                                "151936x1024, M=1"),
                   "engine": args.engine, "compose": args.compose, "graph": used_graph,
                   "bytes_per_step": int(bytes_step)},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "us_per_token_equiv": round(ms_per_step * 1e3, 2),
        "ternary_us_per_token_equiv": round(tern_ms * 1e3, 2),
        "us_per_layer": round(layer_us, 2),
        "head": {"us": round(head_ms * 1e3, 2),
                 "GB/s": round(head_bytes / (head_ms * 1e-3) / 1e9, 1)},
        "per_shape": shapes,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
