"""Host-side parts of bench.py (no GPU): the one-GPU guard and the memory-traffic
figure it reads from the committed counter summary."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_figure_follows_the_kernel_sources(tmp_path):
    """The figure is read from the counter summary only while the GEMV sources hash to the value
    recorded with the counters: a copy of the sources, a summary written for them, then one edit."""
    import hashlib
    src_dir = tmp_path / "ternary_weight_decode_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    blob = b""
    for f in bench.GEMV_SOURCES:
        data = open(os.path.join(ROOT, "ternary_weight_decode_amd", "csrc", f), "rb").read()
        (src_dir / f).write_bytes(data)
        blob += data
    summary = ("ternary GEMV per launch (mean over the four launch kinds of a layer): HBM 13.023 MB, "
               "algorithmic 12.863 MB, ratio 1.012\n"
               f"kernel sources sha256 ({', '.join(bench.GEMV_SOURCES)}) at measurement: "
               f"{hashlib.sha256(blob).hexdigest()}\n")
    (tmp_path / bench.TRAFFIC_PROFILE).write_text(summary)
    assert bench.measured_traffic(str(tmp_path), "fused") == 13023000
    # other compositions have no counter figure
    assert bench.measured_traffic(str(tmp_path), "separate") is None
    assert bench.measured_traffic(str(tmp_path), "fused", 1) is None     # the summary covers the 8B shapes
    # a changed source voids it
    (src_dir / bench.GEMV_SOURCES[0]).write_bytes(blob[:10])
    assert bench.measured_traffic(str(tmp_path), "fused") is None
    # and the committed summary names the same sources in the same form
    text = open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)).read()
    assert f"kernel sources sha256 ({', '.join(bench.GEMV_SOURCES)}) at measurement:" in text


def test_traced_figure_follows_the_kernel_sources(tmp_path):
    """The traced mean duration is read from the trace summary only while the GEMV sources hash
    to the value recorded with the trace, and the committed summary yields it now."""
    import hashlib
    src_dir = tmp_path / "ternary_weight_decode_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    blob = b""
    for f in bench.GEMV_SOURCES:
        data = open(os.path.join(ROOT, "ternary_weight_decode_amd", "csrc", f), "rb").read()
        (src_dir / f).write_bytes(data)
        blob += data
    summary = (f"kernel sources sha256 ({', '.join(bench.GEMV_SOURCES)}): {hashlib.sha256(blob).hexdigest()}\n"
               "roofline of the dominant kernel from the trace: 12,863,488 algorithmic bytes per launch (mean over the four\n"
               "kinds) / 5.130 us (roofline replays) = 2.508 TB/s = 0.313 of 8 TB/s.\n")
    (tmp_path / bench.TRACE_PROFILE).write_text(summary)
    t = bench.measured_trace(str(tmp_path), "fused")
    assert t == {"avg_launch_us": 5.130, "frac": 0.313, "source": bench.TRACE_PROFILE}
    assert bench.measured_trace(str(tmp_path), "separate") is None
    assert bench.measured_trace(str(tmp_path), "fused", 1) is None
    (src_dir / bench.GEMV_SOURCES[0]).write_bytes(blob[:10])
    assert bench.measured_trace(str(tmp_path), "fused") is None
    assert bench.measured_trace(ROOT, "fused") is not None
