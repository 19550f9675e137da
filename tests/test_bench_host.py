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
    # the committed summary was taken with the current GEMV sources: the figure applies
    got = bench.measured_traffic(ROOT, "fused")
    assert got is not None and 12.8e6 < got < 13.5e6
    # other compositions have no counter figure
    assert bench.measured_traffic(ROOT, "separate") is None
    # a changed source voids it: copy the tree's summary and sources, edit one source
    src_dir = tmp_path / "ternary_weight_decode_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (tmp_path / bench.TRAFFIC_PROFILE).write_text(open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)).read())
    for f in bench.GEMV_SOURCES:
        (src_dir / f).write_bytes(open(os.path.join(ROOT, "ternary_weight_decode_amd", "csrc", f), "rb").read())
    assert bench.measured_traffic(str(tmp_path), "fused") == got
    (src_dir / bench.GEMV_SOURCES[0]).write_bytes((src_dir / bench.GEMV_SOURCES[0]).read_bytes() + b"\n")
    assert bench.measured_traffic(str(tmp_path), "fused") is None
