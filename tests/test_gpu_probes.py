"""The measurement probes on the device: the launch-floor kernels store what
they are documented to store, the streaming read leaves the sink alone on a
zero-filled buffer, and each kind runs inside a hipGraph replayed several
times."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tw():
    import torch
    import ternary_weight_decode_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def test_launch_probe_kinds(tw):
    import torch
    grid = 300
    src = torch.zeros(grid * 512 * 16, dtype=torch.uint8, device="cuda")
    want = torch.arange(grid, dtype=torch.float32, device="cuda")
    tw.tern_launch_probe("empty", 1)
    for kind in ("store", "load"):
        sink = torch.full((grid + 5,), -7.0, device="cuda")
        tw.tern_launch_probe(kind, grid, src=src if kind == "load" else None, sink=sink)
        torch.cuda.synchronize()
        assert torch.equal(sink[:grid], want) and torch.all(sink[grid:] == -7.0), kind
    sink = torch.full((64,), -7.0, device="cuda")
    tw.tern_launch_probe("read", 64, src=src, sink=sink)
    torch.cuda.synchronize()
    assert torch.all(sink == -7.0)


def test_launch_probe_in_graph(tw):
    import torch
    from bench import capture
    src = torch.zeros(256 * 512 * 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, device="cuda")
    g = capture(torch, lambda: [tw.tern_launch_probe(k, 256, src=src, sink=sink) for k in ("empty", "store", "load")])
    for _ in range(3):
        sink.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sink, torch.arange(256, dtype=torch.float32, device="cuda"))
