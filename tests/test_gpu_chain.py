"""GPU parity of the GEMV chain (tern_gemv_chain): every step's fp32 output
against the fp64 oracle (relative L2 <= 1e-5) on the activations it read;
for a step that reads an earlier step's output, those are that output's
first K values rounded to bf16 (nearest-even, written out below), so a step
that ran before its input was complete, or read a stale hand-off from an
earlier run, would fail."""
import numpy as np
import pytest

import oracle
from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def tw():
    import torch
    import ternary_weight_decode_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rne_bf16(y32):
    """Nearest-even bf16 bits of finite fp32 values (written out for the check)."""
    u = np.ascontiguousarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


class Step:
    def __init__(self, tw, n, k, seed, x_from=-1):
        import torch
        rng = np.random.default_rng(seed)
        self.n, self.k, self.x_from = n, k, x_from
        self.t = synth.gen_ternary(rng, n, k, synth.P_ZERO, synth.P_PLUS)
        self.s = synth.gen_scales(rng, n, k // 128)
        self.x_host = synth.gen_x_bf16(rng, 1, k)[0]
        self.packed_host = oracle.pack(self.t, self.s)
        self.packed = dev(self.packed_host)
        self.x = dev(self.x_host) if x_from < 0 else None
        self.y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")

    def spec(self):
        return (self.packed, self.n, self.k, self.x, self.x_from, self.y)


def x_of(steps, p):
    """The activations step p read: its input vector, or its producer's first K outputs rounded to bf16."""
    st = steps[p]
    if st.x_from < 0:
        return st.x_host
    y = host(steps[st.x_from].y)
    assert not np.any(np.isnan(y[:st.k]))
    return rne_bf16(y[:st.k])


def check_step(steps, p, rows=None):
    st = steps[p]
    x_bits = x_of(steps, p)
    y = host(st.y)
    assert not np.any(np.isnan(y))
    y64, _ = oracle.gemv_bf16(st.packed_host, st.n, st.k, x_bits[None, :], rows=rows)
    got = y if rows is None else y[np.asarray(rows)]
    err = oracle.rel_l2(got, y64[0])
    assert err <= TOL, (p, err)


def run_chain(tw, steps, nrun=None, ws=None):
    specs = [s.spec() for s in steps]
    if ws is None:
        ws = tw.tern_chain_workspace(specs)
    tw.tern_chain_plan(specs, ws)
    tw.tern_gemv_chain(ws, len(steps) if nrun is None else nrun)
    return ws


def test_chain_independent_steps(tw):
    shapes = [(4096, 4096), (100, 512), (16, 1024), (1000, 2048), (12288, 4096), (4096, 12288), (37, 16384),
              (6144, 4096), (3072, 1024)]
    steps = [Step(tw, n, k, seed=11 * i + 1) for i, (n, k) in enumerate(shapes)]
    ws = run_chain(tw, steps)
    for p in range(len(steps)):
        check_step(steps, p)
    assert tw.tern_chain_errors(ws) == 0


def linked_steps(tw, seed):
    """Steps reading earlier outputs: whole vectors, prefixes, and a step two back."""
    spec = [(12288, 4096, -1), (4096, 12288, 0), (6144, 4096, 1), (4096, 4096, 2), (24576, 4096, 3),
            (4096, 12288, 4), (1000, 4096, 5), (512, 2048, 0), (3000, 512, 6)]
    return [Step(tw, n, k, seed=seed + i, x_from=q) for i, (n, k, q) in enumerate(spec)]


def test_chain_steps_read_earlier_outputs(tw):
    steps = linked_steps(tw, 101)
    ws = run_chain(tw, steps)
    for p in range(len(steps)):
        check_step(steps, p)
    assert tw.tern_chain_errors(ws) == 0


def test_chain_reruns_are_identical(tw):
    steps = linked_steps(tw, 201)
    specs = [s.spec() for s in steps]
    ws = tw.tern_chain_workspace(specs)
    tw.tern_chain_plan(specs, ws)
    first = None
    for rep in range(4):
        for s in steps:          # outputs of an earlier run must not leak into this one
            s.y.fill_(float("nan"))
        tw.tern_gemv_chain(ws, len(steps))
        outs = [host(s.y).copy() for s in steps]
        if first is None:
            first = outs
            for p in range(len(steps)):
                check_step(steps, p)
        for a, b in zip(first, outs):
            assert np.array_equal(a, b), rep
    assert tw.tern_chain_errors(ws) == 0


def test_chain_runs_a_prefix_and_replans(tw):
    import torch
    steps = [Step(tw, 512, 1024, seed=301), Step(tw, 1024, 512, seed=302, x_from=0),
             Step(tw, 64, 1024, seed=303, x_from=1)]
    specs = [s.spec() for s in steps]
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    tw.tern_chain_plan(specs, ws)
    tw.tern_gemv_chain(ws, 2)
    check_step(steps, 0)
    check_step(steps, 1)
    assert bool(torch.isnan(steps[2].y).all().item())
    # asking for more steps than were planned runs the plan only
    tw.tern_gemv_chain(ws, 8)
    check_step(steps, 2)
    # re-plan the same workspace with a different chain
    more = [Step(tw, 4096, 4096, seed=401), Step(tw, 16, 4096, seed=402, x_from=0),
            Step(tw, 2048, 512, seed=403)]
    tw.tern_chain_plan([s.spec() for s in more], ws)
    tw.tern_gemv_chain(ws, 3)
    for p in range(len(more)):
        check_step(more, p)
    assert tw.tern_chain_errors(ws) == 0


def test_chain_8b_layer_as_decoded(tw):
    """One 8B layer, each linear reading the previous one's output (a prefix
    where the real model would apply attention or the gated activation), at
    full shapes, sampled rows; then a second layer."""
    shapes = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)] * 2
    steps = [Step(tw, n, k, seed=501 + i, x_from=i - 1) for i, (n, k) in enumerate(shapes)]
    ws = run_chain(tw, steps)
    rng = np.random.default_rng(7)
    for p, st in enumerate(steps):
        rows = np.unique(np.concatenate([rng.integers(0, st.n, 200), [0, st.n - 1]]))
        check_step(steps, p, rows=rows)
    assert tw.tern_chain_errors(ws) == 0
