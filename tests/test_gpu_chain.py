"""GPU parity of the dependent-GEMV chain (tern_gemv_chain): every step's fp32
output against the fp64 oracle (relative L2 <= 1e-5), its bf16 copy bit for
bit against nearest-even rounding of that output, and chains whose steps read
earlier steps' outputs, so a step that ran before its input was complete would
read stale or zero activations and fail."""
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
    def __init__(self, tw, n, k, seed, x=None):
        import torch
        rng = np.random.default_rng(seed)
        self.n, self.k = n, k
        self.t = synth.gen_ternary(rng, n, k, synth.P_ZERO, synth.P_PLUS)
        self.s = synth.gen_scales(rng, n, k // 128)
        self.x_host = synth.gen_x_bf16(rng, 1, k)[0]
        self.packed_host = oracle.pack(self.t, self.s)
        self.packed = dev(self.packed_host)
        self.x = dev(self.x_host) if x is None else x
        self.y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        self.yb = torch.full((n,), 0x7F7F, dtype=torch.int16, device="cuda")

    def spec(self):
        return (self.packed, self.n, self.k, self.x, self.y, self.yb)


def check_step(st, x_bits, rows=None):
    y = host(st.y)
    yb = host(st.yb).view(np.uint16)
    assert np.array_equal(yb, rne_bf16(y)), "y_bf16 is not y rounded to nearest-even"
    y64, _ = oracle.gemv_bf16(st.packed_host, st.n, st.k, x_bits[None, :], rows=rows)
    got = y if rows is None else y[np.asarray(rows)]
    err = oracle.rel_l2(got, y64[0])
    assert err <= TOL, err


def run_chain(tw, steps, nrun=None, ws=None):
    if ws is None:
        ws = tw.tern_chain_workspace(len(steps))
    tw.tern_chain_plan([s.spec() for s in steps], ws)
    tw.tern_gemv_chain(ws, len(steps) if nrun is None else nrun)
    return ws


def test_chain_independent_steps(tw):
    shapes = [(4096, 4096), (100, 512), (16, 1024), (1000, 2048), (12288, 4096), (4096, 12288), (37, 16384),
              (6144, 4096), (3072, 1024)]
    steps = [Step(tw, n, k, seed=11 * i + 1) for i, (n, k) in enumerate(shapes)]
    ws = run_chain(tw, steps)
    for st in steps:
        check_step(st, st.x_host)
    assert tw.tern_chain_errors(ws) == 0


def test_chain_dependent_steps_read_earlier_outputs(tw):
    # K of each step is N of the previous: x_{p+1} = y_bf16_p
    dims = [4096, 12288, 4096, 1024, 3072, 1024, 512]
    steps = [Step(tw, dims[1], dims[0], seed=101)]
    for p in range(1, len(dims) - 1):
        steps.append(Step(tw, dims[p + 1], dims[p], seed=101 + p, x=steps[-1].yb))
    ws = run_chain(tw, steps)
    check_step(steps[0], steps[0].x_host)
    for p in range(1, len(steps)):
        x_bits = host(steps[p - 1].yb).view(np.uint16)
        assert np.any(x_bits != 0)
        check_step(steps[p], x_bits)
    assert tw.tern_chain_errors(ws) == 0


def test_chain_reruns_are_identical(tw):
    import torch
    dims = [1024, 4096, 2048, 4096]
    steps = [Step(tw, dims[1], dims[0], seed=201)]
    for p in range(1, len(dims) - 1):
        steps.append(Step(tw, dims[p + 1], dims[p], seed=201 + p, x=steps[-1].yb))
    ws = tw.tern_chain_workspace(len(steps))
    tw.tern_chain_plan([s.spec() for s in steps], ws)
    first = None
    for rep in range(4):
        for s in steps:          # stale outputs from a previous run must not survive
            s.y.fill_(float("nan"))
            s.yb.fill_(0x7F7F)
        tw.tern_gemv_chain(ws, len(steps))
        outs = [host(s.y).copy() for s in steps]
        if first is None:
            first = outs
        for a, b in zip(first, outs):
            assert np.array_equal(a, b), rep
    assert tw.tern_chain_errors(ws) == 0
    torch.cuda.synchronize()


def test_chain_runs_a_prefix_and_replans(tw):
    import torch
    steps = [Step(tw, n, k, seed=301 + i) for i, (n, k) in enumerate([(512, 1024), (1024, 512), (64, 2048)])]
    ws = tw.tern_chain_workspace(8)
    tw.tern_chain_plan([s.spec() for s in steps], ws)
    tw.tern_gemv_chain(ws, 2)
    check_step(steps[0], steps[0].x_host)
    check_step(steps[1], steps[1].x_host)
    assert bool(torch.isnan(steps[2].y).all().item())
    # asking for more steps than were planned runs the plan only
    tw.tern_gemv_chain(ws, 8)
    check_step(steps[2], steps[2].x_host)
    # re-plan the same workspace with a different chain
    more = [Step(tw, n, k, seed=401 + i) for i, (n, k) in enumerate([(4096, 4096), (16, 512)])]
    tw.tern_chain_plan([s.spec() for s in more], ws)
    tw.tern_gemv_chain(ws, 2)
    for s in more:
        check_step(s, s.x_host)
    assert tw.tern_chain_errors(ws) == 0


def test_chain_8b_layer_full_shapes(tw):
    """One 8B layer as the decode runs it (q|k|v, o, gate|up, down), sampled rows."""
    shapes = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
    steps = [Step(tw, n, k, seed=501 + i) for i, (n, k) in enumerate(shapes)]
    ws = run_chain(tw, steps)
    rng = np.random.default_rng(7)
    for st in steps:
        rows = np.unique(np.concatenate([rng.integers(0, st.n, 200), [0, st.n - 1]]))
        check_step(st, st.x_host, rows=rows)
        assert not np.any(np.isnan(host(st.y)))
    assert tw.tern_chain_errors(ws) == 0
