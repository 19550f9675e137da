"""GPU parity of the fused head + greedy argmax (i8_head_argmax[_i8]).

int8 activations: the logits come from exact int32 sums and two fp32
products in a stated order, so the oracle reproduces them bit for bit and
the argmax (index and value) must match exactly.  bf16 activations: the
kernel's fp32 sums round differently from the fp64 oracle, so the chosen
row must be a valid maximum (its exact logit within the fp32 error of the
largest) and must equal the oracle's choice wherever the top two are
separated by more than that error."""
import numpy as np
import pytest

import oracle
from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu


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


def head_inputs(v, k, m, seed):
    rng = np.random.default_rng(seed)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    return w, rs, x


@pytest.mark.parametrize("v,k,m", [(300, 512, 1), (5003, 1024, 3), (151936, 4096, 1), (20000, 4096, 16)])
def test_head_argmax_i8_exact(tw, v, k, m):
    import torch
    w, rs, x = head_inputs(v, k, m, seed=v + m)
    q, sx = oracle.quantize_i8(x)
    logits = torch.full((m, v), float("nan"), dtype=torch.float32, device="cuda")
    idx, val = tw.i8_head_argmax_i8(dev(w), dev(rs), dev(q), dev(sx), logits=logits)
    acc, y64, _ = oracle.head_i8(w, rs, q, sx)
    l32 = oracle.head_i8_logits_f32(acc, rs, sx)
    i0, v0 = oracle.greedy_argmax(l32)
    assert np.array_equal(host(idx), i0)
    assert np.array_equal(host(val).view(np.uint32), v0.view(np.uint32))
    assert np.array_equal(host(logits), l32)
    # independent of the stated fp32 product order: the chosen row is a maximum of the
    # fp64 logits up to the two fp32 roundings of each logit, and it is the fp64 argmax
    # wherever the top two are further apart than that
    for r in range(m):
        top = np.sort(y64[r])[::-1]
        tol = 4 * 2.0 ** -24 * np.abs(y64[r]).max()
        assert y64[r, i0[r]] >= top[0] - tol, (r, i0[r])
        if top[0] - top[1] > 2 * tol:
            assert i0[r] == int(np.argmax(y64[r]))


def test_head_argmax_i8_ties_take_the_lowest_row(tw):
    """Duplicates of the winning row placed at lower indices: the lowest wins;
    a head of identical rows returns row 0."""
    v, k, m = 4099, 512, 2
    w, rs, x = head_inputs(v, k, m, seed=9)
    q, sx = oracle.quantize_i8(x)
    acc, _, _ = oracle.head_i8(w, rs, q, sx)
    i0, _ = oracle.greedy_argmax(oracle.head_i8_logits_f32(acc, rs, sx))
    w2, rs2 = w.copy(), rs.copy()
    for m_, dup in zip(range(m), (17, 3001)):
        w2[dup] = w[i0[m_]]
        rs2[dup] = rs[i0[m_]]
    acc2, _, _ = oracle.head_i8(w2, rs2, q, sx)
    i2, v2 = oracle.greedy_argmax(oracle.head_i8_logits_f32(acc2, rs2, sx))
    idx, val = tw.i8_head_argmax_i8(dev(w2), dev(rs2), dev(q), dev(sx))
    assert np.array_equal(host(idx), i2) and np.array_equal(host(val), v2)
    assert all(i2[m_] == min(d, i0[m_]) for m_, d in zip(range(m), (17, 3001)))
    same = np.repeat(w[:1], v, axis=0)
    idx, _ = tw.i8_head_argmax_i8(dev(same), dev(np.full(v, 0.01, np.float32)), dev(q), dev(sx))
    assert host(idx).tolist() == [0, 0]


@pytest.mark.parametrize("v,k,m", [(300, 512, 1), (151936, 4096, 1), (151936, 1024, 4), (20000, 4096, 16)])
def test_head_argmax_bf16_valid(tw, v, k, m):
    import torch
    w, rs, x = head_inputs(v, k, m, seed=3 * v + m)
    logits = torch.empty((m, v), dtype=torch.float32, device="cuda")
    idx, val = tw.i8_head_argmax(dev(w), dev(rs), dev(x), logits=logits)
    idx, val, lg = host(idx), host(val), host(logits)
    y64, _ = oracle.head_bf16(w, rs, x)
    assert oracle.rel_l2(lg, y64) <= 1e-5
    for r in range(m):
        top = np.sort(y64[r])[::-1]
        tol = 1e-5 * np.abs(y64[r]).max()
        assert y64[r, idx[r]] >= top[0] - tol, (r, idx[r])
        assert abs(val[r] - y64[r, idx[r]]) <= tol
        assert val[r] == lg[r].max() and idx[r] == int(np.argmax(lg[r] + np.float32(0)))
        if top[0] - top[1] > 2 * tol:
            assert idx[r] == int(np.argmax(y64[r]))


def test_head_argmax_reuses_its_workspace(tw):
    v, k, m = 7000, 1024, 2
    w, rs, x = head_inputs(v, k, m, seed=5)
    q, sx = oracle.quantize_i8(x)
    ws = tw.i8_head_argmax_workspace(v, m)
    first = [host(t) for t in tw.i8_head_argmax_i8(dev(w), dev(rs), dev(q), dev(sx), workspace=ws)]
    for _ in range(3):
        again = [host(t) for t in tw.i8_head_argmax_i8(dev(w), dev(rs), dev(q), dev(sx), workspace=ws)]
        assert all(np.array_equal(a, b) for a, b in zip(first, again))
    # a smaller call on the same workspace
    idx, _ = tw.i8_head_argmax_i8(dev(w), dev(rs), dev(q[:1]), dev(sx[:1]), workspace=ws)
    assert host(idx)[0] == first[0][0]
