"""GPU parity of the packed int8 output head: the packed copy against the
oracle's byte for byte, and the GEMV over it against the fp64 oracle
(relative L2 1e-5; int32 sums exact) and against the row-major single-pass
head kernel bit for bit (every lane multiplies the same weights in the same
order)."""
import numpy as np
import pytest

import oracle
from oracle import head_pack
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


# V: one row, a whole group, ragged groups, the 8B head; K: one unit up to 8192
SHAPES = [(1, 128), (64, 256), (70, 256), (300, 512), (2374, 1024), (1000, 4096), (77, 8192)]


@pytest.mark.parametrize("v,k", SHAPES)
def test_pack_bit_exact(tw, v, k):
    rng = np.random.default_rng(v + 3 * k)
    w, _ = synth.gen_head(rng, rng, v, k)
    p = host(tw.i8_head_pack(dev(w)))
    assert np.array_equal(p, head_pack.pack(w))


@pytest.mark.parametrize("v,k,m", [(1, 128, 1), (70, 256, 2), (300, 512, 1), (2374, 1024, 3), (1000, 4096, 8),
                                   (1000, 4096, 16), (77, 8192, 9), (130, 128, 16)])
def test_packed_gemv(tw, v, k, m):
    import torch
    rng = np.random.default_rng(v + k + m)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    wd, rsd = dev(w), dev(rs)
    wp = tw.i8_head_pack(wd)
    ws = tw.i8_head_argmax_workspace(v, m)
    y = host(tw.i8_head_gemv_packed(wp, rsd, v, k, dev(x)))
    y64, _ = oracle.head_bf16(w, rs, x)
    assert oracle.rel_l2(y, y64) <= TOL
    # the row-major single-pass kernel (the logits of the fused argmax) gives the same bits
    y_rm = torch.empty((m, v), dtype=torch.float32, device="cuda")
    tw.i8_head_argmax(wd, rsd, dev(x), workspace=ws, logits=y_rm)
    assert np.array_equal(y, host(y_rm))
    if m * k * 2 <= 48 * 1024:              # where i8_head_gemv takes that kernel as well
        assert np.array_equal(y, host(tw.i8_head_gemv(wd, rsd, dev(x))))
    q, sx = oracle.quantize_i8(x)
    acc = torch.empty((m, v), dtype=torch.int32, device="cuda")
    yi = host(tw.i8_head_gemv_packed_i8(wp, rsd, v, k, dev(q), dev(sx), acc=acc))
    acc0, yi64, _ = oracle.head_i8(w, rs, q, sx)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(yi, yi64) <= TOL
    tw.i8_head_argmax_i8(wd, rsd, dev(q), dev(sx), workspace=ws, logits=y_rm)
    assert np.array_equal(yi, host(y_rm))


def test_packed_head_full_size_sampled(tw):
    """The 151936 x 4096 head at M = 1, the shape and launch of the decode
    step: the packed copy sampled against the oracle's layout, the logits
    against the row-major kernel everywhere and against the oracle on
    sampled rows."""
    import torch
    v, k = 151936, 4096
    rng = np.random.default_rng(151936)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, 1, k)
    wd, rsd, xd = dev(w), dev(rs), dev(x)
    wp = tw.i8_head_pack(wd)
    assert wp.numel() == head_pack.packed_bytes(v, k)
    groups = rng.choice(v // 64, size=24, replace=False)
    for gi in groups:
        got = wp[gi * 64 * k:(gi + 1) * 64 * k].cpu().numpy()
        want = head_pack.pack(w[gi * 64:(gi + 1) * 64])
        assert np.array_equal(got, want), gi
    y = host(tw.i8_head_gemv_packed(wp, rsd, v, k, xd))
    assert np.array_equal(y, host(tw.i8_head_gemv(wd, rsd, xd)))
    rows = np.sort(np.concatenate([rng.choice(v, size=500, replace=False), [0, v - 1]]))
    y64, _ = oracle.head_bf16(w, rs, x, rows=rows)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    torch.cuda.synchronize()


def test_pack_leaves_bytes_past_its_size(tw):
    import torch
    v, k = 70, 256
    rng = np.random.default_rng(9)
    w, _ = synth.gen_head(rng, rng, v, k)
    n = tw.i8_head_packed_bytes(v, k)
    out = torch.full((n + 4096,), 77, dtype=torch.int8, device="cuda")
    tw.i8_head_pack(dev(w), out=out[:n])
    o = host(out)
    assert np.array_equal(o[:n], head_pack.pack(w))
    assert (o[n:] == 77).all()


@pytest.mark.parametrize("v,k,m", [(70, 256, 1), (1000, 4096, 4), (2374, 1024, 16), (151936, 4096, 1)])
def test_packed_argmax_matches_row_major(tw, v, k, m):
    """The fused head + greedy argmax over the packed copy: index, value and
    logits bit for bit those of the row-major call (bf16 and int8
    activations), and the int8 result the oracle's exact greedy choice."""
    import torch
    rng = np.random.default_rng(v + 5 * k + m)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    q, sx = oracle.quantize_i8(x)
    wd, rsd, xd, qd, sxd = dev(w), dev(rs), dev(x), dev(q), dev(sx)
    wp = tw.i8_head_pack(wd)
    ws = tw.i8_head_argmax_workspace(v, m)
    for fn_rm, fn_p, args in ((tw.i8_head_argmax, tw.i8_head_argmax_packed, (xd,)),
                              (tw.i8_head_argmax_i8, tw.i8_head_argmax_packed_i8, (qd, sxd))):
        y_rm = torch.empty((m, v), dtype=torch.float32, device="cuda")
        y_p = torch.empty((m, v), dtype=torch.float32, device="cuda")
        i_rm, v_rm = fn_rm(wd, rsd, *args, workspace=ws, logits=y_rm)
        i_rm, v_rm, y_rm = host(i_rm), host(v_rm), host(y_rm)
        i_p, v_p = fn_p(wp, rsd, v, k, *args, workspace=ws, logits=y_p)
        assert np.array_equal(host(i_p), i_rm)
        assert np.array_equal(host(v_p).view(np.uint32), v_rm.view(np.uint32))
        assert np.array_equal(host(y_p), y_rm)
    if v * k <= 4096 * 1000:
        acc0, _, _ = oracle.head_i8(w, rs, q, sx)
        idx0, val0 = oracle.greedy_argmax(oracle.head_i8_logits_f32(acc0, rs, sx))
        assert np.array_equal(host(i_p), idx0) and np.array_equal(host(v_p), val0)


def test_packed_argmax_padding_rows_never_win(tw):
    """V = 70 (58 zero padding rows in the copy) with every real logit
    negative: the winner is a real row, the oracle's exact greedy choice."""
    v, k, m = 70, 256, 2
    rng = np.random.default_rng(70)
    w = -rng.integers(1, 128, size=(v, k)).astype(np.int8)          # every weight in [-127, -1]
    rs = rng.uniform(0.002, 0.02, size=v).astype(np.float32)
    q = rng.integers(1, 128, size=(m, k)).astype(np.int8)           # positive activations
    sx = np.array([0.01, 0.5], np.float32)
    x = synth.f32_to_bf16_bits(np.ones((m, k), np.float32))
    wp = tw.i8_head_pack(dev(w))
    idx, val = tw.i8_head_argmax_packed_i8(wp, dev(rs), v, k, dev(q), dev(sx))
    acc0, _, _ = oracle.head_i8(w, rs, q, sx)
    idx0, val0 = oracle.greedy_argmax(oracle.head_i8_logits_f32(acc0, rs, sx))
    assert (val0 < 0).all()
    assert np.array_equal(host(idx), idx0) and np.array_equal(host(val), val0)
    idx_b, val_b = tw.i8_head_argmax_packed(wp, dev(rs), v, k, dev(x))
    idx_r, val_r = tw.i8_head_argmax(dev(w), dev(rs), dev(x))
    assert (host(idx_b) < v).all() and (host(val_b) < 0).all()
    assert np.array_equal(host(idx_b), host(idx_r)) and np.array_equal(host(val_b), host(val_r))


@pytest.mark.parametrize("v,k,m", [(70, 256, 1), (1000, 4096, 4), (300, 1024, 16), (151936, 4096, 1)])
def test_fv5b_packed_matches_row_major(tw, v, k, m):
    """The block-scaled (FV5B-style) head over the packed copy of its int8
    rows: logits, block sums, and the fused argmax's index, value and logits
    bit for bit those of the row-major calls (bf16 and int8 activations);
    against the oracle where it runs in seconds."""
    import torch
    from oracle import fv5b
    rng = np.random.default_rng(v + 3 * k + m)
    w, S = synth.gen_head_blocks(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    q, sx = oracle.quantize_i8(x)
    wd, Sd, xd, qd, sxd = dev(w), dev(S), dev(x), dev(q), dev(sx)
    wp = tw.i8_head_pack(wd)
    y_rm = host(tw.fv5b_head_gemv(wd, Sd, xd))
    assert np.array_equal(host(tw.fv5b_head_gemv_packed(wp, Sd, v, k, xd)), y_rm)
    acc_rm = torch.empty((m, v, k // 256), dtype=torch.int32, device="cuda")
    acc_p = torch.empty((m, v, k // 256), dtype=torch.int32, device="cuda")
    yi_rm = host(tw.fv5b_head_gemv_i8(wd, Sd, qd, sxd, acc=acc_rm))
    yi_p = host(tw.fv5b_head_gemv_packed_i8(wp, Sd, v, k, qd, sxd, acc=acc_p))
    assert np.array_equal(yi_p, yi_rm) and np.array_equal(host(acc_p), host(acc_rm))
    ws = tw.i8_head_argmax_workspace(v, m)
    for fn_rm, fn_p, args in ((tw.fv5b_head_argmax, tw.fv5b_head_argmax_packed, (xd,)),
                              (tw.fv5b_head_argmax_i8, tw.fv5b_head_argmax_packed_i8, (qd, sxd))):
        l_rm = torch.empty((m, v), dtype=torch.float32, device="cuda")
        l_p = torch.empty((m, v), dtype=torch.float32, device="cuda")
        i_rm, v_rm = fn_rm(wd, Sd, *args, workspace=ws, logits=l_rm)
        i_rm, v_rm, l_rm = host(i_rm), host(v_rm), host(l_rm)
        i_p, v_p = fn_p(wp, Sd, v, k, *args, workspace=ws, logits=l_p)
        assert np.array_equal(host(i_p), i_rm)
        assert np.array_equal(host(v_p).view(np.uint32), v_rm.view(np.uint32))
        assert np.array_equal(host(l_p), l_rm)
    if v * k <= 4096 * 1000:
        y64, _ = fv5b.head_bf16(w, S, x)
        assert oracle.rel_l2(y_rm, y64) <= TOL
        acc0 = fv5b.head_i8(w, S, q, sx)[0]
        assert np.array_equal(host(acc_p), acc0)
