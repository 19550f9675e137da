"""GPU parity: every call of the C ABI against the CPU oracle on the same
seeded inputs.  Integer results (packed bytes, statistics, int8 codes, int32
block accumulators) must match bit for bit; float outputs within a relative
L2 error of 1e-5 of the fp64 oracle (fp32 accumulation gives ~1e-7), or bit
for bit where the result is exact by construction."""
import numpy as np
import pytest

import oracle
from oracle import brute
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


def gen(n, k, m=1, seed=0, p0=synth.P_ZERO, pp=synth.P_PLUS):
    rng = np.random.default_rng(seed)
    t = synth.gen_ternary(rng, n, k, p0, pp)
    s = synth.gen_scales(rng, n, k // 128)
    x = synth.gen_x_bf16(rng, m, k)
    return t, s, x


def gpu_pack(tw, t, s):
    return tw.tern_pack(dev(t), dev(s))


SHAPES = [(16, 128), (20, 640), (3072, 1024), (37, 1536), (100, 2560), (1024, 4096), (48, 12288), (5, 384)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_pack_bit_exact(tw, n, k):
    t, s, _ = gen(n, k, seed=n + k)
    p = host(gpu_pack(tw, t, s))
    assert np.array_equal(p, oracle.pack(t, s))
    c = host(tw.tern_stats(gpu_pack(tw, t, s), n, k))
    assert c.tolist() == oracle.stats(oracle.pack(t, s), n, k).astype(np.int64).tolist()


def test_pack_golden_examples(tw):
    from test_oracle import _golden_inputs, _read_golden
    for name, e in _read_golden().items():
        t, s, x = _golden_inputs(e)
        p = host(gpu_pack(tw, t, s))
        assert p.size == e["total"]
        for off, val in e["bytes"].items():
            assert p[off] == val, (name, off)
        y = host(tw.tern_gemv(gpu_pack(tw, t, s), e["N"], e["K"], dev(x)))
        want = np.zeros(e["N"], np.float32)
        for r, v in e["y"].items():
            want[r] = v
        assert np.array_equal(y[0], want), name


@pytest.mark.parametrize("n,k,m", [(3072, 1024, 1), (16, 128, 1), (20, 640, 3), (37, 1536, 2), (100, 2560, 4),
                                   (1024, 4096, 7), (1024, 4096, 8), (48, 12288, 1), (48, 12288, 8),
                                   (64, 4096, 16), (33, 2048, 5), (256, 1152, 1)])
def test_gemv_bf16(tw, n, k, m):
    t, s, x = gen(n, k, m, seed=3 * n + k + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert y.shape == (m, n)
    assert oracle.rel_l2(y, y64) <= TOL, oracle.rel_l2(y, y64)
    # per-row check too: no single row may be badly off
    err = np.abs(y - y64).max(axis=1) / np.maximum(np.abs(y64).max(axis=1), 1e-30)
    assert err.max() < 1e-4


# Shapes that take the one-pass kernel (K a multiple of 512, M <= 4) in its
# different configurations on a 256-CU device: several row tiles per
# workgroup (interleaved across workgroups, the last ones holding fewer),
# 1 to 4 units per wave, spare unit slots, and activation staging of 1 to 4
# chunks per thread.  Rows are sampled (plus the last row tiles, which the
# short workgroups hold) and compared with the oracle.
@pytest.mark.parametrize("n,k,m", [(8813, 1024, 1),     # 3 row tiles per workgroup, last workgroup short
                                   (24576, 4096, 1),    # 2 units per wave
                                   (500, 20480, 1),     # 3 units per wave, 4 activation chunks per thread
                                   (53243, 2048, 1),    # 13 row tiles per workgroup, 4 units per wave
                                   (8813, 1536, 2),     # 9 units on 5 waves (one spare slot), M = 2
                                   (24576, 4096, 4),    # M = 4, 4 activation chunks per thread
                                   (100, 4096, 3)])     # M = 3, partial row tile
def test_gemv_bf16_one_pass_configs(tw, n, k, m):
    t, s, x = gen(n, k, m, seed=n + 7 * k + m)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemv(p, n, k, dev(x)))
    assert y.shape == (m, n) and np.isfinite(y).all()
    rng = np.random.default_rng(n)
    tail = np.arange(max(0, n - 3 * 16 * 13), n)
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 300), replace=False), tail, [0]]))
    y64, _ = oracle.gemv_bf16(oracle.pack(t[rows], s[rows]), len(rows), k, x)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL, oracle.rel_l2(y[:, rows], y64)
    # fixed summation order: a second call gives the same bytes
    assert np.array_equal(y, host(tw.tern_gemv(p, n, k, dev(x))))


# The one-pass kernel with int8 activations and with M = 5..8 bf16 rows:
# int32 block accumulators bit for bit where the shape allows the full
# oracle, sampled rows otherwise.
@pytest.mark.parametrize("n,k,m", [(8813, 1024, 1),     # 3 row tiles per workgroup, last workgroup short
                                   (24576, 4096, 2),    # 2 units per wave
                                   (500, 20480, 4),     # 3 units per wave, 4 activation chunks per thread
                                   (4096, 12288, 8),    # the 8B down shape at M = 8 (x fits only as int8)
                                   (1000, 4096, 5),     # M = 5, partial row tile
                                   (300, 1536, 7)])     # M = 7
def test_gemv_i8_one_pass_configs(tw, n, k, m):
    import torch
    t, s, x = gen(n, k, m, seed=n + 3 * k + m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    full = n * k * m <= 64 * 1024 * 1024
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemv_i8(p, n, k, dev(q0), dev(s0), acc=acc))
    assert y.shape == (m, n) and np.isfinite(y).all()
    if full:
        acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
        assert np.array_equal(host(acc), acc0)
        assert oracle.rel_l2(y, y64) <= TOL
    else:
        rng = np.random.default_rng(n)
        rows = np.unique(np.concatenate([rng.choice(n, 300, replace=False), np.arange(n - 48, n)]))
        acc0, y64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
        # the block sums of the sampled rows bit for bit (the one-pass int8
        # kernel on the 8B down shape at M = 8 and on 24576 x 4096 at M = 2)
        assert np.array_equal(host(acc)[:, rows], acc0)
        assert oracle.rel_l2(y[:, rows], y64) <= TOL
    # the instance without the debug accumulators (the production one) gives the same bytes
    assert np.array_equal(y, host(tw.tern_gemv_i8(p, n, k, dev(q0), dev(s0))))


@pytest.mark.parametrize("n,k,m", [(8813, 1024, 5), (24576, 4096, 8), (1000, 2048, 6), (300, 4096, 7)])
def test_gemv_bf16_one_pass_m5_to_8(tw, n, k, m):
    t, s, x = gen(n, k, m, seed=n + 5 * k + m)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemv(p, n, k, dev(x)))
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 300), replace=False), np.arange(max(0, n - 48), n)]))
    y64, _ = oracle.gemv_bf16(oracle.pack(t[rows], s[rows]), len(rows), k, x)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL, oracle.rel_l2(y[:, rows], y64)
    assert np.array_equal(y, host(tw.tern_gemv(p, n, k, dev(x))))


def test_gemv_config0(tw):
    """Config 0: one 3072x1024 ternary linear, M=1, seed 0."""
    t, s, x = synth.config0_inputs()
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), 3072, 1024, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), 3072, 1024, x)
    assert oracle.rel_l2(y, y64) <= TOL


def test_gemv_exact_cases(tw):
    n, k = 300, 1536
    t, s, x = gen(n, k, 2, seed=5)
    p = gpu_pack(tw, t, s)
    # all-zero weights -> exactly zero
    z = host(tw.tern_gemv(gpu_pack(tw, np.zeros_like(t), s), n, k, dev(x)))
    assert not z.any()
    # negated weights -> bit-exact negation (fixed summation order)
    ya = host(tw.tern_gemv(p, n, k, dev(x)))
    yb = host(tw.tern_gemv(gpu_pack(tw, -t, s), n, k, dev(x)))
    assert np.array_equal(ya, -yb)
    # deterministic: same inputs, same bytes
    assert np.array_equal(ya, host(tw.tern_gemv(p, n, k, dev(x))))
    # one-hot activation -> t[n,k] * scale exactly
    for kk in (0, 517, 1535):
        e = np.zeros((1, k), np.float32)
        e[0, kk] = 1.0
        y = host(tw.tern_gemv(p, n, k, dev(synth.f32_to_bf16_bits(e))))
        want = (t[:, kk] * s[:, kk // 128].view(np.float16).astype(np.float64)).astype(np.float32)
        assert np.array_equal(y[0], want)
    # scales 2^-6 and small-integer activations: exact binary fractions
    s6 = np.full_like(s, 0x2400)
    xi = synth.f32_to_bf16_bits(np.random.default_rng(1).integers(-8, 9, size=(3, k)).astype(np.float32))
    y = host(tw.tern_gemv(gpu_pack(tw, t, s6), n, k, dev(xi)))
    want = (synth.bf16_bits_to_f32(xi).astype(np.int64) @ t.T.astype(np.int64)) / 64.0
    assert np.array_equal(y, want.astype(np.float32))


def test_gemv_k_zero_and_empty(tw):
    import torch
    y = torch.full((2, 16), 7.0, device="cuda")
    p = torch.zeros(16, dtype=torch.uint8, device="cuda")
    x = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    tw.tern_gemv(p, 16, 0, x, y=y)
    assert not host(y).any()


@pytest.mark.parametrize("m,k", [(1, 1024), (3, 4096), (8, 12288), (2, 128), (16, 2048)])
def test_quantize_bit_exact(tw, m, k):
    x = synth.gen_x_bf16(np.random.default_rng(m * k), m, k)
    x[0, 5] = synth.f32_to_bf16_bits(np.array([9.5], np.float32))[0]
    q, sx = tw.tern_quantize_i8(dev(x))
    q0, s0 = oracle.quantize_i8(x)
    assert np.array_equal(host(q), q0)
    assert np.array_equal(host(sx).view(np.uint32), s0.view(np.uint32))


def test_quantize_edge_rows(tw):
    rows = np.zeros((4, 256), np.float32)
    rows[1, :10] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 126.5, -127.0, 0.0]
    rows[2, :5] = [254.0, 5.0, 7.0, -5.0, -254.0]
    rows[3, 7] = -3.0e-3
    x = synth.f32_to_bf16_bits(rows)
    q, sx = tw.tern_quantize_i8(dev(x))
    q0, s0 = oracle.quantize_i8(x)
    assert np.array_equal(host(q), q0) and np.array_equal(host(sx), s0)
    assert host(q)[1, :10].tolist() == [127, 2, 4, -2, 0, 0, 2, 126, -127, 0]
    assert host(sx)[0] == 0.0 and host(q)[3, 7] == -127


@pytest.mark.parametrize("n,k,m", [(16, 128, 1), (37, 640, 3), (300, 1536, 8), (1024, 4096, 7), (48, 12288, 2),
                                   (64, 2048, 16)])
def test_gemv_i8(tw, n, k, m):
    t, s, x = gen(n, k, m, seed=n * 7 + m)
    q, sx = tw.tern_quantize_i8(dev(x))
    q0, s0 = oracle.quantize_i8(x)
    assert np.array_equal(host(q), q0)
    p = gpu_pack(tw, t, s)
    import torch
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemv_i8(p, n, k, q, sx, acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL


def test_gemv_i8_unit_scale_full_shape(tw):
    """Scales 1.0 and s_x = 1: y is an exact integer (< 2^24), so bit-exact y
    proves the int32 block accumulators through the production path at a
    full 8B gate shape."""
    n, k = 12288, 4096
    rng = np.random.default_rng(21)
    t = synth.gen_ternary(rng, n, k)
    s1 = np.full((n, k // 128), 0x3C00, np.uint16)
    q = rng.integers(-127, 128, size=(2, k)).astype(np.int8)
    y = host(tw.tern_gemv_i8(gpu_pack(tw, t, s1), n, k, dev(q), dev(np.ones(2, np.float32))))
    want = (q.astype(np.int64) @ t.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("v,k,m", [(300, 512, 1), (151936 // 64, 1024, 3), (1000, 4096, 8), (77, 128, 16)])
def test_head(tw, v, k, m):
    rng = np.random.default_rng(v + k)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    y = host(tw.i8_head_gemv(dev(w), dev(rs), dev(x)))
    y64, _ = oracle.head_bf16(w, rs, x)
    assert oracle.rel_l2(y, y64) <= TOL
    q, sx = oracle.quantize_i8(x)
    import torch
    acc = torch.empty((m, v), dtype=torch.int32, device="cuda")
    yi = host(tw.i8_head_gemv_i8(dev(w), dev(rs), dev(q), dev(sx), acc=acc))
    acc0, yi64, _ = oracle.head_i8(w, rs, q, sx)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(yi, yi64) <= TOL


def test_head_one_hot_exact(tw):
    rng = np.random.default_rng(2)
    v, k = 500, 1024
    w, rs = synth.gen_head(rng, rng, v, k)
    e = np.zeros((1, k), np.float32)
    e[0, 333] = 1.0
    y = host(tw.i8_head_gemv(dev(w), dev(rs), dev(synth.f32_to_bf16_bits(e))))
    assert np.array_equal(y[0], (rs.astype(np.float64) * w[:, 333]).astype(np.float32))


@pytest.mark.parametrize("n,k,m", [(16, 128, 1), (40, 640, 64), (256, 1536, 130), (200, 2048, 300),
                                   (200, 4608, 300), (203, 4096, 300), (100, 8192, 1100)])
def test_prefill_small(tw, n, k, m):
    """Block sums bit for bit and y against the oracle.  The last three cases run the
    workgroup-shared decode with K split in two halves (9, 8 and 16 k-tiles of 512;
    N = 203 takes the row-scaling pass with 4-byte accesses)."""
    if k >= 4096:
        assert tw.tern_prefill_config(n, k, m)["split"] == 1
    t, s, x = gen(n, k, m, seed=n + m)
    q0, s0 = oracle.quantize_i8(x)
    import torch
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(gpu_pack(tw, t, s), n, k, dev(q0), dev(s0), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL


@pytest.mark.parametrize("proj,m", [("gate", 512), ("down", 512), ("gate", 2048), ("down", 2048)])
def test_prefill_full_shape_sampled(tw, proj, m):
    """8B gate / down shapes at M=512 (128 x 64 workgroup tiles) and M=2048
    (256 x 128 tiles): sampled output rows and activation rows against the
    oracle, plus the GEMV-i8 kernel on other rows (same arithmetic)."""
    n, k = synth.SHAPES_8B[proj]
    t, s, x = gen(n, k, m, seed=42)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0)))
    rng = np.random.default_rng(1)
    rows = rng.choice(n, 64, replace=False)
    mrows = np.unique(np.concatenate([rng.choice(m, 62, replace=False), [0, m - 1]]))
    _, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0[mrows], s0[mrows], rows=rows, want_acc=False)
    assert oracle.rel_l2(y[np.ix_(mrows, rows)], y64) <= TOL
    y8 = host(tw.tern_gemv_i8(p, n, k, dev(q0[m - 12:m - 4]), dev(s0[m - 12:m - 4])))
    assert oracle.rel_l2(y[m - 12:m - 4], y8) <= TOL


@pytest.mark.parametrize("n,k,m", [(40, 512, 128), (256, 1536, 130), (300, 2048, 300), (1000, 4096, 257),
                                   (17, 2560, 640)])
def test_prefill_no_debug_matches_oracle(tw, n, k, m):
    """The kernel instance without the debug accumulators (the one the
    benchmark times): several workgroup tiles, ragged in M and N, against the
    fp64 oracle, and bit for bit the same y as the instance that also writes
    the block sums."""
    import torch
    t, s, x = gen(n, k, m, seed=3 * n + m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0)))
    _, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0, want_acc=False)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    yi = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    assert np.array_equal(y, yi)


@pytest.mark.parametrize("n,k,m", [(300, 4096, 200), (300, 2048, 200), (200, 4096, 1100), (100, 2048, 1100),
                                   (4096, 2048, 2048)])
def test_prefill_exact_on_power_of_two_scales(tw, n, k, m):
    """Block scales from {1/4, 1/2, 1, 2}: every scaled block sum and every
    partial sum of the fold is a multiple of 1/4 below 2^22, so fp32 holds it
    exactly and y must equal fl32(s_x * sum_b scale_b * acc_b) bit for bit,
    with acc the oracle's exact block sums (on 64 sampled rows for the largest
    case).  K split in two halves (K = 4096 on a small grid) and whole
    (K = 2048); the last case has enough tiles to run the 256 x 128 workgroup
    tile, the others the 128 x 64 one."""
    c = tw.tern_prefill_config(n, k, m)
    assert c["BM"] == (256 if n == 4096 else 128) and c["split"] == (1 if k == 4096 else 0)
    rng = np.random.default_rng(8)
    t = synth.gen_ternary(rng, n, k)
    s = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float16), size=(n, k // 128)).view(np.uint16)
    q0 = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    s0 = rng.uniform(0.001, 0.01, m).astype(np.float32)
    y = host(tw.tern_gemm_prefill(gpu_pack(tw, t, s), n, k, dev(q0), dev(s0)))
    rows = np.arange(n) if n <= 300 else np.sort(np.random.default_rng(9).choice(n, 64, replace=False))
    acc0, _, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
    exact = (acc0.astype(np.float64) * s[rows].view(np.float16).astype(np.float64)[None]).sum(axis=2)
    assert np.abs(exact).max() < 2 ** 22 and np.array_equal(exact, exact.astype(np.float32).astype(np.float64))
    want = s0[:, None] * exact.astype(np.float32)
    assert np.array_equal(y[:, rows], want)


@pytest.mark.parametrize("n,k,m", [(300, 8192, 64), (100, 4096, 37), (37, 12288, 17), (1000, 4096, 48),
                                   (5000, 12288, 33), (77, 1536, 64)])
def test_prefill_small_m_split_k(tw, n, k, m):
    """17 <= M <= 64 (K a multiple of 512): above K = 4096, K split across the
    waves of a workgroup, activations staged a phase at a time, each decoded
    weight tile reused over the 16-row groups (ragged last group and last row
    tile); up to K = 4096 the register-resident kernel:
    block sums bit for bit, y against the oracle, and the production
    instance (no block sums) the same bytes."""
    import torch
    t, s, x = gen(n, k, m, seed=n + 7 * m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL
    y2 = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0)))
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("n,k,m", [(16, 512, 17), (1000, 1024, 40), (9000, 2048, 64), (12290, 4096, 33),
                                   (6000, 4096, 64), (333, 2560, 50), (700, 8192, 50), (130, 12288, 64),
                                   (4100, 12288, 19)])
def test_prefill_register_activations(tw, n, k, m):
    """17 <= M <= 64, K a multiple of 512: up to K = 4096 one wave per k-tile,
    above (K = 8192, 12288) eight waves of two or three k-tiles, holding their
    activations in registers over 1 to 4 row tiles per workgroup (ragged last
    row tile and last 16-row group, one to four row groups per grid row):
    block sums bit for bit, y against the oracle, and the production instance
    (no block sums) the same bytes."""
    import torch
    t, s, x = gen(n, k, m, seed=n + 11 * m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL
    assert np.array_equal(y, host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0))))


def test_prefill_register_activations_four_row_tiles_sampled(tw):
    """The fused 8B gate|up shape (24576 x 4096) at M = 64: four row tiles per
    workgroup, more workgroups than CUs; sampled rows' block sums bit for bit
    and y against the oracle, the production instance the same bytes."""
    import torch
    n, k, m = 24576, 4096, 64
    t, s, x = gen(n, k, m, seed=2457)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.choice(n, 80, replace=False), np.arange(n - 16, n), [0]]))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
    assert np.array_equal(host(acc)[:, rows], acc0)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    assert np.array_equal(y, host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0))))


@pytest.mark.parametrize("n,k,m", [(37, 12288, 100), (100, 4096, 16), (37, 12288, 9)])
def test_prefill_small_m_through_gemv_slices(tw, n, k, m):
    """Outside the split-K kernel's range with many 128-k blocks (M <= 16, or
    65 <= M < 128 where the shared-decode kernel does not pay) the call runs the
    int8 GEMV on 16-row slices of q (ragged last slice): block sums bit for bit,
    y against the oracle."""
    import torch
    assert tw.tern_prefill_config(n, k, m) is None
    t, s, x = gen(n, k, m, seed=n + 7 * m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL
    y2 = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0)))
    assert oracle.rel_l2(y2, y64) <= TOL


@pytest.mark.parametrize("n,k,m", [(300, 8192, 100), (100, 4096, 65), (2000, 12288, 127)])
def test_prefill_shared_decode_below_128(tw, n, k, m):
    """65 <= M < 128 where the measured model picks the shared-decode kernel with K
    split in two halves: block sums bit for bit and y against the oracle (sampled
    output rows for the largest case), the no-debug instance bit for bit the same."""
    import torch
    c = tw.tern_prefill_config(n, k, m)
    assert c is not None and c["BM"] == 128 and c["split"] == 1
    t, s, x = gen(n, k, m, seed=5 * n + m)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    rows = np.arange(n) if n <= 300 else np.sort(np.random.default_rng(3).choice(n, 64, replace=False))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
    assert np.array_equal(host(acc)[:, rows], acc0)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    assert np.array_equal(y, host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0))))


def test_prefill_split_full_down_shape_repeatable(tw):
    """The 8B down shape at M = 256 runs with K split in two halves (two atomic fp32
    addends per output): five calls give the same bytes, and sampled rows match the
    oracle with their block sums bit for bit."""
    import torch
    n, k = synth.SHAPES_8B["down"]
    m = 256
    c = tw.tern_prefill_config(n, k, m)
    assert c["split"] == 1 and c["grid_z"] == 2
    t, s, x = gen(n, k, m, seed=11)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    q, sx = dev(q0), dev(s0)
    ys = [host(tw.tern_gemm_prefill(p, n, k, q, sx)) for _ in range(5)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])
    rows = np.sort(np.random.default_rng(4).choice(n, 48, replace=False))
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    yd = host(tw.tern_gemm_prefill(p, n, k, q, sx, acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
    assert np.array_equal(host(acc)[:, rows], acc0)
    assert oracle.rel_l2(ys[0][:, rows], y64) <= TOL
    assert np.array_equal(yd, ys[0])


def test_prefill_down_m64_sampled(tw):
    """The 8B down shape at M = 64 (four GEMV slices): sampled rows."""
    n, k = synth.SHAPES_8B["down"]
    m = 64
    t, s, x = gen(n, k, m, seed=64)
    q0, s0 = oracle.quantize_i8(x)
    y = host(tw.tern_gemm_prefill(gpu_pack(tw, t, s), n, k, dev(q0), dev(s0)))
    rows = np.random.default_rng(5).choice(n, 64, replace=False)
    _, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0, rows=rows, want_acc=False)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL


def test_prefill_large_tiles_exact(tw):
    """A shape that takes the 256 x 128 workgroup tiles (M >= 1024), ragged
    in M: int32 block accumulators bit for bit."""
    n, k, m = 8192, 512, 1100
    t, s, x = gen(n, k, m, seed=77)
    q0, s0 = oracle.quantize_i8(x)
    import torch
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(gpu_pack(tw, t, s), n, k, dev(q0), dev(s0), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q0, s0)
    assert np.array_equal(host(acc), acc0)
    assert oracle.rel_l2(y, y64) <= TOL


def test_stats_noncanonical_hand_built(tw):
    """tern_stats on the hand-derived blob of tests/golden/stats_noncanonical.txt
    (three non-canonical sign bits in real rows, eight in a padding row that
    must not count), and the bf16 GEMV on it: non-canonical bits decode to 0."""
    from test_oracle import read_noncanonical_blob
    blob, n, k, counts, y_want = read_noncanonical_blob()
    p = dev(blob)
    assert host(tw.tern_stats(p, n, k)).astype(np.int64).tolist() == counts == [34, 3, 3]
    x = synth.f32_to_bf16_bits((np.arange(k) % 7 - 3).astype(np.float32)[None, :])
    y = host(tw.tern_gemv(p, n, k, dev(x)))
    assert np.array_equal(y[0], y_want.astype(np.float32))


@pytest.mark.parametrize("n,k", [(5, 256), (100, 2560), (3000, 4096)])
def test_stats_random_bytes(tw, n, k):
    """tern_stats on blobs of uniformly random bytes (about a quarter of all
    sign bits non-canonical) against the oracle's bit-by-bit count."""
    blob = np.random.default_rng(n + k).integers(0, 256, size=oracle.packed_bytes(n, k), dtype=np.uint8)
    c = host(tw.tern_stats(dev(blob), n, k)).astype(np.int64).tolist()
    want = oracle.stats(blob, n, k).astype(np.int64).tolist()
    assert c == want and want[2] > 0


FUSED_06B = {"qkv": (4096, 1024), "gateup": (6144, 1024)}


@pytest.mark.parametrize("shape", list(synth.SHAPES_06B) + list(FUSED_06B))
def test_06b_shapes_m1(tw, shape):
    """Every Qwen3-0.6B linear shape at M = 1 (and the fused q|k|v and
    gate|up launches of that model) in the benchmark's launch configuration:
    every output row against the oracle."""
    n, k = synth.SHAPES_06B[shape] if shape in synth.SHAPES_06B else FUSED_06B[shape]
    t, s, x = gen(n, k, 1, seed=n + 3 * k)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL, oracle.rel_l2(y, y64)
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max() + 1e-30)
    assert err.max() < 1e-5


@pytest.mark.parametrize("proj", ["gate", "up"])
def test_prefill_gate_up_m64_sampled(tw, proj):
    """The 8B gate and up shapes (12288 x 4096) at M = 64, which run the
    small-M prefill kernel: block sums of sampled output rows bit for bit
    (all 64 activation rows), y against the oracle on those rows, and the
    production instance (no debug output) bit for bit the same y."""
    import torch
    n, k = synth.SHAPES_8B[proj]
    m = 64
    lin = synth.Linear(2, 0, proj, n, k, synth.P_ZERO, synth.P_PLUS)
    t, s, _ = synth.linear_inputs(lin)
    x = synth.gen_x_bf16(np.random.default_rng(640 + len(proj)), m, k)
    q0, s0 = oracle.quantize_i8(x)
    p = gpu_pack(tw, t, s)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0), acc=acc))
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(n, 96, replace=False), np.arange(n - 16, n), [0]]))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, q0, s0)
    assert np.array_equal(host(acc)[:, rows], acc0)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    assert np.array_equal(y, host(tw.tern_gemm_prefill(p, n, k, dev(q0), dev(s0))))


@pytest.mark.parametrize("proj", list(synth.PROJ))
def test_full_8b_shapes_sampled(tw, proj):
    """Every 8B linear shape at M=1 (the decode configuration) in the launch
    configuration the benchmark uses: all rows vs brute force over a sampled
    set computed by the oracle."""
    n, k = synth.SHAPES_8B[proj]
    lin = synth.Linear(2, 1, proj, n, k, synth.P_ZERO_SPARSE if proj in ("gate", "down") else synth.P_ZERO,
                       synth.P_PLUS_SPARSE if proj in ("gate", "down") else synth.P_PLUS)
    t, s, x = synth.linear_inputs(lin)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemv(p, n, k, dev(x)))
    rows = np.random.default_rng(0).choice(n, 256, replace=False)
    y64, _ = oracle.gemv_bf16(oracle.pack(t[rows], s[rows]), 256, k, x)
    assert oracle.rel_l2(y[0, rows], y64[0]) <= TOL
    # occupancy of the packed blob matches the drawn states
    c = host(tw.tern_stats(p, n, k))
    assert c[0] == np.count_nonzero(t) and c[1] == np.count_nonzero(t < 0) and c[2] == 0


@pytest.mark.parametrize("m", [1, 3])
def test_gemv_multi_round_grid(tw, m):
    """A matrix too large for any one-round split (65541 x 4096): the one-pass
    kernel's grid runs in several rounds.  Sampled rows (incl. the ragged last
    tile) against the oracle, bf16 and int8 activations; the int8 block
    accumulators of the sampled rows bit for bit."""
    import torch
    n, k = 65541, 4096
    t, s, x = gen(n, k, m, seed=m)
    p = gpu_pack(tw, t, s)
    y = host(tw.tern_gemv(p, n, k, dev(x)))
    rows = np.unique(np.concatenate([np.random.default_rng(m).choice(n, 200, replace=False),
                                     np.arange(n - 21, n)]))
    packed_rows = oracle.pack(t[rows], s[rows])
    y64, _ = oracle.gemv_bf16(packed_rows, len(rows), k, x)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    q, sx = oracle.quantize_i8(x)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    yi = host(tw.tern_gemv_i8(p, n, k, dev(q), dev(sx), acc=acc))
    acc_o, yi64, _ = oracle.tern_i8(packed_rows, len(rows), k, q, sx)
    assert np.array_equal(host(acc)[:, rows], acc_o)
    assert oracle.rel_l2(yi[:, rows], yi64) <= TOL


@pytest.mark.parametrize("n,k,m", [(4096, 12288, 6), (4096, 12288, 8), (1005, 12288, 7), (300, 16384, 6)])
def test_gemv_bf16_two_phase(tw, n, k, m):
    """bf16 activations too large for LDS (large K, M >= 6): x staged half
    of K at a time; every output against the oracle."""
    assert tw.tern_gemv_config(n, k, m) is None and tw.tern_gemv_config(n, k, m, "ternary_bf16_phased")
    t, s, x = gen(n, k, m, seed=n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(37, 8192, 11), (1000, 8192, 9), (4100, 8192, 15), (4096, 8192, 12)])
def test_gemv_bf16_two_phase_two_row_tiles(tw, n, k, m):
    """bf16 activations whose halves of K would need more than 8 chunks per
    thread with one row tile per workgroup and whose x fits neither a
    one-pass split nor the persistent fast path (K = 8192 at M = 9..15): the
    two-phase kernel with two row tiles per workgroup, the weights read once.
    37, 1000 and 4100 rows give odd row-tile counts, so the last workgroup's
    second tile loads its first and stores nothing.  Every output against
    the oracle."""
    c = tw.tern_gemv_config(n, k, m, "ternary_bf16_phased")
    assert tw.tern_gemv_config(n, k, m) is None and c is not None and c["R"] == 2
    t, s, x = gen(n, k, m, seed=3 * n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(1000, 4096, 9), (37, 4096, 12), (4100, 4096, 16), (12288, 4096, 13),
                                   (2000, 2048, 16)])
def test_gemv_bf16_sixteen_chunks(tw, n, k, m):
    """bf16 activations of 9..16 rows whose x (up to 128 KiB) fits a CU's LDS
    only with 16 staged chunks per thread: the one-pass kernel in one
    resident round (4100 rows: two row tiles per workgroup, the last
    workgroup's second tile past the end; 12288 rows: three row tiles and two
    units per wave).  Every output against the oracle."""
    c = tw.tern_gemv_config(n, k, m)
    assert c is not None and c["XC"] == 16 and not c["rounds"]
    t, s, x = gen(n, k, m, seed=7 * n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(21000, 4096, 14), (20001, 4096, 16), (24576, 4096, 16)])
def test_gemv_bf16_partials_over_x(tw, n, k, m):
    """bf16 activations of 9..16 rows whose x and the partials of a one-round
    split do not fit a CU's LDS side by side (the 8B fused gate|up at M = 16):
    the one-pass kernel writes the partials over x after a second barrier.
    20001 rows: 16 staged chunks and a last workgroup with tiles past the end;
    the fused shape on sampled rows, the others in full."""
    c = tw.tern_gemv_config(n, k, m)
    side = m * (k + 8) * 2 + (c["R"] * (k // 512) + 1) * 4 * 64 * 4
    assert c is not None and not c["rounds"] and side > 160 * 1024 and c["lds"] < side
    t, s, x = gen(n, k, m, seed=13 * n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    rows = np.arange(n) if n < 24000 else np.unique(np.r_[np.arange(0, 40), np.random.default_rng(6).choice(n, 400),
                                                           np.arange(n - 40, n)])
    y64, _ = oracle.gemv_bf16(oracle.pack(t[rows], s[rows]), len(rows), k, x)
    assert oracle.rel_l2(y[:, rows], y64) <= TOL
    err = np.abs(y[:, rows] - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(4096, 12288, 16), (1005, 12288, 9), (37, 12288, 12), (300, 12288, 13)])
def test_gemv_bf16_three_phase(tw, n, k, m):
    """bf16 activations of more than 8 rows whose halves of K exceed LDS (the
    8B down shape at M = 9..16): x staged a third of K at a time, the weights
    read once; every output against the oracle."""
    assert tw.tern_gemv_config(n, k, m) is None and tw.tern_gemv_config(n, k, m, "ternary_bf16_phased") is None
    assert tw.tern_gemv_config(n, k, m, "ternary_bf16_phased3") is not None
    t, s, x = gen(n, k, m, seed=5 * n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(1000, 8192, 16), (37, 8192, 16)])
def test_gemv_bf16_row_halves(tw, n, k, m):
    """bf16 activations of more than 8 rows that fit no one-pass, two-phase
    or three-phase configuration (K = 8192 at M = 16: half of x is 131 KB,
    and K is not a multiple of 3 k-tiles): the call runs on rows 0..7 and
    8..M-1 through those kernels; every output against the oracle."""
    assert tw.tern_gemv_config(n, k, m) is None and tw.tern_gemv_config(n, k, m, "ternary_bf16_phased") is None
    assert tw.tern_gemv_config(n, k, m, "ternary_bf16_phased3") is None
    assert (tw.tern_gemv_config(n, k, 8) is not None or
            tw.tern_gemv_config(n, k, 8, "ternary_bf16_phased") is not None)
    t, s, x = gen(n, k, m, seed=2 * n + m)
    y = host(tw.tern_gemv(gpu_pack(tw, t, s), n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL
    err = np.abs(y - y64).max(axis=0) / (np.abs(y64).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(4096, 12288, 13), (1005, 12288, 16)])
def test_gemv_i8_two_phase(tw, n, k, m):
    """int8 activations too large for LDS (M >= 13 at K = 12288): block
    accumulators bit for bit, y within tolerance."""
    import torch
    assert tw.tern_gemv_config(n, k, m, "ternary_int8") is None
    assert tw.tern_gemv_config(n, k, m, "ternary_int8_phased")
    t, s, x = gen(n, k, m, seed=2 * n + m)
    q, sx = oracle.quantize_i8(x)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemv_i8(gpu_pack(tw, t, s), n, k, dev(q), dev(sx), acc=acc))
    acc_o, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q, sx)
    assert np.array_equal(host(acc), acc_o)
    assert oracle.rel_l2(y, y64) <= TOL
