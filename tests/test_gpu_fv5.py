"""GPU parity of the five-level (FV5-style) calls against the CPU oracle
(oracle/fv5.py) on the same seeded inputs: packed bytes and the int8 path's
per-block sums of each magnitude bit for bit, GEMV outputs within a relative
L2 error of 1e-5 of the fp64 oracle (fp32 accumulation of exact products
gives ~1e-7)."""
import numpy as np
import pytest

from oracle import fv5
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


def gen(n, k, m=1, seed=0):
    rng = np.random.default_rng(seed)
    lv = synth.gen_levels5(rng, n, k)
    lo, hi = synth.gen_scales5(rng, n, k // 256)
    x = synth.gen_x_bf16(rng, m, k)
    return lv, lo, hi, x


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def gpu_pack(tw, lv, lo, hi):
    return tw.tern5_pack(dev(lv), dev(lo), dev(hi))


@pytest.mark.parametrize("n,k", [(16, 512), (1, 512), (37, 1536), (100, 1024), (5, 2560)])
def test_pack5_bit_exact(tw, n, k):
    lv, lo, hi, _ = gen(n, k, seed=n + k)
    assert np.array_equal(host(gpu_pack(tw, lv, lo, hi)), fv5.pack(lv, lo, hi))


def test_pack5_golden_examples(tw):
    from test_oracle_fv5 import _read_golden, golden_inputs
    for name, e in _read_golden().items():
        lv, lo, hi, x = golden_inputs(e)
        p = host(gpu_pack(tw, lv, lo, hi))
        assert p.size == e["total"]
        nzb = {off: int(p[off]) for off in np.nonzero(p)[0]}
        assert nzb == e["bytes"], name
        y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), e["N"], e["K"], dev(x)))
        want = np.zeros(e["N"], np.float32)
        for r, v in e["y"].items():
            want[r] = v
        assert np.array_equal(y[0], want), name


def test_pack5_clamps_out_of_range_levels(tw):
    rng = np.random.default_rng(7)
    n, k = 20, 1024
    lv = rng.integers(-128, 128, size=(n, k), dtype=np.int16).astype(np.int8)
    lo, hi = synth.gen_scales5(rng, n, k // 256)
    want = fv5.pack(np.clip(lv, -2, 2), lo, hi)
    assert np.array_equal(host(gpu_pack(tw, lv, lo, hi)), want)


CASES = [(16, 512, 1), (37, 1536, 1), (37, 1536, 2), (100, 2048, 3), (300, 4096, 4), (1000, 2560, 5),
         (600, 1024, 8), (129, 3072, 16), (4100, 512, 1), (257, 8192, 12)]


@pytest.mark.parametrize("n,k,m", CASES)
def test_gemv5_matches_oracle(tw, n, k, m):
    lv, lo, hi, x = gen(n, k, m, seed=3 * n + k + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    want, _ = fv5.gemv_bf16_levels(lv, lo, hi, x)
    assert y.shape == (m, n)
    assert rel_l2(y, want) < TOL
    # row by row too: no row may hide behind the others
    err = np.abs(y - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(40, 24576, 8), (64, 32768, 16), (33, 20480, 1)])
def test_gemv5_general_path(tw, n, k, m):
    """Activations too large to stage in LDS: the general kernel runs."""
    lv, lo, hi, x = gen(n, k, m, seed=n + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    want, _ = fv5.gemv_bf16_levels(lv, lo, hi, x)
    assert rel_l2(y, want) < TOL


@pytest.mark.parametrize("n,k,m", [(37, 12288, 6), (300, 12288, 8), (100, 16384, 5), (17, 16384, 4)])
def test_gemv5_two_phase(tw, n, k, m):
    """bf16 activations larger than LDS but half of them not: the two-phase
    kernel (K staged one half at a time); ragged row tiles included."""
    assert tw.tern_gemv_config(n, k, m, "fv5_bf16_phased") is not None
    lv, lo, hi, x = gen(n, k, m, seed=7 * n + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    want, _ = fv5.gemv_bf16_levels(lv, lo, hi, x)
    assert rel_l2(y, want) < TOL
    err = np.abs(y - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(1000, 4096, 9), (4100, 4096, 16), (12288, 4096, 13)])
def test_gemv5_sixteen_chunks(tw, n, k, m):
    """bf16 activations of 9..16 rows that fit a CU's LDS only with 16 staged
    chunks per thread (the one-pass kernel in one resident round, where the
    occupancy allows it; the two-phase kernel otherwise): every output
    against the oracle."""
    c = tw.tern_gemv_config(n, k, m, "fv5_bf16")
    assert c is not None and c["XC"] == 16
    lv, lo, hi, x = gen(n, k, m, seed=11 * n + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    want, _ = fv5.gemv_bf16_levels(lv, lo, hi, x)
    assert rel_l2(y, want) < TOL
    err = np.abs(y - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(12300, 4096, 16), (21000, 4096, 14), (24576, 4096, 16)])
def test_gemv5_partials_over_x(tw, n, k, m):
    """bf16 M = 14..16 at K = 4096 where x and the partials of a one-round
    split do not fit side by side (the 8B fused gate|up shape): the one-pass
    kernel with the partials written over x after a second barrier; 12300 and
    21000 rows in full (the last workgroup with tiles past the end), the fused
    shape on sampled rows."""
    c = tw.tern_gemv_config(n, k, m, "fv5_bf16")
    side = m * (k + 8) * 2 + (c["R"] * (k // 512) + 1) * 4 * 64 * 4
    assert not c["rounds"] and side > 160 * 1024 and c["lds"] < side
    lv, lo, hi, x = gen(n, k, m, seed=17 * n + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    rows = np.arange(n) if n < 24000 else np.unique(np.r_[np.arange(0, 40), np.random.default_rng(7).choice(n, 300),
                                                           np.arange(n - 40, n)])
    want, _ = fv5.gemv_bf16_levels(lv[rows], lo[rows], hi[rows], x)
    assert rel_l2(y[:, rows], want) < TOL
    err = np.abs(y[:, rows] - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


@pytest.mark.parametrize("n,k,m", [(4000, 8192, 12), (6150, 8192, 10)])
def test_gemv5_two_phase_two_row_tiles(tw, n, k, m):
    """bf16 M = 10..15 at K = 8192, x beyond LDS and a half of it more than 8
    chunks per thread with one row tile per workgroup: the two-phase kernel
    with two row tiles per workgroup (6150 rows: the last workgroup's second
    tile past the end); every output against the oracle."""
    c = tw.tern_gemv_config(n, k, m, "fv5_bf16_phased")
    assert tw.tern_gemv_config(n, k, m, "fv5_bf16") is None and c is not None and c["R"] == 2
    lv, lo, hi, x = gen(n, k, m, seed=9 * n + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    rows = np.arange(n) if n < 16000 else np.unique(np.r_[np.arange(0, 40), np.random.default_rng(5).choice(n, 300),
                                                                np.arange(n - 40, n)])
    want, _ = fv5.gemv_bf16_levels(lv[rows], lo[rows], hi[rows], x)
    assert rel_l2(y[:, rows], want) < TOL
    err = np.abs(y[:, rows] - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    assert err.max() < 1e-4


def test_gemv5_deterministic_and_stream_order(tw):
    import torch
    n, k, m = 6144, 4096, 1
    lv, lo, hi, x = gen(n, k, m, seed=11)
    p = gpu_pack(tw, lv, lo, hi)
    xd = dev(x)
    y1 = host(tw.tern5_gemv(p, n, k, xd))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = tw.tern5_gemv(p, n, k, xd)
    s.synchronize()
    assert np.array_equal(y1, y2.cpu().numpy())


# the five-level linears of one 8B layer (q|k|v and gate|up fused) at decode
# and verify sizes; outputs sampled on rows the oracle computes one by one
FULL = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]


@pytest.mark.parametrize("n,k", FULL)
@pytest.mark.parametrize("m", [1, 8, 16])
def test_gemv5_full_size_sampled_rows(tw, n, k, m):
    lv, lo, hi, x = gen(n, k, m, seed=n + k + m)
    y = host(tw.tern5_gemv(gpu_pack(tw, lv, lo, hi), n, k, dev(x)))
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([rng.choice(n, 48, replace=False), [0, 15, 16, n - 1]]))
    want, _ = fv5.gemv_bf16_levels(lv[rows], lo[rows], hi[rows], x)
    assert rel_l2(y[:, rows], want) < TOL
    assert np.isfinite(y).all()


def test_pack5_full_size_sampled_tiles(tw):
    """Tiles are contiguous in the blob (row tile outermost), so a 16-row
    slice packed by the oracle equals that tile's bytes of the full blob."""
    n, k = 4096, 12288
    lv, lo, hi, _ = gen(n, k, seed=5)
    p = host(gpu_pack(tw, lv, lo, hi))
    nkt = k // 512
    plane_tile = 3072 * nkt                    # plane bytes per row tile
    scale_tile = 16 * (k // 256) * 8           # scale bytes per row tile
    planes_total = n * k * 3 // 8
    for rt in (0, 137, n // 16 - 1):
        sub = fv5.pack(lv[16 * rt:16 * rt + 16], lo[16 * rt:16 * rt + 16], hi[16 * rt:16 * rt + 16])
        assert np.array_equal(p[rt * plane_tile:(rt + 1) * plane_tile], sub[:plane_tile])
        s0 = planes_total + rt * scale_tile
        assert np.array_equal(p[s0:s0 + scale_tile], sub[plane_tile:])


# ---------------------------------------------------------------- int8 activations

def gen_q(m, k, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(-127, 128, size=(m, k)).astype(np.int8), rng.uniform(0.005, 0.05, m).astype(np.float32)


def test_gemv5_i8_golden_examples(tw):
    import torch
    from test_oracle_fv5 import _read_golden, golden_inputs, golden_q
    for name, e in _read_golden().items():
        lv, lo, hi, _ = golden_inputs(e)
        q, sx = golden_q(e["K"])
        acc = torch.empty((1, e["N"], e["K"] // 256, 2), dtype=torch.int32, device="cuda")
        y = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), e["N"], e["K"], dev(q), dev(sx), acc=acc))
        want = np.zeros((1, e["N"], e["K"] // 256, 2), np.int64)
        for (r, b), (a_lo, a_hi) in e["acc"].items():
            want[0, r, b] = (a_lo, a_hi)
        assert np.array_equal(host(acc).astype(np.int64), want), name
        wy = np.zeros(e["N"], np.float32)
        for r, v in e["yq"].items():
            wy[r] = v
        assert np.array_equal(y[0], wy), name


I8_CASES = [(16, 512, 1), (37, 1536, 1), (37, 1536, 2), (100, 2048, 3), (300, 4096, 4), (1000, 2560, 5),
            (600, 1024, 8), (129, 3072, 16), (4100, 512, 1), (40, 24576, 8), (64, 32768, 16)]


@pytest.mark.parametrize("n,k,m", I8_CASES)
def test_gemv5_i8_block_sums_exact(tw, n, k, m):
    import torch
    lv, lo, hi, _ = gen(n, k, 1, seed=5 * n + k + m)
    q, sx = gen_q(m, k, seed=n + m)
    acc = torch.empty((m, n, k // 256, 2), dtype=torch.int32, device="cuda")
    y = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), n, k, dev(q), dev(sx), acc=acc))
    acc64, y64, _ = fv5.gemv_i8_levels(lv, lo, hi, q, sx)
    assert np.array_equal(host(acc).astype(np.int64), acc64)
    assert rel_l2(y, y64) < TOL
    # without the debug output the same kernel gives the same y
    y2 = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), n, k, dev(q), dev(sx)))
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("n,k", FULL)
@pytest.mark.parametrize("m", [1, 8])
def test_gemv5_i8_full_size_sampled_rows(tw, n, k, m):
    lv, lo, hi, _ = gen(n, k, 1, seed=n + 2 * k + m)
    q, sx = gen_q(m, k, seed=n + m)
    y = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), n, k, dev(q), dev(sx)))
    rng = np.random.default_rng(n + 1)
    rows = np.unique(np.concatenate([rng.choice(n, 48, replace=False), [0, 15, 16, n - 1]]))
    _, want, _ = fv5.gemv_i8_levels(lv[rows], lo[rows], hi[rows], q, sx)
    assert rel_l2(y[:, rows], want) < TOL


@pytest.mark.parametrize("n,k,m", [(37, 12288, 13), (100, 12288, 16), (40, 16384, 14)])
def test_gemv5_i8_two_phase_block_sums_exact(tw, n, k, m):
    """int8 activations larger than LDS: the two-phase kernel; per-block sums
    of each magnitude bit exact."""
    import torch
    assert tw.tern_gemv_config(n, k, m, "fv5_int8_phased") is not None
    lv, lo, hi, _ = gen(n, k, 1, seed=9 * n + m)
    q, sx = gen_q(m, k, seed=n + 3 * m)
    acc = torch.empty((m, n, k // 256, 2), dtype=torch.int32, device="cuda")
    y = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), n, k, dev(q), dev(sx), acc=acc))
    acc64, y64, _ = fv5.gemv_i8_levels(lv, lo, hi, q, sx)
    assert np.array_equal(host(acc).astype(np.int64), acc64)
    assert rel_l2(y, y64) < TOL


@pytest.mark.parametrize("m", [13, 16])
def test_gemv5_i8_down_full_size_two_phase(tw, m):
    n, k = 4096, 12288
    lv, lo, hi, _ = gen(n, k, 1, seed=m)
    q, sx = gen_q(m, k, seed=m + 1)
    y = host(tw.tern5_gemv_i8(gpu_pack(tw, lv, lo, hi), n, k, dev(q), dev(sx)))
    rows = np.unique(np.concatenate([np.random.default_rng(m).choice(n, 48, replace=False), [0, 15, n - 1]]))
    _, want, _ = fv5.gemv_i8_levels(lv[rows], lo[rows], hi[rows], q, sx)
    assert rel_l2(y[:, rows], want) < TOL


def test_gemv5_multi_round_grid(tw):
    """65541 x 4096 five-level weights: the one-pass grid runs in several
    rounds; sampled rows (incl. the ragged last tile), bf16 and int8."""
    n, k, m = 65541, 4096, 2
    lv, lo, hi, x = gen(n, k, m, seed=41)
    q, sx = gen_q(m, k, seed=42)
    p = gpu_pack(tw, lv, lo, hi)
    y = host(tw.tern5_gemv(p, n, k, dev(x)))
    yi = host(tw.tern5_gemv_i8(p, n, k, dev(q), dev(sx)))
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(n, 200, replace=False), np.arange(n - 21, n)]))
    want, _ = fv5.gemv_bf16_levels(lv[rows], lo[rows], hi[rows], x)
    assert rel_l2(y[:, rows], want) < TOL
    _, want_i, _ = fv5.gemv_i8_levels(lv[rows], lo[rows], hi[rows], q, sx)
    assert rel_l2(yi[:, rows], want_i) < TOL
