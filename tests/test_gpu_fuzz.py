"""Seeded random shapes through every GEMV path against the oracle: N from 1
to about 13000 (ragged row tiles), K any multiple of 128 up to 12288 (k-tiles
of fewer than four blocks included), M from 1 to 16, so the launch pickers
land on every kernel (one-pass with 1..16 staged chunks, per-wave slices,
two- and three-phase, persistent, general) with shapes no targeted test
names; the same for the prefill contraction over M from 17 to about 2300.
bf16: relative L2 within 1e-5 and every output row within 1e-4;
int8: the int32 block sums bit for bit; five-level (K a multiple of 512):
as bf16."""
import numpy as np
import pytest

import oracle
from oracle import fv5
from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _cases(seed, count, kmult, max_elems):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        kind = rng.integers(0, 3)
        n = int(rng.integers(1, 41) if kind == 0 else (rng.integers(41, 3001) if kind == 1 else
                                                        rng.integers(3001, 13001)))
        if rng.random() < 0.5:
            k = kmult * int(rng.integers(1, 12288 // kmult + 1))
        else:
            k = 512 * int(rng.integers(1, 25))
        if k % kmult:
            continue
        m = int(rng.integers(1, 17))
        if n * k > max_elems:
            continue
        out.append((n, k, m))
    return out


TERN_CASES = _cases(20261203, 36, 128, 40_000_000)


def _prefill_cases(seed, count):
    """M over every prefill kernel's range (17..64 K-split, 65..127 general, 128..1023 and
    1024.. workgroup-shared decode), K a multiple of 512 mostly, 128 otherwise."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m = int(rng.choice([rng.integers(17, 65), rng.integers(65, 128), rng.integers(128, 1024),
                            rng.integers(1024, 2300)]))
        k = 512 * int(rng.integers(1, 17)) if rng.random() < 0.7 else 128 * int(rng.integers(1, 49))
        n_max = min(3000, 12_000_000 // (m * (k // 128)))        # block sums within 48 MB
        if n_max < 1:
            continue
        out.append((int(rng.integers(1, n_max + 1)), k, m))
    return out


PREFILL_CASES = _prefill_cases(20261205, 16)
FV5_CASES = _cases(20261204, 14, 512, 24_000_000)      # the five-level blob needs K % 512 == 0


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


def _rows_ok(y, want):
    err = np.abs(y - want).max(axis=0) / (np.abs(want).max(axis=0) + 1e-3)
    return float(err.max())


@pytest.mark.parametrize("n,k,m", TERN_CASES)
def test_fuzz_ternary(tw, n, k, m):
    import torch
    rng = np.random.default_rng(n * 131 + k * 7 + m)
    t = synth.gen_ternary(rng, n, k)
    s = synth.gen_scales(rng, n, k // 128)
    x = synth.gen_x_bf16(rng, m, k)
    packed = tw.tern_pack(dev(t), dev(s))
    blob = oracle.pack(t, s)
    where = (n, k, m, tw.tern_gemv_config(n, k, m), tw.tern_gemv_config(n, k, m, "ternary_int8"))
    y = host(tw.tern_gemv(packed, n, k, dev(x)))
    y64, _ = oracle.gemv_bf16(blob, n, k, x)
    assert oracle.rel_l2(y, y64) <= TOL, where
    assert _rows_ok(y, y64) < 1e-4, where
    q, sx = oracle.quantize_i8(x)
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    yi = host(tw.tern_gemv_i8(packed, n, k, dev(q), dev(sx), acc=acc))
    acc0, yi64, _ = oracle.tern_i8(blob, n, k, q, sx)
    assert np.array_equal(host(acc), acc0), where
    assert oracle.rel_l2(yi, yi64) <= TOL, where


@pytest.mark.parametrize("n,k,m", PREFILL_CASES)
def test_fuzz_prefill(tw, n, k, m):
    import torch
    rng = np.random.default_rng(n * 139 + k * 13 + m)
    t = synth.gen_ternary(rng, n, k)
    s = synth.gen_scales(rng, n, k // 128)
    x = synth.gen_x_bf16(rng, m, k)
    q, sx = oracle.quantize_i8(x)
    packed = tw.tern_pack(dev(t), dev(s))
    acc = torch.empty((m, n, k // 128), dtype=torch.int32, device="cuda")
    y = host(tw.tern_gemm_prefill(packed, n, k, dev(q), dev(sx), acc=acc))
    acc0, y64, _ = oracle.tern_i8(oracle.pack(t, s), n, k, q, sx)
    assert np.array_equal(host(acc), acc0), (n, k, m)
    assert oracle.rel_l2(y, y64) <= TOL, (n, k, m)
    # the production instance (no block sums) gives the same bytes
    assert np.array_equal(y, host(tw.tern_gemm_prefill(packed, n, k, dev(q), dev(sx)))), (n, k, m)


@pytest.mark.parametrize("n,k,m", FV5_CASES)
def test_fuzz_five_level(tw, n, k, m):
    rng = np.random.default_rng(n * 137 + k * 11 + m)
    lv = synth.gen_levels5(rng, n, k)
    lo, hi = synth.gen_scales5(rng, n, k // 256)
    x = synth.gen_x_bf16(rng, m, k)
    packed = tw.tern5_pack(dev(lv), dev(lo), dev(hi))
    where = (n, k, m, tw.tern_gemv_config(n, k, m, "fv5_bf16"))
    y = host(tw.tern5_gemv(packed, n, k, dev(x)))
    want, _ = fv5.gemv_bf16_levels(lv, lo, hi, x)
    assert oracle.rel_l2(y, want) <= TOL, where
    assert _rows_ok(y, want) < 1e-4, where
