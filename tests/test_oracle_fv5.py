"""The five-level oracle (oracle/fv5.py) pinned to things other than itself:
hand-derived bytes and outputs, brute force, the ternary oracle where the two
formats coincide, and invariants."""
import os

import numpy as np
import pytest

import oracle
from oracle import fv5
from ternary_weight_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fv5_examples.txt")


def _read_golden():
    ex, cur = {}, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "example":
            cur = {"name": tok[1], "N": int(tok[3]), "K": int(tok[5]), "total": int(tok[7]),
                   "l": [], "s": [], "bytes": {}, "y": {}, "acc": {}, "yq": {}}
        elif tok[0] == "l":
            cur["l"].append((int(tok[1]), int(tok[2]), int(tok[3])))
        elif tok[0] == "s":
            cur["s"].append((int(tok[1]), int(tok[2]), float(tok[3]), float(tok[4])))
        elif tok[0] == "byte":
            cur["bytes"][int(tok[1])] = int(tok[2], 16)
        elif tok[0] == "y":
            cur["y"][int(tok[1])] = float(tok[2])
        elif tok[0] == "acc":
            cur["acc"][(int(tok[1]), int(tok[2]))] = (int(tok[3]), int(tok[4]))
        elif tok[0] == "yq":
            cur["yq"][int(tok[1])] = float(tok[2])
        elif tok[0] == "end":
            ex[cur["name"]] = cur
    return ex


def golden_inputs(e):
    n, k = e["N"], e["K"]
    lv = np.zeros((n, k), np.int8)
    for (r, c, v) in e["l"]:
        lv[r, c] = v
    lo = np.zeros((n, k // 256), np.float32)
    hi = np.zeros((n, k // 256), np.float32)
    for (r, b, a, c) in e["s"]:
        lo[r, b], hi[r, b] = a, c
    x = synth.f32_to_bf16_bits((np.arange(k) % 7 - 3).astype(np.float32)[None, :])
    return lv, lo, hi, x


def golden_q(k):
    return ((np.arange(k) % 5) - 2).astype(np.int8)[None, :], np.array([0.5], np.float32)


@pytest.mark.parametrize("name", ["ex1", "ex2"])
def test_golden_gemv_i8(name):
    e = _read_golden()[name]
    lv, lo, hi, _ = golden_inputs(e)
    q, sx = golden_q(e["K"])
    acc, y64, _ = fv5.gemv_i8(fv5.pack(lv, lo, hi), e["N"], e["K"], q, sx)
    want = np.zeros_like(acc)
    for (r, b), (a_lo, a_hi) in e["acc"].items():
        want[0, r, b] = (a_lo, a_hi)
    assert np.array_equal(acc, want)
    wy = np.zeros(e["N"])
    for r, v in e["yq"].items():
        wy[r] = v
    assert np.array_equal(y64[0], wy)


def test_gemv_i8_vs_brute_force_and_ternary():
    rng = np.random.default_rng(5)
    n, k, m = 4, 512, 2
    lv, lo, hi = gen5(rng, n, k)
    q = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.01, 0.1, m).astype(np.float32)
    acc, y64, _ = fv5.gemv_i8(fv5.pack(lv, lo, hi), n, k, q, sx)
    for mm in range(m):
        for nn in range(n):
            tot = 0.0
            for b in range(k // 256):
                a = [0, 0]
                for kk in range(256 * b, 256 * b + 256):
                    lvl = int(lv[nn, kk])
                    if lvl:
                        a[abs(lvl) - 1] += (1 if lvl > 0 else -1) * int(q[mm, kk])
                assert acc[mm, nn, b].tolist() == a
                tot += float(lo[nn, b]) * a[0] + float(hi[nn, b]) * a[1]
            assert abs(y64[mm, nn] - float(sx[mm]) * tot) <= 1e-12 * (1 + abs(tot))
    # levels in {-1, 0, +1}: the ternary int8 oracle (plain C) with scale s_lo
    t = synth.gen_ternary(rng, 40, 1024)
    s16 = synth.gen_scales(rng, 40, 4)
    lo2 = s16.view(np.float16).astype(np.float32)
    q2 = rng.integers(-127, 128, size=(3, 1024)).astype(np.int8)
    sx2 = rng.uniform(0.01, 0.1, 3).astype(np.float32)
    acc5, y5, _ = fv5.gemv_i8_levels(t, lo2, lo2 * 3, q2, sx2)
    acc3, y3, _ = oracle.tern_i8(oracle.pack(t, np.repeat(s16, 2, axis=1)), 40, 1024, q2, sx2)
    assert np.array_equal(acc5[..., 0], acc3.astype(np.int64).reshape(3, 40, 4, 2).sum(axis=3))
    assert not acc5[..., 1].any()
    assert oracle.rel_l2(y5, y3) < 1e-13


def gen5(rng, n, k, p=(0.1, 0.1, 0.6, 0.1, 0.1)):
    lv = rng.choice([-2, -1, 0, 1, 2], size=(n, k), p=p).astype(np.int8)
    lo = rng.uniform(0.01, 0.05, (n, k // 256)).astype(np.float32)
    hi = (lo * rng.uniform(1.5, 3.0, lo.shape)).astype(np.float32)
    return lv, lo, hi


@pytest.mark.parametrize("name", ["ex1", "ex2"])
def test_golden_bytes(name):
    e = _read_golden()[name]
    lv, lo, hi, _ = golden_inputs(e)
    p = fv5.pack(lv, lo, hi)
    assert p.size == e["total"] == fv5.packed_bytes(e["N"], e["K"])
    for off, val in e["bytes"].items():
        assert p[off] == val, (off, p[off], val)
    rest = p.copy()
    rest[list(e["bytes"])] = 0
    assert not rest.any(), np.nonzero(rest)


@pytest.mark.parametrize("name", ["ex1", "ex2"])
def test_golden_gemv(name):
    e = _read_golden()[name]
    lv, lo, hi, x = golden_inputs(e)
    y64, _ = fv5.gemv_bf16(fv5.pack(lv, lo, hi), e["N"], e["K"], x)
    want = np.zeros(e["N"])
    for r, v in e["y"].items():
        want[r] = v
    assert np.array_equal(y64[0], want)


def test_round_trip_and_rows():
    rng = np.random.default_rng(1)
    n, k = 37, 1536
    lv, lo, hi = gen5(rng, n, k)
    p = fv5.pack(lv, lo, hi)
    l2, lo2, hi2 = fv5.unpack(p, n, k)
    assert np.array_equal(l2, lv) and np.array_equal(lo2, lo) and np.array_equal(hi2, hi)
    rows = [0, 15, 16, 36]
    lr, lor, hir = fv5._unpack_rows(p, n, k, rows)
    assert np.array_equal(lr, lv[rows]) and np.array_equal(lor, lo[rows]) and np.array_equal(hir, hi[rows])
    assert fv5.packed_bytes(n, k) == (48 * 1536 * 3 // 8 + 255) // 256 * 256 + 48 * 6 * 8
    assert fv5.packed_bytes(16, 768) == -1


def test_gemv_vs_brute_force():
    rng = np.random.default_rng(2)
    n, k, m = 5, 512, 2
    lv, lo, hi = gen5(rng, n, k)
    x = synth.gen_x_bf16(rng, m, k)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    want = np.zeros((m, n))
    for mm in range(m):
        for nn in range(n):
            acc = 0.0
            for kk in range(k):
                lvl = int(lv[nn, kk])
                if lvl == 0:
                    continue
                scale = float(hi[nn, kk // 256]) if abs(lvl) == 2 else float(lo[nn, kk // 256])
                acc += (scale if lvl > 0 else -scale) * xf[mm, kk]
            want[mm, nn] = acc
    y64, _ = fv5.gemv_bf16(fv5.pack(lv, lo, hi), n, k, x)
    assert np.allclose(y64, want, rtol=1e-13, atol=1e-13)


def test_reduces_to_the_ternary_format():
    """Levels in {-1, 0, +1}: the weights are t * s_lo, which the ternary
    format holds with its fp16 scale per 128 weights set to s_lo of the
    enclosing 256 (s_lo chosen fp16-representable); both oracles agree."""
    rng = np.random.default_rng(3)
    n, k = 40, 1024
    t = synth.gen_ternary(rng, n, k)
    s16 = synth.gen_scales(rng, n, k // 256)                       # fp16 bits
    lo = s16.view(np.float16).astype(np.float32)
    hi = rng.uniform(0.1, 0.2, lo.shape).astype(np.float32)        # unused by levels +-1
    s128 = np.repeat(s16, 2, axis=1)
    x = synth.gen_x_bf16(rng, 3, k)
    y5, _ = fv5.gemv_bf16(fv5.pack(t, lo, hi), n, k, x)
    y3, _ = oracle.gemv_bf16(oracle.pack(t, s128), n, k, x)
    assert oracle.rel_l2(y5, y3) < 1e-14


def test_invariants():
    rng = np.random.default_rng(4)
    n, k = 20, 512
    lv, lo, hi = gen5(rng, n, k)
    x = synth.gen_x_bf16(rng, 2, k)
    y, _ = fv5.gemv_bf16(fv5.pack(lv, lo, hi), n, k, x)
    yneg, _ = fv5.gemv_bf16(fv5.pack(-lv, lo, hi), n, k, x)
    assert np.array_equal(yneg, -y)
    z, _ = fv5.gemv_bf16(fv5.pack(np.zeros_like(lv), lo, hi), n, k, x)
    assert not z.any()
    # s_hi = s_lo: levels +-2 act as +-1
    same, _ = fv5.gemv_bf16(fv5.pack(lv, lo, lo), n, k, x)
    ones, _ = fv5.gemv_bf16(fv5.pack(np.sign(lv).astype(np.int8), lo, lo), n, k, x)
    assert np.array_equal(same, ones)
