"""Host logic of the one-pass GEMV launch picker (tern_gemv_config, no GPU):
over a grid of shapes, every configuration it returns must be launchable
and cover the problem: LDS within one CU, every unit of every row tile
owned by a wave, the activations fully staged, the grid covering all row
tiles, and one-round configurations resident on 256 CUs.  The 8B decode
shapes take the configurations the design measured."""
import itertools

import pytest

import ternary_weight_decode_amd as tw

CU_LDS = 160 * 1024
CUS = 256
WAVES_PER_SIMD = {"ternary_bf16": (0, 8, 7, 6, 5), "ternary_int8": (0, 8, 7, 6, 5),
                  "fv5_bf16": (0, 8, 6, 4, 4), "fv5_int8": (0, 7, 6, 5, 4)}

NS = [1, 16, 17, 1000, 4096, 6144, 24576, 65541, 196608]
KS = [512, 1024, 4096, 12288, 16384, 32768]
MS = [1, 2, 3, 4, 5, 8, 12, 16]


@pytest.mark.parametrize("kind", [k for k in tw.GEMV_KINDS if not k.endswith("phased")])
def test_picker_invariants(kind):
    i8 = kind.endswith("int8")
    taken = 0
    for n, k, m in itertools.product(NS, KS, MS):
        c = tw.tern_gemv_config(n, k, m, kind)
        if c is None:
            continue
        taken += 1
        nrt, nkt = (n + 15) // 16, k // 512
        units = c["R"] * nkt
        where = (kind, n, k, m, c)
        assert 1 <= c["U"] <= 4 and c["XC"] in (1, 2, 4, 8), where
        assert 64 * c["waves"] <= 1024, where
        assert c["waves"] * c["U"] >= units > (c["waves"] - 1) * c["U"], where   # every unit owned, no idle wave
        assert c["grid"] == (nrt + c["R"] - 1) // c["R"], where
        assert c["lds"] <= CU_LDS, where
        xrow = k + 16 if i8 else (k + 8) * 2
        ni = 1 if m == 1 else (2 if m == 2 else 4)
        assert c["lds"] == m * xrow + (units + 1) * ni * 64 * 4, where
        chunk = 32 if i8 else 16
        assert c["XC"] * 64 * c["waves"] * chunk >= m * k * (1 if i8 else 2), where       # x fully staged
        assert c["MT"] >= m and (c["XC"] < 8 or c["MT"] == 16), where
        if c["XC"] == 8:
            assert m > 2, where          # the MT = 16 partial area needs 4 rows per lane group
        if not c["rounds"]:
            per_cu = (c["grid"] + CUS - 1) // CUS
            assert per_cu * c["waves"] <= 4 * WAVES_PER_SIMD[kind][c["U"]], where
            assert per_cu * c["lds"] <= CU_LDS, where
    assert taken > 100


@pytest.mark.parametrize("kind", ["ternary_bf16_phased", "ternary_int8_phased", "fv5_bf16_phased",
                                  "fv5_int8_phased"])
def test_phased_picker_invariants(kind):
    """The two-phase configuration: taken only where no one-pass one fits; one
    row tile per workgroup, nkt / 2 waves with two units each (unit i in half
    i of K), half of the activations staged at a time."""
    i8 = "int8" in kind
    taken = 0
    for n, k, m in itertools.product(NS, KS, MS):
        c = tw.tern_gemv_config(n, k, m, kind)
        one = tw.tern_gemv_config(n, k, m, kind[:-len("_phased")])
        if c is None:
            continue
        taken += 1
        where = (kind, n, k, m, c)
        assert one is None, where
        nkt = k // 512
        assert c["R"] == 1 and c["U"] == 2 and c["waves"] * 2 == nkt and c["waves"] <= 16, where
        assert c["grid"] == (n + 15) // 16 and c["MT"] == 16, where
        pk = c["waves"] * 512
        xrow = pk + 16 if i8 else (pk + 8) * 2
        slots = nkt + 1 if kind.startswith("ternary") else nkt         # partials (+ a spare in the ternary kernel)
        assert c["lds"] == m * xrow + slots * 4 * 64 * 4 + 32 <= CU_LDS, where   # + a dummy staging slot
        chunk = 32 if i8 else 16
        assert c["XC"] * 64 * c["waves"] * chunk >= m * pk * (1 if i8 else 2), where   # a half fully staged
        assert c["XC"] <= (4 if i8 else 8), where
    assert taken > 0
    # the shapes it exists for: down (4096 x 12288) at bf16 M = 7 and 8 and, five-level, int8 M = 16
    fam = kind.split("_")[0]
    for m in (7, 8):
        c = tw.tern_gemv_config(4096, 12288, m, fam + "_bf16_phased")
        assert c is not None and c["waves"] == 12 and c["XC"] == 8   # M chunks per thread, rounded up to 8
    if fam == "fv5":
        c = tw.tern_gemv_config(4096, 12288, 16, "fv5_int8_phased")
        assert c is not None and c["waves"] == 12 and c["XC"] == 4


def test_picker_8b_decode_shapes():
    """The configurations measured for the fused 8B linears at M = 1."""
    want = {(6144, 4096): (2, 8, 2, 192), (4096, 4096): (1, 8, 1, 256), (24576, 4096): (2, 8, 2, 768),
            (4096, 12288): (1, 12, 2, 256)}
    for (n, k), (r, waves, u, grid) in want.items():
        c = tw.tern_gemv_config(n, k, 1)
        assert (c["R"], c["waves"], c["U"], c["grid"], c["rounds"]) == (r, waves, u, grid, 0), (n, k, c)


def test_picker_large_matrix_runs_in_rounds_and_large_x_falls_back():
    c = tw.tern_gemv_config(196608, 4096, 1)
    assert c["rounds"] == 1 and c["grid"] * c["R"] >= 196608 // 16
    # bf16 activations of 8 x 12288 (197 KB) do not fit a CU's LDS: another kernel
    assert tw.tern_gemv_config(4096, 12288, 8) is None
    # the same activations as int8 (98 KB) do
    assert tw.tern_gemv_config(4096, 12288, 8, "ternary_int8") is not None
    # K not a multiple of 512: the one-pass kernel does not apply
    assert tw.tern_gemv_config(4096, 640, 1) is None


def test_picker_argument_errors():
    L = tw.lib()
    import ctypes
    out = (ctypes.c_int64 * 8)()
    assert L.tern_gemv_config(16, 512, 1, 0, None) == -1
    assert L.tern_gemv_config(16, 512, 17, 0, out) == -2
    assert L.tern_gemv_config(16, 512, 1, 8, out) == -2
    assert L.tern_gemv_config(0, 512, 1, 0, out) == -2
