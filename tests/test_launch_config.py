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


@pytest.mark.parametrize("kind", [k for k in tw.GEMV_KINDS if "phased" not in k])
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
        assert 1 <= c["U"] <= 4 and c["XC"] in (1, 2, 4, 8, 16), where
        if c["XC"] == 16:
            # 16 chunks: bf16 rows above 8, in one resident round, at most three units per wave
            assert not i8 and m > 8 and not c["rounds"] and c["U"] <= 3, where
        assert 64 * c["waves"] <= 1024, where
        assert c["waves"] * c["U"] >= units > (c["waves"] - 1) * c["U"], where   # every unit owned, no idle wave
        assert c["grid"] == (nrt + c["R"] - 1) // c["R"], where
        assert c["lds"] <= CU_LDS, where
        ni = 1 if m == 1 else (2 if m == 2 else 4)
        if kind == "ternary_bf16" and m == 1:
            # each wave stages the 1 KB activation slice of each of its units
            assert c["XC"] == 1 and c["lds"] == c["waves"] * c["U"] * 1024 + (units + 1) * 64 * 4, where
        elif kind == "ternary_bf16" and m <= 8 and c["R"] == 1 and c["U"] <= 2:
            # each wave stages its units' slices: 2, 4 or 8 rows of 1040 bytes
            mr = 2 if m <= 2 else (4 if m <= 4 else 8)
            assert c["XC"] == 1, where
            assert c["lds"] == c["waves"] * c["U"] * mr * 1040 + (units + 1) * ni * 64 * 4, where
        else:
            xrow = k + 16 if i8 else (k + 8) * 2
            side = m * xrow + (units + 1) * ni * 64 * 4
            if c["lds"] != side:
                # bf16 rows above 8 with no side-by-side split in one round: the partials
                # overwrite x after the compute (x plus its dummy slot, or the partials)
                assert kind in ("ternary_bf16", "fv5_bf16") and m > 8 and not c["rounds"], where
                assert c["lds"] == max(m * xrow + 16, (units + 1) * ni * 64 * 4), where
                assert 2 <= c["U"] and c["XC"] in (8, 16), where
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
    row tile per workgroup (two for bf16 when one tile's waves would each stage
    more than 8 chunks), nkt / 2 waves per row tile with two units each (unit i
    in half i of K), half of the activations staged at a time."""
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
        R = c["R"]
        assert R in (1, 2) and c["U"] == 2 and c["waves"] * 2 == R * nkt and c["waves"] <= 16, where
        assert c["grid"] == ((n + 15) // 16 + R - 1) // R and c["MT"] == 16, where
        pk = nkt // 2 * 512
        xrow = pk + 16 if i8 else (pk + 8) * 2
        slots = R * nkt + 1 if kind.startswith("ternary") else R * nkt   # partials (+ a spare in the ternary kernel)
        assert c["lds"] == m * xrow + slots * 4 * 64 * 4 + 32 <= CU_LDS, where   # + a dummy staging slot
        chunk = 32 if i8 else 16
        assert c["XC"] * 64 * c["waves"] * chunk >= m * pk * (1 if i8 else 2), where   # a half fully staged
        assert c["XC"] <= (4 if i8 else 8), where
        if R == 2:   # only where one row tile's waves would stage more than 8 chunks each
            assert not i8 and m * pk * 2 > 8 * 64 * (nkt // 2) * 16, where
    assert taken > 0
    # the shapes it exists for: down (4096 x 12288) at bf16 M = 7 and 8 and, five-level, int8 M = 16
    fam = kind.split("_")[0]
    for m in (7, 8):
        c = tw.tern_gemv_config(4096, 12288, m, fam + "_bf16_phased")
        assert c is not None and c["waves"] == 12 and c["XC"] == 8   # M chunks per thread, rounded up to 8
    if fam == "fv5":
        c = tw.tern_gemv_config(4096, 12288, 16, "fv5_int8_phased")
        assert c is not None and c["waves"] == 12 and c["XC"] == 4
    # the 8B fused gate|up (24576 x 4096) at bf16 M = 15 and 16: the one-pass split with the partials
    # over x (six row tiles per workgroup, one round); two row tiles per workgroup in the two-phase
    # kernel where x exceeds LDS: the five-level format at K = 8192, M = 10..15, the ternary one only
    # where x does not fit the persistent fast path either (K = 8192 at M = 9..15)
    if fam == "fv5":
        for m in (15, 16):
            assert tw.tern_gemv_config(24576, 4096, m, "fv5_bf16_phased") is None
            c = tw.tern_gemv_config(24576, 4096, m, "fv5_bf16")
            assert c is not None and (c["R"], c["waves"], c["U"], c["XC"], c["grid"]) == (6, 16, 3, 8, 256), (m, c)
            assert c["lds"] == max(m * (4096 + 8) * 2 + 16, 49 * 4 * 64 * 4), (m, c)
        for m in (10, 12):
            assert tw.tern_gemv_config(4000, 8192, m, "fv5_bf16") is None
            c = tw.tern_gemv_config(4000, 8192, m, "fv5_bf16_phased")
            assert c is not None and (c["R"], c["waves"], c["XC"], c["grid"]) == (2, 16, 8, 125), (m, c)
    else:
        assert tw.tern_gemv_config(24576, 4096, 16, "ternary_bf16_phased") is None
        for m in (9, 15):
            assert tw.tern_gemv_config(4096, 8192, m) is None
            c = tw.tern_gemv_config(4096, 8192, m, "ternary_bf16_phased")
            assert c is not None and (c["R"], c["waves"], c["XC"], c["grid"]) == (2, 16, 8, 128), (m, c)
        assert tw.tern_gemv_config(4096, 8192, 16, "ternary_bf16_phased") is None   # half of x: 131 KB


def test_phased3_picker_invariants():
    """The three-phase configuration (bf16): taken only where neither the
    one-pass nor the two-phase one fits; one row tile per workgroup, nkt / 3
    waves with three units each, a third of the activations staged at a
    time; the 8B down shape at M = 9..16 takes it."""
    taken = 0
    for n, k, m in itertools.product(NS, KS, MS):
        c = tw.tern_gemv_config(n, k, m, "ternary_bf16_phased3")
        if c is None:
            continue
        taken += 1
        where = (n, k, m, c)
        assert tw.tern_gemv_config(n, k, m) is None and tw.tern_gemv_config(n, k, m, "ternary_bf16_phased") is None
        nkt = k // 512
        assert c["R"] == 1 and c["U"] == 3 and c["waves"] * 3 == nkt and c["waves"] <= 8, where
        assert c["grid"] == (n + 15) // 16 and c["MT"] == 16, where
        pk = c["waves"] * 512
        assert c["lds"] == m * (pk + 8) * 2 + nkt * 4 * 64 * 4 + 16 <= CU_LDS, where   # + a dummy staging slot
        assert c["XC"] * 64 * c["waves"] * 16 >= m * pk * 2 and c["XC"] in (4, 8, 16), where   # a third staged
    assert taken > 0
    for m in range(9, 17):
        c = tw.tern_gemv_config(4096, 12288, m, "ternary_bf16_phased3")
        assert c is not None and c["waves"] == 8 and c["XC"] == 16, (m, c)
    for m in range(1, 9):
        assert tw.tern_gemv_config(4096, 12288, m, "ternary_bf16_phased3") is None, m


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
    assert L.tern_gemv_config(16, 512, 1, 9, out) == -2
    assert L.tern_gemv_config(0, 512, 1, 0, out) == -2


def test_prefill_tile_and_split_on_the_8b_shapes():
    """The workgroup-shared-decode prefill's tile and K split on the 8B gate / down shapes
    (a 256-CU device): the 256 x 128 tile where its tiles fill whole rounds, the 128 x 64
    tile elsewhere, and K split in two halves only where the doubled grid still fits one
    workgroup per CU (the measured choices)."""
    big, small = (256, 128), (128, 64)
    want = {(12288, 4096, 512): (small, 0), (12288, 4096, 1024): (small, 0), (12288, 4096, 1536): (small, 0),
            (12288, 4096, 2048): (big, 0), (12288, 4096, 4096): (big, 0),
            (4096, 12288, 128): (small, 1), (4096, 12288, 256): (small, 1), (4096, 12288, 512): (small, 0),
            (4096, 12288, 1024): (small, 0), (4096, 12288, 3072): (small, 0), (4096, 12288, 2048): (big, 0),
            (4096, 12288, 4096): (big, 0)}
    for (n, k, m), (tile, split) in want.items():
        c = tw.tern_prefill_config(n, k, m)
        assert (c["BM"], c["BN"]) == tile and c["split"] == split, (n, k, m, c)


@pytest.mark.parametrize("m", [128, 129, 200, 255, 256, 300, 511, 512, 777, 1024, 1100, 2048, 3000, 4096])
def test_prefill_config_invariants(m):
    """Over N and K: the grid covers M x N with the chosen tile, z = 2 exactly when K is
    split, a split keeps at least 4 of 512-k tiles per half and at most one workgroup per
    CU, and the shapes the kernel does not take (M < 128, K % 512 != 0) return None."""
    for n, k in itertools.product([1, 16, 17, 300, 1000, 4096, 12288, 24576], [512, 1024, 3584, 4096, 4608, 12288]):
        c = tw.tern_prefill_config(n, k, m)
        assert c is not None
        assert c["grid_x"] * c["BN"] >= n > (c["grid_x"] - 1) * c["BN"]
        assert c["grid_y"] * c["BM"] >= m > (c["grid_y"] - 1) * c["BM"]
        assert c["grid_z"] == (2 if c["split"] else 1)
        if c["split"]:
            assert k // 512 >= 8 and 2 * c["grid_x"] * c["grid_y"] <= 256
        else:
            assert k // 512 < 8 or 2 * c["grid_x"] * c["grid_y"] > 256
    assert tw.tern_prefill_config(4096, 4096, 64) is None
    assert tw.tern_prefill_config(4096, 4096 + 128, m) is None


def test_prefill_config_below_128():
    """65 <= M < 128: the shared-decode kernel only where the measured model puts it
    ahead of the per-block kernel and the GEMV slices (8B down at M >= 96 with K split;
    8B gate and down at M = 65 / 80 keep their paths); never at M <= 64."""
    for m in (96, 112, 127):
        c = tw.tern_prefill_config(4096, 12288, m)
        assert c is not None and (c["BM"], c["split"], c["grid_z"]) == (128, 1, 2), (m, c)
    for m in (65, 80):
        assert tw.tern_prefill_config(4096, 12288, m) is None
    for m in (65, 96, 127):
        assert tw.tern_prefill_config(12288, 4096, m) is None
    for m in (1, 16, 17, 64):
        assert tw.tern_prefill_config(4096, 12288, m) is None


def test_prefill_config_argument_errors():
    L = tw.lib()
    import ctypes
    out = (ctypes.c_int64 * 6)()
    assert L.tern_prefill_config(16, 512, 128, None) == -1
    assert L.tern_prefill_config(0, 512, 128, out) == -2
    assert L.tern_prefill_config(16, 0, 128, out) == -2
    assert L.tern_prefill_config(16, 96, 128, out) == -2
    assert L.tern_prefill_config(16, 512, 0, out) == -2
