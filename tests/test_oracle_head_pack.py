"""The packed copy of the int8 output head in oracle/head_pack.py against
positions derived by hand (tests/golden/head_pack_examples.txt), and its
inverse, on the CPU."""
import os

import numpy as np
import pytest

from oracle import head_pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "head_pack_examples.txt")


def read_golden():
    lines = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    hdr = lines[0]
    assert hdr[0] == "V" and hdr[2] == "K" and hdr[4] == "bytes"
    v, k, nbytes = int(hdr[1]), int(hdr[3]), int(hdr[5])
    return v, k, nbytes, lines[1:]


def test_golden_positions():
    v, k, nbytes, rows = read_golden()
    assert head_pack.packed_bytes(v, k) == nbytes
    w = np.random.default_rng(5).integers(-127, 128, size=(v, k)).astype(np.int8)
    w[w == 0] = 1                                   # no zero weights: a zero piece is padding only
    p = head_pack.pack(w)
    assert p.dtype == np.int8 and p.size == nbytes
    assert len(rows) >= 15
    for r in rows:
        off = int(r[0])
        if r[1] == "zero":
            assert not p[off:off + 16].any(), off
        else:
            row, col = int(r[1]), int(r[2])
            assert np.array_equal(p[off:off + 16], w[row, col:col + 16]), off


@pytest.mark.parametrize("v,k", [(1, 128), (64, 128), (65, 384), (70, 256), (200, 1024), (129, 4096)])
def test_round_trip_and_padding(v, k):
    rng = np.random.default_rng(v * 7 + k)
    w = rng.integers(-127, 128, size=(v, k)).astype(np.int8)
    w[w == 0] = -1
    p = head_pack.pack(w)
    assert p.size == -(-v // 64) * 64 * k
    assert np.array_equal(head_pack.unpack(p, v, k), w)
    # every nonzero byte is a weight, each weight appears once: the padding is the only zero
    assert np.count_nonzero(p) == v * k
    assert np.array_equal(np.sort(p[p != 0]), np.sort(w.reshape(-1)))


def test_lane_pieces_are_the_row_major_pieces():
    """A 16-row tile's 2 KiB of one unit hold, lane by lane, the 16-byte pieces
    a row-major reader gives lane (r, g): bytes 16g.. of row r in the low
    KiB and 64 + 16g.. in the high KiB."""
    v, k = 128, 512
    w = np.arange(v * k, dtype=np.int64).reshape(v, k)
    w8 = (w % 251 - 125).astype(np.int8)
    p = head_pack.pack(w8)
    grp, j, tile = 1, 3, 2
    base = grp * 64 * k + j * 8192 + tile * 2048
    for lane in range(64):
        r, g = lane % 16, lane // 16
        row = 64 * grp + 16 * tile + r
        lo = p[base + 16 * lane: base + 16 * lane + 16]
        hi = p[base + 1024 + 16 * lane: base + 1024 + 16 * lane + 16]
        assert np.array_equal(lo, w8[row, 128 * j + 16 * g: 128 * j + 16 * g + 16])
        assert np.array_equal(hi, w8[row, 128 * j + 64 + 16 * g: 128 * j + 64 + 16 * g + 16])
