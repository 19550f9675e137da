"""Five-level (FV5-style) weights: CPU oracle — TEST INFRASTRUCTURE ONLY.

Plain NumPy, fp64 arithmetic, written from the layout definition below; it
shares no code with the HIP library (or with the ternary oracle).  Only the
tests, the package's smoke check and the benchmark's CPU-baseline leg may
use it.

What it follows: the FV5 row of the block-format table on the
discuss.pytorch.kr page ("Fermion Research, 3진 계열 포맷으로 직접 학습한
Neutrino-1 모델군 3종 공개", section "FV5와 FV5B: llama.cpp 포크가 공개한
블록 구조"): 256-weight blocks of 104 bytes holding two f32 scales (s_lo,
s_hi) and three 32-byte bit-planes, read there as sign, zero and two
magnitude steps, i.e. five levels at 3.25 bits per weight.  The bit-level
encoding is not published; the one below is this project's own.

Definition.  Levels l[n][k] in {-2, -1, 0, +1, +2}; block (n, b) covers
k in [256b, 256b+256) and has f32 scales s_lo[n][b], s_hi[n][b]; the weight
is  w = sign(l) * (s_hi if |l| == 2 else s_lo)  (0 when l == 0).
Packed layout (K % 512 == 0; rows padded to Np = ceil(N/16)*16 with zero
planes and zero scales):
  * three planes per block, p = 0 nonzero (l != 0), p = 1 sign (l < 0),
    p = 2 high (|l| == 2); each 256 bits = eight little-endian 32-bit words;
    word w holds weights k = 256b + 32w + i (i = 0..31), weight i at bit
    16*(i & 1) + (i >> 1).  Canonical form: sign = high = 0 where nonzero = 0.
  * row tile rt = n/16, r = n%16; k-tile kt = b/2 (512 k), bh = b%2;
    nkt = K/512; word w of block bh sits in group g = w%4 at slot
    j = 2*bh + w//4:
        word_index = ((rt*nkt + kt)*3 + p)*256 + (g*16 + r)*4 + j
    byte offset = 4*word_index (3072 bytes of planes per row tile and k-tile).
  * scales are f32 from byte align256(Np*K*3/8): s_lo of (n, b) at element
    ((rt*nkt + kt)*16 + r)*4 + 2*bh, s_hi at the next element.
  * total bytes = align256(Np*K*3/8) + Np*(K/256)*8.
"""
from __future__ import annotations

import numpy as np


def _npad(n: int) -> int:
    return (n + 15) // 16 * 16


def _align256(v: int) -> int:
    return (v + 255) // 256 * 256


def packed_bytes(n: int, k: int) -> int:
    if n < 0 or k < 0 or k % 512:
        return -1
    return _align256(_npad(n) * k * 3 // 8) + _npad(n) * (k // 256) * 8


def _bit_of(i):
    """Bit position of weight i (0..31) inside its word."""
    return 16 * (i & 1) + (i >> 1)


def pack(levels, s_lo, s_hi) -> np.ndarray:
    """levels int8 [N][K] in {-2..2}; s_lo, s_hi f32 [N][K/256] -> packed bytes."""
    levels = np.asarray(levels, dtype=np.int8)
    n, k = levels.shape
    assert k % 512 == 0 and np.all(np.abs(levels.astype(np.int32)) <= 2)
    s_lo = np.asarray(s_lo, dtype=np.float32).reshape(n, k // 256)
    s_hi = np.asarray(s_hi, dtype=np.float32).reshape(n, k // 256)
    nkt = k // 512
    total = packed_bytes(n, k)
    words = np.zeros((_align256(_npad(n) * k * 3 // 8)) // 4, dtype=np.uint32)
    planes = [levels != 0, levels < 0, np.abs(levels.astype(np.int32)) == 2]
    for row in range(n):
        rt, r = divmod(row, 16)
        for kk in range(k):
            b, off = divmod(kk, 256)
            kt, bh = divmod(b, 2)
            w, i = divmod(off, 32)
            g, hw = w % 4, w // 4
            for p in range(3):
                if planes[p][row, kk]:
                    idx = ((rt * nkt + kt) * 3 + p) * 256 + (g * 16 + r) * 4 + (2 * bh + hw)
                    words[idx] |= np.uint32(1) << np.uint32(_bit_of(i))
    out = np.zeros(total, dtype=np.uint8)
    out[: words.size * 4] = words.view(np.uint8)
    sc = np.zeros(_npad(n) * (k // 256) * 2, dtype=np.float32)
    for row in range(n):
        rt, r = divmod(row, 16)
        for b in range(k // 256):
            kt, bh = divmod(b, 2)
            e = ((rt * nkt + kt) * 16 + r) * 4 + 2 * bh
            sc[e] = s_lo[row, b]
            sc[e + 1] = s_hi[row, b]
    base = words.size * 4
    out[base:base + sc.size * 4] = sc.view(np.uint8)
    return out


def unpack(packed, n: int, k: int):
    """packed bytes -> (levels int8 [N][K], s_lo f32 [N][K/256], s_hi f32 [N][K/256])."""
    packed = np.asarray(packed, dtype=np.uint8)
    assert packed.size == packed_bytes(n, k)
    nkt = k // 512
    base = _align256(_npad(n) * k * 3 // 8)
    words = packed[:base].view(np.uint32)
    sc = packed[base:].view(np.float32)
    levels = np.zeros((n, k), dtype=np.int8)
    s_lo = np.zeros((n, k // 256), dtype=np.float32)
    s_hi = np.zeros((n, k // 256), dtype=np.float32)
    for row in range(n):
        rt, r = divmod(row, 16)
        for kk in range(k):
            b, off = divmod(kk, 256)
            kt, bh = divmod(b, 2)
            w, i = divmod(off, 32)
            g, hw = w % 4, w // 4
            bits = []
            for p in range(3):
                idx = ((rt * nkt + kt) * 3 + p) * 256 + (g * 16 + r) * 4 + (2 * bh + hw)
                bits.append((int(words[idx]) >> _bit_of(i)) & 1)
            nz, neg, high = bits
            levels[row, kk] = 0 if not nz else (-1 if neg else 1) * (2 if high else 1)
        for b in range(k // 256):
            kt, bh = divmod(b, 2)
            e = ((rt * nkt + kt) * 16 + r) * 4 + 2 * bh
            s_lo[row, b] = sc[e]
            s_hi[row, b] = sc[e + 1]
    return levels, s_lo, s_hi


def dense(levels, s_lo, s_hi) -> np.ndarray:
    """The weight matrix in fp64: w = sign(l) * (s_hi if |l| == 2 else s_lo)."""
    levels = np.asarray(levels, dtype=np.int32)
    n, k = levels.shape
    lo = np.repeat(np.asarray(s_lo, np.float64), 256, axis=1)
    hi = np.repeat(np.asarray(s_hi, np.float64), 256, axis=1)
    mag = np.where(np.abs(levels) == 2, hi, lo)
    return np.sign(levels) * mag * (levels != 0)


def gemv_bf16_levels(levels, s_lo, s_hi, x_bf16):
    """y[m][n] = sum_k w[n][k] * x[m][k] in fp64 from unpacked levels and
    scales, x given as bf16 bits.  Returns (y64, y32)."""
    x = (np.asarray(x_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y64 = x @ dense(levels, s_lo, s_hi).T
    return y64, y64.astype(np.float32)


def gemv_bf16(packed, n: int, k: int, x_bf16, rows=None):
    """The same product read from a packed blob; rows (optional) selects
    output rows.  Returns (y64, y32)."""
    levels, s_lo, s_hi = unpack(packed, n, k) if rows is None else _unpack_rows(packed, n, k, rows)
    return gemv_bf16_levels(levels, s_lo, s_hi, x_bf16)


def acc_i8_levels(levels, q):
    """Exact block sums for int8 activations q [M][K]: acc[m][n][b][0] =
    sum over block b of sign(l)*q where |l| = 1, acc[m][n][b][1] the same
    where |l| = 2 (int64)."""
    levels = np.asarray(levels, dtype=np.int64)
    n, k = levels.shape
    nb = k // 256
    qb = np.asarray(q, dtype=np.int8).astype(np.int64).reshape(-1, nb, 256)
    sign = np.sign(levels).reshape(n, nb, 256)
    mag = np.abs(levels).reshape(n, nb, 256)
    lo = np.einsum("mbk,nbk->mnb", qb, sign * (mag == 1))
    hi = np.einsum("mbk,nbk->mnb", qb, sign * (mag == 2))
    return np.stack([lo, hi], axis=3)


def gemv_i8_levels(levels, s_lo, s_hi, q, s_x):
    """int8 activations q with row scales s_x: y[m][n] = s_x[m] * sum_b
    (s_lo[n][b] * acc_lo + s_hi[n][b] * acc_hi) in fp64.  Returns
    (acc int64 [M][N][K/256][2], y64, y32)."""
    acc = acc_i8_levels(levels, q)
    lo = np.asarray(s_lo, np.float32).astype(np.float64)
    hi = np.asarray(s_hi, np.float32).astype(np.float64)
    tot = np.einsum("mnb,nb->mn", acc[..., 0], lo) + np.einsum("mnb,nb->mn", acc[..., 1], hi)
    y64 = np.asarray(s_x, np.float32).astype(np.float64)[:, None] * tot
    return acc, y64, y64.astype(np.float32)


def gemv_i8(packed, n: int, k: int, q, s_x, rows=None):
    """The int8-activation product read from a packed blob (rows optional)."""
    levels, s_lo, s_hi = unpack(packed, n, k) if rows is None else _unpack_rows(packed, n, k, rows)
    return gemv_i8_levels(levels, s_lo, s_hi, q, s_x)


def _unpack_rows(packed, n, k, rows):
    """unpack restricted to the given rows (same bit-level reading)."""
    levels, s_lo, s_hi = [], [], []
    nkt = k // 512
    base = _align256(_npad(n) * k * 3 // 8)
    words = np.asarray(packed, np.uint8)[:base].view(np.uint32)
    sc = np.asarray(packed, np.uint8)[base:].view(np.float32)
    kk = np.arange(k)
    b, off = kk // 256, kk % 256
    kt, bh = b // 2, b % 2
    w, i = off // 32, off % 32
    g, hw = w % 4, w // 4
    bit = 16 * (i & 1) + (i >> 1)
    for row in rows:
        rt, r = divmod(int(row), 16)
        bits = []
        for p in range(3):
            idx = ((rt * nkt + kt) * 3 + p) * 256 + (g * 16 + r) * 4 + (2 * bh + hw)
            bits.append((words[idx] >> bit.astype(np.uint32)) & 1)
        nz, neg, high = [x.astype(np.int32) for x in bits]
        levels.append((nz * (1 - 2 * neg) * (1 + high)).astype(np.int8))
        bb = np.arange(k // 256)
        e = ((rt * nkt + bb // 2) * 16 + r) * 4 + 2 * (bb % 2)
        s_lo.append(sc[e])
        s_hi.append(sc[e + 1])
    return np.array(levels), np.array(s_lo), np.array(s_hi)
