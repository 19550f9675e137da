"""Packed copy of the int8 output head: CPU oracle — TEST INFRASTRUCTURE ONLY.

Plain NumPy, integer byte moves only; it shares no code with the HIP
library.  Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may use it.

Why the copy exists: the output head (int8 [V][K] with one fp32 scale per
row, kept in int8 by the discuss.pytorch.kr page "Fermion Research, 3진 계열
포맷으로 직접 학습한 Neutrino-1 모델군 3종 공개", section "3진 계열이라는
이름의 실체") is the largest tensor of a decode step and its GEMV runs on the
DRAM roofline (the same page, section "뉴트리노 엔진: 토큰 하나의 시간은
어디로 가는가").  The pages fix the values, not a storage order; the order
below is this library's own.  The logits over the copy are those of the
row-major head (oracle.head_bf16 / oracle.head_i8), so the oracle needs only
the byte permutation.

Layout (a definition, written out from its statement):
  rows are taken in groups of 64 (V padded to a multiple of 64 with zero
  rows); group G occupies bytes [64*K*G, 64*K*(G+1)).  Within a group, for
  each 128-byte column unit j (K/128 of them), 8192 bytes; within those, for
  each 16-row tile w (0..3), 2048 bytes; within those, half h (0, 1) at
  1024*h, and in a half, 16 bytes per lane l (0..63) at 16*l.  Lane
  l = r + 16*g (r < 16, g < 4) of tile w, half h, unit j holds
      W[64*G + 16*w + r][128*j + 64*h + 16*g .. 128*j + 64*h + 16*g + 15].

Functions:
  packed_bytes(V, K)    ceil(V/64) * 64 * K
  pack(W)               int8 [V][K] -> int8 [packed_bytes(V, K)]
  unpack(P, V, K)       the inverse on the first V rows
"""
from __future__ import annotations

import numpy as np


def packed_bytes(v: int, k: int) -> int:
    assert v >= 1 and k >= 128 and k % 128 == 0
    return (v + 63) // 64 * 64 * k


def _axes(v: int, k: int):
    """W padded to whole groups, viewed with one axis per term of the row and
    column: row = 64*G + 16*w + r, col = 128*j + 64*h + 16*g + b."""
    groups = (v + 63) // 64
    return groups, (groups, 4, 16, k // 128, 2, 4, 16)   # G, w, r, j, h, g, b


def pack(w8) -> np.ndarray:
    w8 = np.asarray(w8, dtype=np.int8)
    v, k = w8.shape
    groups, shape = _axes(v, k)
    padded = np.zeros((groups * 64, k), dtype=np.int8)
    padded[:v] = w8
    a = padded.reshape(shape)                      # [G][w][r][j][h][g][b]
    # storage order G, j, w, h, then lane l = r + 16*g (g outer, r inner), then the 16 bytes b
    out = a.transpose(0, 3, 1, 4, 5, 2, 6)         # [G][j][w][h][g][r][b]
    return np.ascontiguousarray(out).reshape(-1)


def unpack(p, v: int, k: int) -> np.ndarray:
    p = np.asarray(p, dtype=np.int8)
    groups, shape = _axes(v, k)
    assert p.size == groups * 64 * k
    a = p.reshape(groups, k // 128, 4, 2, 4, 16, 16)   # [G][j][w][h][g][r][b]
    w = a.transpose(0, 2, 5, 1, 3, 4, 6)                # [G][w][r][j][h][g][b]
    return np.ascontiguousarray(w).reshape(groups * 64, k)[:v]
