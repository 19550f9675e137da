"""FV5B-style int8 tensors (output head and token embedding): CPU oracle —
TEST INFRASTRUCTURE ONLY.

Plain NumPy, fp64 arithmetic; it shares no code with the HIP library.  Only
the tests, the package's smoke check and the benchmark's CPU-baseline leg
may use it.

What it follows: the FV5B row of the block-format table on the
discuss.pytorch.kr page ("Fermion Research, 3진 계열 포맷으로 직접 학습한
Neutrino-1 모델군 3종 공개", section "FV5와 FV5B: llama.cpp 포크가 공개한
블록 구조"): blocks of 256 int8 weights with one f32 scale (8.125 bits per
weight), used for the token embedding and the output head; the same page
(section "3진 계열이라는 이름의 실체") keeps embedding and head in int8.
Storage here is W int8 [V][K] row-major and S f32 [V][K/256]; the weight is
W[v][k] * S[v][k/256].

Functions:
  head_bf16     logits[m][v] = sum_b S[v][b] * sum_{k in b} W[v][k] x[m][k]
  head_i8       acc[m][v][b] = sum_{k in b} W[v][k] q[m][k] (exact integers),
                logits[m][v] = s_x[m] * sum_b S[v][b] * acc[m][v][b]
  embed_f32     out[m][k] = W[id][k] * S[id][k/256] rounded once to fp32;
                a row of zeros when id is outside [0, V)
  round_bf16    fp32 -> bf16 bits, nearest with ties to even
  embed_bf16    round_bf16(embed_f32(...))
"""
from __future__ import annotations

import numpy as np


def _x64(x_bf16):
    return (np.asarray(x_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _blocks(k: int) -> int:
    assert k % 256 == 0
    return k // 256


def _row_chunks(v, rows, chunk=8192):
    r = np.arange(v) if rows is None else np.asarray(rows)
    return [r[i:i + chunk] for i in range(0, len(r), chunk)] or [r]


def head_bf16(w8, s, x_bf16, rows=None):
    """fp64 logits [M][rows] of the block-scaled int8 head for bf16 x; returns
    (y64, y32).  Rows are independent; they are taken in chunks to bound
    memory."""
    w8 = np.asarray(w8, dtype=np.int8)
    s = np.asarray(s, dtype=np.float32)
    v, k = w8.shape
    _blocks(k)
    x = _x64(x_bf16)
    parts = []
    for r in _row_chunks(v, rows):
        wd = w8[r].astype(np.float64) * np.repeat(s[r].astype(np.float64), 256, axis=1)
        parts.append(x @ wd.T)
    y64 = np.concatenate(parts, axis=1)
    return y64, y64.astype(np.float32)


def head_acc_i8(w8, q, rows=None):
    """Exact block sums acc[m][v][b] = sum_{k in block b} W[v][k] q[m][k] (int64)."""
    w8 = np.asarray(w8, dtype=np.int8)
    v, k = w8.shape
    nb = _blocks(k)
    qb = np.asarray(q, dtype=np.int8).astype(np.int64).reshape(-1, nb, 256)
    parts = []
    for r in _row_chunks(v, rows):
        wb = w8[r].astype(np.int64).reshape(len(r), nb, 256)
        parts.append(np.einsum("mbk,vbk->mvb", qb, wb))
    return np.concatenate(parts, axis=1)


def head_i8(w8, s, q, s_x, rows=None):
    """int8 activations: (acc int64 [M][rows][K/256], y64, y32)."""
    acc = head_acc_i8(w8, q, rows)
    v = np.asarray(w8).shape[0]
    r = np.arange(v) if rows is None else np.asarray(rows)
    sb = np.asarray(s, dtype=np.float32)[r].astype(np.float64)              # [rows][nb]
    y64 = np.asarray(s_x, dtype=np.float32).astype(np.float64)[:, None] * np.einsum("mvb,vb->mv", acc, sb)
    return acc, y64, y64.astype(np.float32)


def embed_f32(w8, s, ids):
    """Rows of the dequantized table for token ids: the exact product (int8 x
    f32 fits fp64) rounded once to fp32; ids outside [0, V) give zero rows."""
    w8 = np.asarray(w8, dtype=np.int8)
    v, k = w8.shape
    nb = _blocks(k)
    s = np.asarray(s, dtype=np.float32).reshape(v, nb)
    ids = np.asarray(ids, dtype=np.int64)
    out = np.zeros((ids.size, k), dtype=np.float32)
    for m, t in enumerate(ids):
        if 0 <= t < v:
            exact = w8[t].astype(np.float64) * np.repeat(s[t].astype(np.float64), 256)
            out[m] = exact.astype(np.float32)
    return out


def round_bf16(f32):
    """fp32 values -> bf16 bit patterns, nearest with ties to the even pattern:
    the two bf16 neighbours of f (truncation of its bits, and the next pattern
    away from zero) are compared by distance in fp64.  Finite inputs only."""
    f = np.ascontiguousarray(f32, dtype=np.float32)
    assert np.isfinite(f).all()
    bits = f.view(np.uint32)
    lo = (bits >> 16).astype(np.uint32)                       # toward zero
    hi = lo + 1                                               # away from zero
    as_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = f.astype(np.float64)
    d_lo, d_hi = np.abs(x - as_f(lo)), np.abs(as_f(hi) - x)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def embed_bf16(w8, s, ids):
    return round_bf16(embed_f32(w8, s, ids))
