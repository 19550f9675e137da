"""NumPy brute-force references — TEST INFRASTRUCTURE ONLY.

These never look at packed bytes: they take the dense ternary matrix and the
block scales and form the dequantized matrix W[n,k] = t[n,k] * scale[n, k//128]
(block-wise scaling, origotech.dev low-bit essay, section "어떻게 작동하나"),
then use a plain fp64 matrix product for y = x W^T (the linear-layer equation
of the discuss.pytorch.kr page, section "학습 중에 포맷이 있어야 하는 이유").
They pin the C oracle, which reads the packed bytes, on small inputs.
"""
from __future__ import annotations

import numpy as np


def f16_bits_to_f64(s):
    return np.asarray(s, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(t, scale):
    t = np.asarray(t, dtype=np.float64)
    s = f16_bits_to_f64(scale)
    return t * np.repeat(s, 128, axis=1)


def gemv_bf16(t, scale, x_bf16):
    """y[m, n] = sum_k W[n,k] x[m,k] with the dequantized W, in fp64."""
    return bf16_bits_to_f64(x_bf16) @ dequant(t, scale).T


def block_acc_i8(t, q):
    """acc[m, n, b] = sum_{k in block b} t[n,k] q[m,k] as exact integers."""
    n, k = t.shape
    m = q.shape[0]
    tb = np.asarray(t, dtype=np.int64).reshape(n, k // 128, 128)
    qb = np.asarray(q, dtype=np.int64).reshape(m, k // 128, 128)
    return np.einsum("nbk,mbk->mnb", tb, qb)


def tern_i8(t, scale, q, s_x):
    acc = block_acc_i8(t, q)
    y = np.asarray(s_x, dtype=np.float64)[:, None] * np.einsum("mnb,nb->mn", acc.astype(np.float64),
                                                                f16_bits_to_f64(scale))
    return acc, y


def head_bf16(w8, rs, x_bf16):
    return (bf16_bits_to_f64(x_bf16) @ np.asarray(w8, dtype=np.float64).T) * np.asarray(rs, np.float64)[None, :]
