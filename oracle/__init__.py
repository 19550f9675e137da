"""CPU oracle for the ternary decode path — TEST INFRASTRUCTURE ONLY.

Plain fp64 C (``tern_oracle.c``) reached through ctypes, plus NumPy
brute-force references.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
never does.  It shares no code with the HIP library.

Every function states what it follows and the reading of the pages it takes
where they are silent.  Functions with no pin other
than their own definition say "parity unpinned" (none at present: each is
pinned by a worked example, a closed form, an invariant or brute force in
``tests/test_oracle.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "tern_oracle.c")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_packed_bytes.restype = _i64
        L.oracle_packed_bytes.argtypes = [_i64, _i64]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        for name, n in [("oracle_pack", 5), ("oracle_unpack", 5), ("oracle_stats", 4),
                        ("oracle_gemv_bf16", 9), ("oracle_quantize_i8", 5), ("oracle_tern_i8", 11),
                        ("oracle_head_bf16", 10), ("oracle_head_i8", 12)]:
            getattr(L, name).restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def packed_bytes(n: int, k: int) -> int:
    return int(lib().oracle_packed_bytes(_i64(n), _i64(k)))


def pack(t, scale) -> np.ndarray:
    """Layout definition: see the header of tern_oracle.c."""
    t = _c(t, np.int8)
    scale = _c(scale, np.uint16)
    n, k = t.shape
    assert scale.shape == (n, k // 128)
    out = np.empty(packed_bytes(n, k), dtype=np.uint8)
    rc = lib().oracle_pack(_ptr(t), _ptr(scale), _i64(n), _i64(k), _ptr(out))
    assert rc == 0, rc
    return out


def unpack(packed, n: int, k: int):
    packed = _c(packed, np.uint8)
    t = np.empty((n, k), dtype=np.int8)
    s = np.empty((n, k // 128), dtype=np.uint16)
    rc = lib().oracle_unpack(_ptr(packed), _i64(n), _i64(k), _ptr(t), _ptr(s))
    assert rc == 0, rc
    return t, s


def stats(packed, n: int, k: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    out = np.zeros(3, dtype=np.uint64)
    rc = lib().oracle_stats(_ptr(packed), _i64(n), _i64(k), _ptr(out))
    assert rc == 0, rc
    return out


def _rows(rows, n):
    if rows is None:
        return None, n
    r = _c(rows, np.int64)
    return r, len(r)


def gemv_bf16(packed, n: int, k: int, x_bf16, rows=None):
    """y[m, n] = sum_b scale[n,b] * sum_{k in b} t[n,k] x[m,k] in fp64; returns (y64, y32)."""
    packed = _c(packed, np.uint8)
    x = _c(x_bf16, np.uint16)
    m = x.shape[0]
    r, nr = _rows(rows, n)
    y64 = np.empty((m, nr), dtype=np.float64)
    y32 = np.empty((m, nr), dtype=np.float32)
    rc = lib().oracle_gemv_bf16(_ptr(packed), _i64(n), _i64(k), _ptr(x), _i64(m), _ptr(r), _i64(nr),
                                _ptr(y64), _ptr(y32))
    assert rc == 0, rc
    return y64, y32


def quantize_i8(x_bf16):
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    rc = lib().oracle_quantize_i8(_ptr(x), _i64(m), _i64(k), _ptr(q), _ptr(s))
    assert rc == 0, rc
    return q, s


def tern_i8(packed, n: int, k: int, q, s_x, rows=None, want_acc: bool = True):
    """int8-activation contraction: returns (acc[m, rows, K/128] int32 or None, y64, y32)."""
    packed = _c(packed, np.uint8)
    q = _c(q, np.int8)
    s_x = _c(s_x, np.float32)
    m = q.shape[0]
    r, nr = _rows(rows, n)
    acc = np.empty((m, nr, k // 128), dtype=np.int32) if want_acc else None
    y64 = np.empty((m, nr), dtype=np.float64)
    y32 = np.empty((m, nr), dtype=np.float32)
    rc = lib().oracle_tern_i8(_ptr(packed), _i64(n), _i64(k), _ptr(q), _ptr(s_x), _i64(m), _ptr(r), _i64(nr),
                              _ptr(acc), _ptr(y64), _ptr(y32))
    assert rc == 0, rc
    return acc, y64, y32


def head_bf16(w8, rs, x_bf16, rows=None):
    w8 = _c(w8, np.int8)
    rs = _c(rs, np.float32)
    x = _c(x_bf16, np.uint16)
    v, k = w8.shape
    m = x.shape[0]
    r, nr = _rows(rows, v)
    y64 = np.empty((m, nr), dtype=np.float64)
    y32 = np.empty((m, nr), dtype=np.float32)
    rc = lib().oracle_head_bf16(_ptr(w8), _ptr(rs), _i64(v), _i64(k), _ptr(x), _i64(m), _ptr(r), _i64(nr),
                                _ptr(y64), _ptr(y32))
    assert rc == 0, rc
    return y64, y32


def head_i8(w8, rs, q, s_x, rows=None):
    w8 = _c(w8, np.int8)
    rs = _c(rs, np.float32)
    q = _c(q, np.int8)
    s_x = _c(s_x, np.float32)
    v, k = w8.shape
    m = q.shape[0]
    r, nr = _rows(rows, v)
    acc = np.empty((m, nr), dtype=np.int32)
    y64 = np.empty((m, nr), dtype=np.float64)
    y32 = np.empty((m, nr), dtype=np.float32)
    rc = lib().oracle_head_i8(_ptr(w8), _ptr(rs), _i64(v), _i64(k), _ptr(q), _ptr(s_x), _i64(m), _ptr(r),
                              _i64(nr), _ptr(acc), _ptr(y64), _ptr(y32))
    assert rc == 0, rc
    return acc, y64, y32


def head_i8_logits_f32(acc, rs, s_x):
    """fp32 logits of the int8-activation head from its exact int32 sums, in
    the operation order the library states: (rs[v] * s_x[m]) * acc[m][v], each
    product rounded to fp32 ([P2] "3진 계열이라는 이름의 실체": the head stays
    int8; greedy decoding compares float32 logits, [P2] "토큰 동일성의 경계:
    그리디, float32, 그리고 두 개의 근접 동점")."""
    acc = np.asarray(acc, dtype=np.int64)
    assert np.abs(acc).max(initial=0) < (1 << 31), "int32 sums"
    # int32 -> fp32 rounds to nearest-even (exact below 2^24)
    rs = np.asarray(rs, dtype=np.float32)
    s_x = np.asarray(s_x, dtype=np.float32)
    scale = (rs[None, :] * s_x[:, None]).astype(np.float32)          # one fp32 product
    return (scale * acc.astype(np.float32)).astype(np.float32)        # a second one


def greedy_argmax(logits):
    """Greedy decode over fp32 logits [M, V] ([P2] "토큰 동일성의 경계: 그리디,
    float32, 그리고 두 개의 근접 동점": the next token is the argmax of float32
    logits, and near ties occur): per row, the index of the largest value, the
    lowest index among equal values, -0 counted as +0.  Returns (idx int32 [M],
    val fp32 [M])."""
    z = np.asarray(logits, dtype=np.float32) + np.float32(0.0)   # -0 -> +0
    assert np.isfinite(z).all()
    idx = np.argmax(z, axis=1)                                   # first (lowest) index of the maximum
    return idx.astype(np.int32), z[np.arange(z.shape[0]), idx]


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_threads(n: int) -> int:
    """OpenMP threads of the oracle's loops from now on; returns the count in effect."""
    return int(lib().oracle_set_threads(int(n)))


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 in fp64 (0 when both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    return float(num / den) if den > 0 else float(num)
