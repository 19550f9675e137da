"""Python binding of libtern.so — gfx950 ternary-weight GEMV / GEMM kernels.

Thin argument marshalling over the C ABI of ``include/tern.h``: every call
takes torch tensors that already live on the GPU, passes their device
pointers and the current HIP stream to the library, and raises
``RuntimeError`` with the library's status text on any error.  torch is used
for device memory and streams only; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if ``libtern.so`` is missing or
fails to load, every call raises.

Names follow the C ABI: ``tern_pack``, ``tern_stats``, ``tern_quantize_i8``,
``tern_gemv``, ``tern_gemv_i8``, ``i8_head_gemv``, ``i8_head_gemv_i8``,
``tern_gemm_prefill``, ``tern_packed_bytes``, and the dependent-GEMV chain
``tern_chain_workspace_bytes``, ``tern_chain_plan``, ``tern_gemv_chain``, the
fused head + greedy argmax ``i8_head_argmax[_i8]``, and the five-level
(FV5-style) weights ``tern5_packed_bytes``, ``tern5_pack``, ``tern5_gemv[_i8]``, and the
block-scaled int8 head and embedding (FV5B-style) ``fv5b_head_gemv[_i8]``,
``fv5b_head_argmax[_i8]``, ``fv5b_head_argmax_embed``, ``fv5b_embed`` (and
``fv5b_head_gemv_packed[_i8]``, ``fv5b_head_argmax_packed[_i8]`` over the
packed copy), the
packed int8 head ``i8_head_packed_bytes``, ``i8_head_pack``,
``i8_head_gemv_packed[_i8]``, ``i8_head_argmax_packed[_i8]``, and the launch-configuration views
``tern_gemv_config`` and ``tern_prefill_config``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtern.so")
MAX_M_GEMV = 16
SYMBOLS = ("tern_strerror", "tern_last_error", "tern_abi_version", "tern_packed_bytes", "tern_pack", "tern_stats",
           "tern_quantize_i8", "tern_gemv", "tern_gemv_i8", "i8_head_gemv", "i8_head_gemv_i8", "tern_gemm_prefill",
           "tern_chain_workspace_bytes", "tern_chain_plan", "tern_gemv_chain", "i8_head_argmax_workspace_bytes",
           "i8_head_argmax", "i8_head_argmax_i8", "tern5_packed_bytes", "tern5_pack", "tern5_gemv", "tern5_gemv_i8",
           "fv5b_head_gemv", "fv5b_head_gemv_i8", "fv5b_head_argmax", "fv5b_head_argmax_i8", "fv5b_head_argmax_embed", "fv5b_embed",
           "tern_gemv_config", "tern_prefill_config", "tern_mfma_peak_ops", "tern_mfma_peak_sink_bytes", "tern_mfma_peak",
           "tern_launch_probe", "i8_head_argmax_noalloc", "i8_head_packed_bytes", "i8_head_pack",
           "i8_head_gemv_packed", "i8_head_gemv_packed_i8", "i8_head_argmax_packed", "i8_head_argmax_packed_i8",
           "fv5b_head_gemv_packed", "fv5b_head_gemv_packed_i8", "fv5b_head_argmax_packed",
           "fv5b_head_argmax_packed_i8")
_INT_STATUS = ("tern_pack", "tern_stats", "tern_quantize_i8", "tern_gemv", "tern_gemv_i8", "i8_head_gemv",
               "i8_head_gemv_i8", "tern_gemm_prefill", "tern_chain_plan", "tern_gemv_chain", "i8_head_argmax",
               "i8_head_argmax_i8", "tern5_pack", "tern5_gemv", "tern5_gemv_i8", "fv5b_head_gemv", "fv5b_head_gemv_i8",
               "fv5b_head_argmax", "fv5b_head_argmax_i8", "fv5b_head_argmax_embed", "fv5b_embed", "tern_mfma_peak",
               "tern_launch_probe", "i8_head_argmax_noalloc", "i8_head_pack", "i8_head_gemv_packed",
               "i8_head_gemv_packed_i8", "i8_head_argmax_packed", "i8_head_argmax_packed_i8",
               "fv5b_head_gemv_packed", "fv5b_head_gemv_packed_i8", "fv5b_head_argmax_packed",
               "fv5b_head_argmax_packed_i8")

_lib = None
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class TernChainStep(ctypes.Structure):
    """struct tern_chain_step of include/tern.h."""
    _fields_ = [("packed", _p), ("N", _i64), ("K", _i64), ("x", _p), ("x_from", _i64), ("y", _p)]


def lib():
    """Load libtern.so (built in-tree by ternary_weight_decode_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ternary_weight_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.tern_strerror.restype = ctypes.c_char_p
        L.tern_strerror.argtypes = [ctypes.c_int]
        L.tern_last_error.restype = ctypes.c_char_p
        L.tern_abi_version.restype = ctypes.c_int
        L.tern_packed_bytes.restype = _i64
        L.tern_packed_bytes.argtypes = [_i64, _i64]
        L.tern_pack.argtypes = [_p, _p, _i64, _i64, _p, _p]
        L.tern_stats.argtypes = [_p, _i64, _i64, _p, _p]
        L.tern_quantize_i8.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.tern_gemv.argtypes = [_p, _i64, _i64, _p, _i64, _p, _p]
        L.tern_gemv_i8.argtypes = [_p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.i8_head_gemv.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.i8_head_gemv_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.tern_gemm_prefill.argtypes = [_p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.tern_chain_workspace_bytes.restype = _i64
        L.tern_chain_workspace_bytes.argtypes = [ctypes.POINTER(TernChainStep), _i64]
        L.tern_chain_plan.argtypes = [ctypes.POINTER(TernChainStep), _i64, _p, _i64, _p]
        L.tern_gemv_chain.argtypes = [_p, _i64, _p]
        L.i8_head_argmax_workspace_bytes.restype = _i64
        L.i8_head_argmax_workspace_bytes.argtypes = [_i64, _i64]
        L.i8_head_argmax.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
        L.i8_head_argmax_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p, _p, _p]
        L.i8_head_argmax_noalloc.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p]
        L.tern5_packed_bytes.restype = _i64
        L.tern5_packed_bytes.argtypes = [_i64, _i64]
        L.tern5_pack.argtypes = [_p, _p, _p, _i64, _i64, _p, _p]
        L.tern5_gemv.argtypes = [_p, _i64, _i64, _p, _i64, _p, _p]
        L.tern5_gemv_i8.argtypes = [_p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.fv5b_head_gemv.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.fv5b_head_gemv_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.fv5b_head_argmax.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
        L.fv5b_head_argmax_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p, _p, _p]
        L.fv5b_embed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p]
        L.fv5b_head_argmax_embed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _i64, _i64, _p, _p,
                                             _p]
        L.tern_gemv_config.restype = ctypes.c_int
        L.tern_gemv_config.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(_i64)]
        L.tern_prefill_config.restype = ctypes.c_int
        L.tern_prefill_config.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_i64)]
        L.tern_mfma_peak_ops.restype = ctypes.c_double
        L.tern_mfma_peak_ops.argtypes = [ctypes.c_int, _i64, _i64]
        L.tern_mfma_peak_sink_bytes.restype = _i64
        L.tern_mfma_peak_sink_bytes.argtypes = [_i64]
        L.tern_mfma_peak.argtypes = [ctypes.c_int, _i64, _i64, _p, _p]
        L.tern_launch_probe.argtypes = [ctypes.c_int, _i64, _p, _i64, _p, _p]
        L.i8_head_packed_bytes.restype = _i64
        L.i8_head_packed_bytes.argtypes = [_i64, _i64]
        L.i8_head_pack.argtypes = [_p, _i64, _i64, _p, _p]
        L.i8_head_gemv_packed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.i8_head_gemv_packed_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.i8_head_argmax_packed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
        L.i8_head_argmax_packed_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p, _p, _p]
        L.fv5b_head_gemv_packed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.fv5b_head_gemv_packed_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.fv5b_head_argmax_packed.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
        L.fv5b_head_argmax_packed_i8.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p, _p, _p]
        for name in _INT_STATUS:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(name: str, rc: int):
    if rc != 0:
        L = lib()
        raise RuntimeError(f"{name}: {L.tern_strerror(rc).decode()} {L.tern_last_error().decode()}".strip())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise RuntimeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype not in dtypes:
        raise RuntimeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise RuntimeError(f"{name} must have {ndim} dimensions")


def tern_packed_bytes(n: int, k: int) -> int:
    return int(lib().tern_packed_bytes(n, k))


def tern_pack(t, scale, out=None, stream=None):
    """t int8 [N,K] in {-1,0,1}; scale fp16 bits [N,K/128] (int16/uint16/float16) -> packed uint8 blob."""
    import torch
    _need(t, "t", (torch.int8,), 2)
    _need(scale, "scale", (torch.int16, torch.uint16, torch.float16), 2)
    n, k = t.shape
    nbytes = tern_packed_bytes(n, k)
    if nbytes < 0:
        _check("tern_pack", 2)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=t.device)
    _check("tern_pack", lib().tern_pack(_ptr(t), _ptr(scale), n, k, _ptr(out), _stream(stream)))
    return out


def tern_stats(packed, n: int, k: int, out=None, stream=None):
    """-> int64 [3]: nonzero weights, -1 weights, non-canonical sign bits."""
    import torch
    if out is None:
        out = torch.empty(3, dtype=torch.int64, device=packed.device)
    _check("tern_stats", lib().tern_stats(_ptr(packed), n, k, _ptr(out), _stream(stream)))
    return out


def tern_quantize_i8(x, q=None, s_x=None, stream=None):
    """x bf16 [M,K] -> (q int8 [M,K], s_x fp32 [M])."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("tern_quantize_i8", lib().tern_quantize_i8(_ptr(x), m, k, _ptr(q), _ptr(s_x), _stream(stream)))
    return q, s_x


def tern_gemv(packed, n: int, k: int, x, y=None, stream=None):
    """y[m,n] = sum_b scale[n,b] sum_{k in b} t[n,k] x[m,k]; x bf16 [M,K], M <= 16 -> y fp32 [M,N]."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check("tern_gemv", lib().tern_gemv(_ptr(packed), n, k, _ptr(x), m, _ptr(y), _stream(stream)))
    return y


def tern_gemv_i8(packed, n: int, k: int, q, s_x, y=None, acc=None, stream=None):
    """int8 activations: y = s_x[m] * sum_b scale[n,b] acc[m,n,b]; acc (optional) int32 [M,N,K/128]."""
    import torch
    _need(q, "q", (torch.int8,), 2)
    m = q.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=q.device)
    _check("tern_gemv_i8", lib().tern_gemv_i8(_ptr(packed), n, k, _ptr(q), _ptr(s_x), m, _ptr(y), _ptr(acc),
                                              _stream(stream)))
    return y


def i8_head_gemv(w, row_scale, x, y=None, stream=None):
    """logits[m,v] = row_scale[v] sum_k W[v,k] x[m,k]; W int8 [V,K], x bf16 [M,K]."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    v, k = w.shape
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=x.device)
    _check("i8_head_gemv", lib().i8_head_gemv(_ptr(w), _ptr(row_scale), v, k, _ptr(x), m, _ptr(y),
                                              _stream(stream)))
    return y


def i8_head_gemv_i8(w, row_scale, q, s_x, y=None, acc=None, stream=None):
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(q, "q", (torch.int8,), 2)
    v, k = w.shape
    m = q.shape[0]
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=q.device)
    _check("i8_head_gemv_i8", lib().i8_head_gemv_i8(_ptr(w), _ptr(row_scale), v, k, _ptr(q), _ptr(s_x), m, _ptr(y),
                                                    _ptr(acc), _stream(stream)))
    return y


def i8_head_packed_bytes(v: int, k: int) -> int:
    return int(lib().i8_head_packed_bytes(v, k))


def i8_head_pack(w, out=None, stream=None):
    """W int8 [V,K] -> its packed copy (int8, i8_head_packed_bytes(V, K) bytes) for i8_head_gemv_packed[_i8]."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    v, k = w.shape
    nbytes = i8_head_packed_bytes(v, k)
    if nbytes < 0:
        _check("i8_head_pack", 2)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.int8, device=w.device)
    _check("i8_head_pack", lib().i8_head_pack(_ptr(w), v, k, _ptr(out), _stream(stream)))
    return out


def i8_head_gemv_packed(wp, row_scale, v: int, k: int, x, y=None, stream=None):
    """i8_head_gemv over the packed copy wp of W [v,k]; x bf16 [M,K] -> logits fp32 [M,V]."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=x.device)
    _check("i8_head_gemv_packed", lib().i8_head_gemv_packed(_ptr(wp), _ptr(row_scale), v, k, _ptr(x), m, _ptr(y),
                                                            _stream(stream)))
    return y


def i8_head_gemv_packed_i8(wp, row_scale, v: int, k: int, q, s_x, y=None, acc=None, stream=None):
    import torch
    _need(q, "q", (torch.int8,), 2)
    m = q.shape[0]
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=q.device)
    _check("i8_head_gemv_packed_i8", lib().i8_head_gemv_packed_i8(_ptr(wp), _ptr(row_scale), v, k, _ptr(q),
                                                                  _ptr(s_x), m, _ptr(y), _ptr(acc), _stream(stream)))
    return y


def i8_head_argmax_packed(wp, row_scale, v: int, k: int, x, workspace=None, logits=None, stream=None):
    """i8_head_argmax over the packed copy wp of W [v,k]: (idx int32 [M], val fp32 [M])."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m = x.shape[0]
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, x.device)
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    val = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("i8_head_argmax_packed", lib().i8_head_argmax_packed(_ptr(wp), _ptr(row_scale), v, k, _ptr(x), m,
                                                                _ptr(idx), _ptr(val), _ptr(logits),
                                                                _ptr(workspace), _stream(stream)))
    return idx, val


def i8_head_argmax_packed_i8(wp, row_scale, v: int, k: int, q, s_x, workspace=None, logits=None, stream=None):
    import torch
    _need(q, "q", (torch.int8,), 2)
    m = q.shape[0]
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, q.device)
    idx = torch.empty(m, dtype=torch.int32, device=q.device)
    val = torch.empty(m, dtype=torch.float32, device=q.device)
    _check("i8_head_argmax_packed_i8", lib().i8_head_argmax_packed_i8(_ptr(wp), _ptr(row_scale), v, k, _ptr(q),
                                                                      _ptr(s_x), m, _ptr(idx), _ptr(val),
                                                                      _ptr(logits), _ptr(workspace),
                                                                      _stream(stream)))
    return idx, val


def i8_head_argmax_workspace_bytes(v: int, m: int) -> int:
    return int(lib().i8_head_argmax_workspace_bytes(v, m))


def i8_head_argmax_workspace(v: int, m: int, device="cuda"):
    """A workspace for i8_head_argmax[_i8] over V head rows and up to m activation rows."""
    import torch
    return torch.empty(i8_head_argmax_workspace_bytes(v, m), dtype=torch.uint8, device=device)


def i8_head_argmax(w, row_scale, x, workspace=None, logits=None, stream=None):
    """Greedy argmax over the head logits of bf16 x: (idx int32 [M], val fp32 [M]); logits [M, V] filled when given."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    v, k = w.shape
    m = x.shape[0]
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, x.device)
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    val = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("i8_head_argmax", lib().i8_head_argmax(_ptr(w), _ptr(row_scale), v, k, _ptr(x), m, _ptr(idx), _ptr(val),
                                                  _ptr(logits), _ptr(workspace), _stream(stream)))
    return idx, val


def i8_head_argmax_noalloc(w, row_scale, x, idx, val, logits=None, stream=None):
    """i8_head_argmax with the keys in the library's own device array: allocates nothing, so the
    caller passes idx (int32 [M]) and val (fp32 [M]); calls overlapping on one device race."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    v, k = w.shape
    m = x.shape[0]
    _check("i8_head_argmax_noalloc", lib().i8_head_argmax_noalloc(_ptr(w), _ptr(row_scale), v, k, _ptr(x), m,
                                                                  _ptr(idx), _ptr(val), _ptr(logits),
                                                                  _stream(stream)))
    return idx, val


def i8_head_argmax_i8(w, row_scale, q, s_x, workspace=None, logits=None, stream=None):
    """Greedy argmax over the head logits of int8 q (row scales s_x): (idx, val)."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(q, "q", (torch.int8,), 2)
    v, k = w.shape
    m = q.shape[0]
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, q.device)
    idx = torch.empty(m, dtype=torch.int32, device=q.device)
    val = torch.empty(m, dtype=torch.float32, device=q.device)
    _check("i8_head_argmax_i8", lib().i8_head_argmax_i8(_ptr(w), _ptr(row_scale), v, k, _ptr(q), _ptr(s_x), m,
                                                        _ptr(idx), _ptr(val), _ptr(logits), _ptr(workspace),
                                                        _stream(stream)))
    return idx, val


def tern_gemm_prefill(packed, n: int, k: int, q, s_x, y=None, acc=None, stream=None):
    import torch
    _need(q, "q", (torch.int8,), 2)
    m = q.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=q.device)
    _check("tern_gemm_prefill", lib().tern_gemm_prefill(_ptr(packed), n, k, _ptr(q), _ptr(s_x), m, _ptr(y),
                                                        _ptr(acc), _stream(stream)))
    return y


def _chain_array(steps):
    """ctypes tern_chain_step array from (packed, N, K, x or None, x_from, y) tuples of tensors."""
    import torch
    arr = (TernChainStep * max(1, len(steps)))()
    for i, (packed, n, k, x, x_from, y) in enumerate(steps):
        _need(packed, "packed", (torch.uint8,))
        _need(y, "y", (torch.float32,))
        if y.numel() != n:
            raise RuntimeError(f"tern_chain: step {i} y has {y.numel()} elements, N = {n}")
        if x is not None:
            _need(x, "x", (torch.int16, torch.uint16, torch.bfloat16))
            if x.numel() != k:
                raise RuntimeError(f"tern_chain: step {i} x has {x.numel()} elements, K = {k}")
        arr[i] = TernChainStep(packed.data_ptr(), n, k, None if x is None else x.data_ptr(), x_from, y.data_ptr())
    return arr


def tern_chain_workspace_bytes(steps) -> int:
    return int(lib().tern_chain_workspace_bytes(_chain_array(steps), len(steps)))


def tern_chain_workspace(steps, device="cuda"):
    """A zero-filled workspace sized for this chain."""
    import torch
    nbytes = tern_chain_workspace_bytes(steps)
    if nbytes < 0:
        _check("tern_chain_workspace_bytes", 2)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def tern_chain_plan(steps, workspace, stream=None):
    """steps: sequence of (packed, N, K, x, x_from, y): x bf16 bits [K] (None when
    x_from >= 0), x_from -1 or an earlier step whose first K outputs, rounded
    to bf16, are x; y fp32 [N].  Writes the device plan into workspace."""
    import torch
    arr = _chain_array(steps)
    _need(workspace, "workspace", (torch.uint8,), 1)
    _check("tern_chain_plan", lib().tern_chain_plan(arr, len(steps), _ptr(workspace), workspace.numel(),
                                                    _stream(stream)))


def tern_gemv_chain(workspace, nsteps: int, stream=None):
    import torch
    _need(workspace, "workspace", (torch.uint8,), 1)
    _check("tern_gemv_chain", lib().tern_gemv_chain(_ptr(workspace), nsteps, _stream(stream)))


def tern_chain_errors(workspace) -> int:
    """Count of aborted waits recorded in a chain workspace (0 in normal operation)."""
    import torch
    return int(workspace[8:12].view(torch.int32).item())


# ---------------------------------------------------------------- five-level

def tern5_packed_bytes(n: int, k: int) -> int:
    return int(lib().tern5_packed_bytes(n, k))


def tern5_pack(levels, s_lo, s_hi, out=None, stream=None):
    """levels int8 [N,K] in [-2,2], K % 512 == 0; s_lo, s_hi fp32 [N,K/256] -> five-level uint8 blob."""
    import torch
    _need(levels, "levels", (torch.int8,), 2)
    _need(s_lo, "s_lo", (torch.float32,), 2)
    _need(s_hi, "s_hi", (torch.float32,), 2)
    n, k = levels.shape
    if tuple(s_lo.shape) != (n, k // 256) or tuple(s_hi.shape) != (n, k // 256):
        raise RuntimeError("tern5_pack: s_lo and s_hi must be [N, K/256]")
    nbytes = tern5_packed_bytes(n, k)
    if nbytes < 0:
        _check("tern5_pack", 2)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=levels.device)
    _check("tern5_pack", lib().tern5_pack(_ptr(levels), _ptr(s_lo), _ptr(s_hi), n, k, _ptr(out), _stream(stream)))
    return out


def tern5_gemv(packed, n: int, k: int, x, y=None, stream=None):
    """y[m,n] = sum_k W[n,k] x[m,k] for the five-level W; x bf16 [M,K], M <= 16 -> y fp32 [M,N]."""
    import torch
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check("tern5_gemv", lib().tern5_gemv(_ptr(packed), n, k, _ptr(x), m, _ptr(y), _stream(stream)))
    return y


def tern5_gemv_i8(packed, n: int, k: int, q, s_x, y=None, acc=None, stream=None):
    """int8 activations for the five-level W: y = s_x[m] sum_b (s_lo acc_lo + s_hi acc_hi);
    acc (optional) int32 [M,N,K/256,2]."""
    import torch
    _need(q, "q", (torch.int8,), 2)
    m = q.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=q.device)
    _check("tern5_gemv_i8", lib().tern5_gemv_i8(_ptr(packed), n, k, _ptr(q), _ptr(s_x), m, _ptr(y), _ptr(acc),
                                                _stream(stream)))
    return y


# ------------------------------------------------- block-scaled int8 (FV5B)

def _fv5b_args(w, s, act, act_dtypes):
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(s, "S", (torch.float32,), 2)
    _need(act, "activations", act_dtypes, 2)
    v, k = w.shape
    if tuple(s.shape) != (v, k // 256):
        raise RuntimeError("S must be [V, K/256]")
    return v, k, act.shape[0]


def fv5b_head_gemv(w, s, x, y=None, stream=None):
    """logits[m,v] = sum_b S[v,b] sum_{k in b} W[v,k] x[m,k]; W int8 [V,K], S fp32 [V,K/256], x bf16 [M,K]."""
    import torch
    v, k, m = _fv5b_args(w, s, x, (torch.bfloat16, torch.int16, torch.uint16))
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=x.device)
    _check("fv5b_head_gemv", lib().fv5b_head_gemv(_ptr(w), _ptr(s), v, k, _ptr(x), m, _ptr(y), _stream(stream)))
    return y


def fv5b_head_gemv_i8(w, s, q, s_x, y=None, acc=None, stream=None):
    """int8 activations: logits = s_x[m] sum_b S[v,b] acc[m,v,b]; acc (optional) int32 [M,V,K/256]."""
    import torch
    v, k, m = _fv5b_args(w, s, q, (torch.int8,))
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=q.device)
    _check("fv5b_head_gemv_i8", lib().fv5b_head_gemv_i8(_ptr(w), _ptr(s), v, k, _ptr(q), _ptr(s_x), m, _ptr(y),
                                                        _ptr(acc), _stream(stream)))
    return y


def fv5b_head_argmax(w, s, x, workspace=None, logits=None, stream=None):
    """Greedy argmax over the block-scaled head's logits of bf16 x: (idx int32 [M], val fp32 [M])."""
    import torch
    v, k, m = _fv5b_args(w, s, x, (torch.bfloat16, torch.int16, torch.uint16))
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, x.device)
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    val = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("fv5b_head_argmax", lib().fv5b_head_argmax(_ptr(w), _ptr(s), v, k, _ptr(x), m, _ptr(idx), _ptr(val),
                                                      _ptr(logits), _ptr(workspace), _stream(stream)))
    return idx, val


def fv5b_head_argmax_i8(w, s, q, s_x, workspace=None, logits=None, stream=None):
    """Greedy argmax over the block-scaled head's logits of int8 q: (idx, val)."""
    import torch
    v, k, m = _fv5b_args(w, s, q, (torch.int8,))
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, q.device)
    idx = torch.empty(m, dtype=torch.int32, device=q.device)
    val = torch.empty(m, dtype=torch.float32, device=q.device)
    _check("fv5b_head_argmax_i8", lib().fv5b_head_argmax_i8(_ptr(w), _ptr(s), v, k, _ptr(q), _ptr(s_x), m,
                                                            _ptr(idx), _ptr(val), _ptr(logits), _ptr(workspace),
                                                            _stream(stream)))
    return idx, val


def _fv5b_packed_args(s, v, k, act, act_dtypes):
    import torch
    _need(s, "S", (torch.float32,), 2)
    _need(act, "activations", act_dtypes, 2)
    if tuple(s.shape) != (v, k // 256):
        raise RuntimeError("S must be [V, K/256]")
    return act.shape[0]


def fv5b_head_gemv_packed(wp, s, v: int, k: int, x, y=None, stream=None):
    """fv5b_head_gemv over the packed copy wp (i8_head_pack) of W [v,k]."""
    import torch
    m = _fv5b_packed_args(s, v, k, x, (torch.bfloat16, torch.int16, torch.uint16))
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=x.device)
    _check("fv5b_head_gemv_packed", lib().fv5b_head_gemv_packed(_ptr(wp), _ptr(s), v, k, _ptr(x), m, _ptr(y),
                                                                _stream(stream)))
    return y


def fv5b_head_gemv_packed_i8(wp, s, v: int, k: int, q, s_x, y=None, acc=None, stream=None):
    import torch
    m = _fv5b_packed_args(s, v, k, q, (torch.int8,))
    if y is None:
        y = torch.empty((m, v), dtype=torch.float32, device=q.device)
    _check("fv5b_head_gemv_packed_i8", lib().fv5b_head_gemv_packed_i8(_ptr(wp), _ptr(s), v, k, _ptr(q), _ptr(s_x),
                                                                      m, _ptr(y), _ptr(acc), _stream(stream)))
    return y


def fv5b_head_argmax_packed(wp, s, v: int, k: int, x, workspace=None, logits=None, stream=None):
    import torch
    m = _fv5b_packed_args(s, v, k, x, (torch.bfloat16, torch.int16, torch.uint16))
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, x.device)
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    val = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("fv5b_head_argmax_packed", lib().fv5b_head_argmax_packed(_ptr(wp), _ptr(s), v, k, _ptr(x), m, _ptr(idx),
                                                                    _ptr(val), _ptr(logits), _ptr(workspace),
                                                                    _stream(stream)))
    return idx, val


def fv5b_head_argmax_packed_i8(wp, s, v: int, k: int, q, s_x, workspace=None, logits=None, stream=None):
    import torch
    m = _fv5b_packed_args(s, v, k, q, (torch.int8,))
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, q.device)
    idx = torch.empty(m, dtype=torch.int32, device=q.device)
    val = torch.empty(m, dtype=torch.float32, device=q.device)
    _check("fv5b_head_argmax_packed_i8", lib().fv5b_head_argmax_packed_i8(_ptr(wp), _ptr(s), v, k, _ptr(q),
                                                                          _ptr(s_x), m, _ptr(idx), _ptr(val),
                                                                          _ptr(logits), _ptr(workspace),
                                                                          _stream(stream)))
    return idx, val


def fv5b_head_argmax_embed(w, s, x, e, es, workspace=None, logits=None, f32=True, bf16=True, out=None,
                           out_bf16=None, stream=None):
    """Greedy argmax over the block-scaled head's logits of bf16 x, then the embedding rows of the chosen
    indices from the block-scaled table (e int8 [Ve,Ke], es fp32 [Ve,Ke/256]), in one call:
    (idx int32 [M], val fp32 [M], emb fp32 [M,Ke] or None, emb bf16 [M,Ke] or None)."""
    import torch
    v, k, m = _fv5b_args(w, s, x, (torch.bfloat16, torch.int16, torch.uint16))
    _need(e, "E", (torch.int8,), 2)
    _need(es, "ES", (torch.float32,), 2)
    ve, ke = e.shape
    if workspace is None:
        workspace = i8_head_argmax_workspace(v, m, x.device)
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    val = torch.empty(m, dtype=torch.float32, device=x.device)
    if out is None and f32:
        out = torch.empty((m, ke), dtype=torch.float32, device=x.device)
    if out_bf16 is None and bf16:
        out_bf16 = torch.empty((m, ke), dtype=torch.bfloat16, device=x.device)
    _check("fv5b_head_argmax_embed",
           lib().fv5b_head_argmax_embed(_ptr(w), _ptr(s), v, k, _ptr(x), m, _ptr(idx), _ptr(val), _ptr(logits),
                                        _ptr(workspace), _ptr(e), _ptr(es), ve, ke, _ptr(out), _ptr(out_bf16),
                                        _stream(stream)))
    return idx, val, out, out_bf16


def fv5b_embed(w, s, ids, f32=True, bf16=True, out=None, out_bf16=None, stream=None):
    """Embedding rows of int32 token ids [M]: (fp32 [M,K] or None, bf16 [M,K] or None); ids outside [0,V)
    give zeros.  Preallocated outputs may be passed as out / out_bf16."""
    import torch
    _need(w, "W", (torch.int8,), 2)
    _need(s, "S", (torch.float32,), 2)
    _need(ids, "ids", (torch.int32,), 1)
    v, k = w.shape
    m = ids.shape[0]
    if out is None and f32:
        out = torch.empty((m, k), dtype=torch.float32, device=ids.device)
    if out_bf16 is None and bf16:
        out_bf16 = torch.empty((m, k), dtype=torch.bfloat16, device=ids.device)
    _check("fv5b_embed", lib().fv5b_embed(_ptr(w), _ptr(s), v, k, _ptr(ids), m, _ptr(out), _ptr(out_bf16),
                                          _stream(stream)))
    return out, out_bf16


GEMV_KINDS = {"ternary_bf16": 0, "ternary_int8": 1, "fv5_bf16": 2, "fv5_int8": 3,
              "ternary_bf16_phased": 4, "ternary_int8_phased": 5, "fv5_bf16_phased": 6, "fv5_int8_phased": 7,
              "ternary_bf16_phased3": 8}


def tern_gemv_config(n: int, k: int, m: int, kind: str = "ternary_bf16"):
    """The one-pass launch configuration for this GEMV shape (host-side, no device needed), as a dict,
    or None when another kernel takes the shape."""
    out = (_i64 * 8)()
    rc = lib().tern_gemv_config(n, k, m, GEMV_KINDS[kind], out)
    if rc < 0:
        _check("tern_gemv_config", -rc)
    if rc == 0:
        return None
    keys = ("R", "waves", "U", "XC", "grid", "lds", "rounds", "MT")
    return dict(zip(keys, (int(v) for v in out)))


def tern_prefill_config(n: int, k: int, m: int):
    """The workgroup-shared-decode prefill launch for this shape (host-side, no device
    needed), as a dict, or None when another kernel takes the shape."""
    out = (_i64 * 6)()
    rc = lib().tern_prefill_config(n, k, m, out)
    if rc < 0:
        _check("tern_prefill_config", -rc)
    if rc == 0:
        return None
    keys = ("BM", "BN", "split", "grid_x", "grid_y", "grid_z")
    return dict(zip(keys, (int(v) for v in out)))


LAUNCH_PROBE_KINDS = {"empty": 0, "store": 1, "load": 2, "read": 3}


def tern_launch_probe(kind: str, grid: int, src=None, sink=None, stream=None):
    """Launch-floor / read-ceiling probe (measurement aid): enqueue one launch
    ("empty", "store": one float per workgroup, "load": one 16-byte load of
    src per thread first, "read": all of src read once by `grid` workgroups of
    256 threads).  src: a zero-filled device tensor (16-byte aligned); sink:
    at least `grid` floats (allocated when None)."""
    import torch
    if sink is None and kind != "empty":
        sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    nbytes = 0 if src is None else src.numel() * src.element_size()
    _check("tern_launch_probe", lib().tern_launch_probe(LAUNCH_PROBE_KINDS[kind], grid, _ptr(src), nbytes,
                                                         _ptr(sink), _stream(stream)))
    return sink


MFMA_PEAK_KINDS = {"int8": 0, "bf16": 1}


def tern_mfma_peak(kind: str, iters: int, grid: int, sink=None, stream=None):
    """Matrix-core throughput probe (measurement aid): enqueue one launch of
    `grid` workgroups running independent MFMA chains of `iters` steps
    ("int8": 16x16x64 i8, "bf16": 16x16x32 bf16).  Returns the operations the
    launch executes; time it with events on the same stream."""
    import torch
    k = MFMA_PEAK_KINDS[kind]
    ops = float(lib().tern_mfma_peak_ops(k, iters, grid))
    if ops < 0:
        _check("tern_mfma_peak", 2)
    if sink is None:
        sink = torch.empty(int(lib().tern_mfma_peak_sink_bytes(grid)) // 4, dtype=torch.int32, device="cuda")
    _check("tern_mfma_peak", lib().tern_mfma_peak(k, iters, grid, _ptr(sink), _stream(stream)))
    return ops
