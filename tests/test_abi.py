"""The C ABI loads, exports every declared symbol, and rejects bad arguments
on the host before any HIP call (runs without a GPU).  Every call below
passes bogus device addresses, so each must fail validation (or be an empty
problem): one that passed would launch a kernel on those addresses on a
machine with a GPU."""
import ctypes
import os
import re

import pytest

import ternary_weight_decode_amd as tw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tern.h")

E_OK, E_NULL, E_SHAPE, E_ALIGN = 0, 1, 2, 3
ALIGNED = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(0x10004)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    L = tw.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tw.SYMBOLS)


def test_version_and_strings():
    L = tw.lib()
    assert L.tern_abi_version() == 10
    for rc in range(6):
        assert len(L.tern_strerror(rc)) > 0
    assert L.tern_last_error() == b""


def test_packed_bytes():
    assert tw.tern_packed_bytes(3072, 1024) == 835_584
    assert tw.tern_packed_bytes(1, 128) == 544
    assert tw.tern_packed_bytes(20, 640) == 5440
    assert tw.tern_packed_bytes(12288, 4096) == 12288 * 4096 // 128 * 34
    assert tw.tern_packed_bytes(0, 128) == 0
    assert tw.tern_packed_bytes(16, 100) == -1
    assert tw.tern_packed_bytes(-1, 128) == -1


def test_shape_errors_before_any_device_call():
    L = tw.lib()
    p, s = ALIGNED, None
    assert L.tern_gemv(p, 16, 100, p, 1, p, s) == E_SHAPE          # K % 128
    assert L.tern_gemv(p, -1, 128, p, 1, p, s) == E_SHAPE          # negative N
    assert L.tern_gemv(p, 16, 128, p, 17, p, s) == E_SHAPE         # M > 16
    assert L.tern_gemv(p, 16, 128, p, -1, p, s) == E_SHAPE
    assert L.tern_gemv_i8(p, 16, 128, p, p, 17, p, None, s) == E_SHAPE
    assert L.i8_head_gemv(p, p, 100, 96, p, 1, p, s) == E_SHAPE            # K % 128 (as tern.h states)
    assert L.i8_head_gemv_i8(p, p, 100, 96, p, p, 1, p, None, s) == E_SHAPE   # K % 128
    assert L.i8_head_gemv_i8(p, p, 100, 128, p, p, 20, p, None, s) == E_SHAPE
    assert L.tern_gemm_prefill(p, 16, 200, p, p, 64, p, None, s) == E_SHAPE
    assert L.tern_gemm_prefill(p, 16, 128, p, p, -5, p, None, s) == E_SHAPE
    assert L.tern_pack(p, p, 16, 130, p, s) == E_SHAPE
    assert L.tern_stats(p, 16, 130, p, s) == E_SHAPE
    assert L.tern_quantize_i8(p, 4, 24, p, p, s) == E_SHAPE        # K % 16
    assert L.tern_quantize_i8(p, -4, 32, p, p, s) == E_SHAPE


def test_empty_problems_are_no_ops():
    L = tw.lib()
    assert L.tern_gemv(None, 0, 128, None, 1, None, None) == E_OK
    assert L.tern_gemv(None, 16, 128, None, 0, None, None) == E_OK
    assert L.tern_gemv_i8(None, 16, 128, None, None, 0, None, None, None) == E_OK
    assert L.i8_head_gemv(None, None, 0, 128, None, 1, None, None) == E_OK
    assert L.tern_gemm_prefill(None, 16, 128, None, None, 0, None, None, None) == E_OK
    assert L.tern_pack(None, None, 0, 128, None, None) == E_OK
    assert L.tern_quantize_i8(None, 0, 128, None, None, None) == E_OK


def test_null_and_alignment_errors():
    L = tw.lib()
    p, m = ALIGNED, MISALIGNED
    assert L.tern_gemv(None, 16, 128, p, 1, p, None) == E_NULL
    assert L.tern_gemv(p, 16, 128, None, 1, p, None) == E_NULL
    assert L.tern_gemv(p, 16, 128, p, 1, None, None) == E_NULL
    assert L.tern_gemv(m, 16, 128, p, 1, p, None) == E_ALIGN
    assert L.tern_gemv(p, 16, 128, m, 1, p, None) == E_ALIGN
    assert L.tern_gemv_i8(p, 16, 128, p, None, 1, p, None, None) == E_NULL
    assert L.tern_gemv_i8(p, 16, 128, m, p, 1, p, None, None) == E_ALIGN
    assert L.i8_head_gemv(p, None, 16, 128, p, 1, p, None) == E_NULL
    assert L.i8_head_gemv(m, p, 16, 128, p, 1, p, None) == E_ALIGN
    assert L.i8_head_gemv_i8(p, p, 16, 128, p, None, 1, p, None, None) == E_NULL
    assert L.tern_gemm_prefill(p, 16, 128, None, p, 64, p, None, None) == E_NULL
    assert L.tern_gemm_prefill(p, 16, 128, m, p, 64, p, None, None) == E_ALIGN
    assert L.tern_pack(None, p, 16, 128, p, None) == E_NULL
    assert L.tern_pack(p, p, 16, 128, m, None) == E_ALIGN
    assert L.tern_stats(p, 16, 128, None, None) == E_NULL
    assert L.tern_quantize_i8(p, 2, 128, p, None, None) == E_NULL
    assert L.tern_quantize_i8(m, 2, 128, p, p, None) == E_ALIGN


def test_head_argmax_workspace_and_argument_errors():
    L = tw.lib()
    assert tw.i8_head_argmax_workspace_bytes(151936, 1) == 9496 * 8
    assert tw.i8_head_argmax_workspace_bytes(100, 16) == 7 * 16 * 8
    assert tw.i8_head_argmax_workspace_bytes(100, 0) == -1 and tw.i8_head_argmax_workspace_bytes(100, 17) == -1
    assert tw.i8_head_argmax_workspace_bytes(0, 1) == -1
    p, m = ALIGNED, MISALIGNED
    f, fi = L.i8_head_argmax, L.i8_head_argmax_i8
    assert f(p, p, 100, 96, p, 1, p, p, None, p, None) == E_SHAPE          # K % 128
    assert f(p, p, 0, 128, p, 1, p, p, None, p, None) == E_SHAPE           # V = 0: no argmax
    assert f(p, p, 100, 128, p, 0, p, p, None, p, None) == E_SHAPE         # M = 0
    assert f(p, p, 100, 128, p, 17, p, p, None, p, None) == E_SHAPE        # M > 16
    assert f(p, p, 100, 8192, p, 16, p, p, None, p, None) == E_SHAPE       # bf16 x of 16 x 8192 does not fit LDS
    # int8 q of the same shape fits: the shape check passes and the missing workspace is reported (a
    # complete argument list would launch on the bogus addresses wherever a GPU is present)
    assert fi(p, p, 100, 8192, p, p, 16, p, p, None, None, None) == E_NULL
    assert f(p, p, 100, 128, p, 1, p, p, None, None, None) == E_NULL       # workspace
    assert f(p, p, 100, 128, p, 1, None, p, None, p, None) == E_NULL       # idx
    assert fi(p, p, 100, 128, p, None, 1, p, p, None, p, None) == E_NULL   # s_x
    assert f(m, p, 100, 128, p, 1, p, p, None, p, None) == E_ALIGN
    assert f(p, p, 100, 128, p, 1, p, p, ctypes.c_void_p(0x10002), p, None) == E_ALIGN   # logits
    assert f(p, p, 100, 128, p, 1, p, p, None, ctypes.c_void_p(0x10004), None) == E_ALIGN


def test_five_level_sizes_and_argument_errors():
    L = tw.lib()
    # planes Np*K*3/8 then Np*(K/256) pairs of f32 scales (3.25 bits per weight)
    assert tw.tern5_packed_bytes(16, 512) == 3072 + 16 * 2 * 8
    assert tw.tern5_packed_bytes(12288, 4096) == 12288 * 4096 * 13 // 32
    assert tw.tern5_packed_bytes(17, 1024) == 13312
    assert tw.tern5_packed_bytes(0, 512) == 0
    assert tw.tern5_packed_bytes(16, 768) == -1 and tw.tern5_packed_bytes(-1, 512) == -1
    p, m = ALIGNED, MISALIGNED
    g, pk = L.tern5_gemv, L.tern5_pack
    assert g(p, 16, 768, p, 1, p, None) == E_SHAPE            # K % 512
    assert g(p, 16, 512, p, 17, p, None) == E_SHAPE           # M > 16
    assert g(p, -1, 512, p, 1, p, None) == E_SHAPE
    assert pk(p, p, p, 16, 256, p, None) == E_SHAPE
    assert g(None, 0, 512, None, 1, None, None) == E_OK
    assert g(None, 16, 512, None, 0, None, None) == E_OK
    assert pk(None, None, None, 0, 512, None, None) == E_OK
    assert g(None, 16, 512, p, 1, p, None) == E_NULL
    assert g(p, 16, 512, p, 1, None, None) == E_NULL
    assert g(m, 16, 512, p, 1, p, None) == E_ALIGN
    assert g(p, 16, 512, m, 1, p, None) == E_ALIGN
    assert pk(p, None, p, 16, 512, p, None) == E_NULL
    assert pk(m, p, p, 16, 512, p, None) == E_ALIGN
    assert pk(p, p, ctypes.c_void_p(0x10002), 16, 512, p, None) == E_ALIGN
    gi = L.tern5_gemv_i8
    assert gi(p, 16, 768, p, p, 1, p, None, None) == E_SHAPE
    assert gi(p, 16, 512, p, p, 17, p, None, None) == E_SHAPE
    assert gi(None, 0, 512, None, None, 1, None, None, None) == E_OK
    assert gi(p, 16, 512, p, None, 1, p, None, None) == E_NULL        # s_x
    assert gi(p, 16, 512, m, p, 1, p, None, None) == E_ALIGN
    assert gi(p, 16, 512, p, p, 1, p, ctypes.c_void_p(0x10002), None) == E_ALIGN


def test_fv5b_argument_errors():
    L = tw.lib()
    p, m = ALIGNED, MISALIGNED
    h, hi, a, e = L.fv5b_head_gemv, L.fv5b_head_gemv_i8, L.fv5b_head_argmax, L.fv5b_embed
    assert h(p, p, 100, 384, p, 1, p, None) == E_SHAPE                 # K % 256
    assert h(p, p, 100, 0, p, 1, p, None) == E_SHAPE                   # K = 0
    assert h(p, p, 0, 256, p, 1, p, None) == E_SHAPE                   # V = 0
    assert h(p, p, 100, 256, p, 17, p, None) == E_SHAPE                # M > 16
    assert h(p, p, 100, 8192, p, 16, p, None) == E_SHAPE               # x does not fit in LDS
    assert hi(p, p, 100, 8192, p, p, 16, None, None, None) == E_NULL   # int8 q of that shape fits (no launch)
    assert h(p, None, 100, 256, p, 1, p, None) == E_NULL
    assert h(p, p, 100, 256, p, 1, None, None) == E_NULL
    assert hi(p, p, 100, 256, p, None, 1, p, None, None) == E_NULL     # s_x
    assert h(m, p, 100, 256, p, 1, p, None) == E_ALIGN
    assert h(p, ctypes.c_void_p(0x10002), 100, 256, p, 1, p, None) == E_ALIGN
    assert hi(p, p, 100, 256, p, p, 1, p, ctypes.c_void_p(0x10002), None) == E_ALIGN
    assert a(p, p, 100, 256, p, 1, None, p, None, p, None) == E_NULL  # idx
    assert a(p, p, 100, 256, p, 1, p, p, None, None, None) == E_NULL  # workspace
    assert a(p, p, 100, 256, p, 1, p, p, None, m, None) == E_ALIGN     # workspace 8-byte
    assert e(p, p, 10, 384, p, 4, p, p, None) == E_SHAPE               # K % 256
    assert e(p, p, 10, 256, p, -1, p, p, None) == E_SHAPE
    assert e(None, None, 10, 256, None, 0, None, None, None) == E_OK   # M = 0
    assert e(p, p, 10, 256, None, 4, p, p, None) == E_NULL             # ids
    assert e(p, p, 10, 256, p, 4, None, None, None) == E_NULL          # no output
    assert e(p, p, 10, 256, p, 4, m, None, None) == E_ALIGN            # out 16-byte
    ae = L.fv5b_head_argmax_embed
    assert ae(p, p, 100, 256, p, 1, p, p, None, p, p, p, 10, 384, p, None, None) == E_SHAPE   # Ke % 256
    assert ae(p, p, 100, 256, p, 1, p, p, None, p, p, p, 0, 256, p, None, None) == E_SHAPE    # Ve = 0
    assert ae(p, p, 100, 256, p, 1, p, p, None, p, None, p, 10, 256, p, None, None) == E_NULL  # E
    assert ae(p, p, 100, 256, p, 1, p, p, None, p, p, p, 10, 256, None, None, None) == E_NULL  # no output
    assert ae(p, p, 100, 256, p, 1, p, p, None, p, m, p, 10, 256, p, None, None) == E_ALIGN    # E 16-byte


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tw, "_lib", None)
    monkeypatch.setattr(tw, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        tw.lib()


def _steps(*specs):
    """ctypes array of tern_chain_step from (packed, N, K, x, x_from, y) tuples of ints/None."""
    arr = (tw.TernChainStep * len(specs))()
    for i, sp in enumerate(specs):
        arr[i] = tw.TernChainStep(*sp)
    return arr


def test_chain_workspace_bytes():
    L = tw.lib()
    a = (0x10000, 4096, 4096, 0x20000, -1, 0x30000)
    b = (0x10000, 6144, 4096, None, 0, 0x40000)          # reads step 0's output
    c = (0x10000, 1000, 4096, None, 1, 0x50000)          # reads step 1's output
    assert L.tern_chain_workspace_bytes(_steps(a), 1) == 4096 + 256            # plan only
    # plan 3 x 64 B -> 4352; hand-off of step 0: 2048 words x 8 B; of step 1: 3072 x 8 B
    assert L.tern_chain_workspace_bytes(_steps(a, b, c), 3) == 4352 + 16384 + 24576
    assert L.tern_chain_workspace_bytes(_steps(a, b), 0) == 4096
    assert L.tern_chain_workspace_bytes(_steps(a, (0x10000, 16, 512, None, 1, 0x40000)), 2) == -1  # not earlier
    assert L.tern_chain_workspace_bytes(_steps(a), -1) == -1
    assert L.tern_chain_workspace_bytes(None, 1) == -1


def test_chain_plan_rejects_bad_steps_before_any_device_call():
    L = tw.lib()
    ws, nb = ctypes.c_void_p(0x1000000), 1 << 22
    good = (0x10000, 4096, 4096, 0x20000, -1, 0x30000)
    assert L.tern_chain_plan(_steps(good), 1, None, nb, None) == E_NULL
    assert L.tern_chain_plan(None, 1, ws, nb, None) == E_NULL
    assert L.tern_chain_plan(_steps(good), 1, ctypes.c_void_p(0x1000010), nb, None) == E_ALIGN   # 256-byte
    assert L.tern_chain_plan(_steps(good), 1, ws, 4096 + 255, None) == E_SHAPE                   # too small
    assert L.tern_chain_plan(_steps(good), -1, ws, nb, None) == E_SHAPE
    assert L.tern_chain_plan(_steps(good), 4096, ws, nb, None) == E_SHAPE
    bad = [(0x10000, 4096, 640, 0x20000, -1, 0x30000),       # K % 512
           (0x10000, 4096, 256, 0x20000, -1, 0x30000),       # K < 512
           (0x10000, 4096, 16896, 0x20000, -1, 0x30000),     # K > 16384
           (0x10000, 0, 4096, 0x20000, -1, 0x30000),         # N < 1
           (0x10000, 64, 4096, None, 1, 0x70000),            # x_from not earlier
           (0x10000, 64, 8192, None, 0, 0x70000),            # K > N of the producer
           (0x10000, 64, 4096, None, -2, 0x70000)]
    for st in bad:
        assert L.tern_chain_plan(_steps(good, st), 2, ws, nb, None) == E_SHAPE, st
    assert L.tern_chain_plan(_steps((None, 16, 512, 0x20000, -1, 0x30000)), 1, ws, nb, None) == E_NULL
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, None, -1, 0x30000)), 1, ws, nb, None) == E_NULL
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, 0x20000, -1, None)), 1, ws, nb, None) == E_NULL
    assert L.tern_chain_plan(_steps((0x10008, 16, 512, 0x20000, -1, 0x30000)), 1, ws, nb, None) == E_ALIGN
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, 0x20008, -1, 0x30000)), 1, ws, nb, None) == E_ALIGN
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, 0x20000, -1, 0x30002)), 1, ws, nb, None) == E_ALIGN
    # outputs may not overlap inputs, packed weights or each other
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, 0x20000, -1, 0x20010)), 1, ws, nb, None) == E_SHAPE
    assert L.tern_chain_plan(_steps((0x10000, 16, 512, 0x20000, -1, 0x10100)), 1, ws, nb, None) == E_SHAPE
    assert L.tern_chain_plan(_steps(good, (0x10000, 16, 512, 0x60000, -1, 0x30020)), 2, ws, nb, None) == E_SHAPE
    assert L.tern_chain_plan(_steps(good, (0x10000, 16, 512, 0x30000, -1, 0x60000)), 2, ws, nb, None) == E_SHAPE


def test_chain_run_argument_errors():
    L = tw.lib()
    assert L.tern_gemv_chain(None, 1, None) == E_NULL
    assert L.tern_gemv_chain(ctypes.c_void_p(0x100010), 1, None) == E_ALIGN
    assert L.tern_gemv_chain(ctypes.c_void_p(0x100000), -1, None) == E_SHAPE
    assert L.tern_gemv_chain(ctypes.c_void_p(0x100000), 0, None) == E_OK


def test_mfma_peak_probe_validation():
    """The matrix-core probe's operation count and its argument checks (no device call)."""
    L = tw.lib()
    assert L.tern_mfma_peak_ops(0, 1000, 1024) == 2.0 * 16 * 16 * 64 * 1000 * 8 * 4 * 1024
    assert L.tern_mfma_peak_ops(1, 10, 3) == 2.0 * 16 * 16 * 32 * 10 * 8 * 4 * 3
    assert L.tern_mfma_peak_ops(2, 10, 3) == -1.0
    assert L.tern_mfma_peak_sink_bytes(5) == 5 * 256 * 16
    assert L.tern_mfma_peak(2, 10, 1, ALIGNED, None) == E_SHAPE
    assert L.tern_mfma_peak(0, 10, 0, ALIGNED, None) == E_SHAPE
    assert L.tern_mfma_peak(0, -1, 1, ALIGNED, None) == E_SHAPE
    assert L.tern_mfma_peak(0, 10, 1, None, None) == E_NULL
    assert L.tern_mfma_peak(0, 10, 1, MISALIGNED, None) == E_ALIGN


def test_launch_probe_validation():
    """The launch-floor / read probe's argument checks (no device call)."""
    L = tw.lib()
    assert L.tern_launch_probe(4, 1, ALIGNED, 16, ALIGNED, None) == E_SHAPE
    assert L.tern_launch_probe(-1, 1, ALIGNED, 16, ALIGNED, None) == E_SHAPE
    assert L.tern_launch_probe(0, 0, None, 0, None, None) == E_SHAPE
    assert L.tern_launch_probe(1, 1, None, 0, None, None) == E_NULL
    assert L.tern_launch_probe(2, 1, None, 16, ALIGNED, None) == E_NULL
    assert L.tern_launch_probe(3, 1, MISALIGNED, 16, ALIGNED, None) == E_ALIGN
    assert L.tern_launch_probe(3, 1, ALIGNED, 0, ALIGNED, None) == E_SHAPE
    assert L.tern_launch_probe(2, 1, ALIGNED, 24, ALIGNED, None) == E_SHAPE


def test_head_argmax_noalloc_validation():
    """The allocation-free head argmax rejects, on the host, a head whose keys
    exceed the library's 2 MiB array, and bad shapes or pointers like
    i8_head_argmax does."""
    L = tw.lib()
    p = ALIGNED
    assert L.i8_head_argmax_noalloc(p, p, 16 * 262144 + 16, 128, p, 1, p, p, None, None) == E_SHAPE
    assert L.i8_head_argmax_noalloc(p, p, 16 * 16384 + 16, 128, p, 16, p, p, None, None) == E_SHAPE
    assert L.i8_head_argmax_noalloc(p, p, 100, 96, p, 1, p, p, None, None) == E_SHAPE       # K % 128
    assert L.i8_head_argmax_noalloc(p, p, 100, 128, p, 17, p, p, None, None) == E_SHAPE     # M > 16
    assert L.i8_head_argmax_noalloc(p, p, 100, 128, p, 1, None, p, None, None) == E_NULL
    assert L.i8_head_argmax_noalloc(p, p, 100, 128, MISALIGNED, 1, p, p, None, None) == E_ALIGN


def test_packed_head_sizes_and_argument_errors():
    L = tw.lib()
    p, m = ALIGNED, MISALIGNED
    assert tw.i8_head_packed_bytes(151936, 4096) == 151936 * 4096          # 151936 = 2374 * 64
    assert tw.i8_head_packed_bytes(70, 256) == 2 * 64 * 256
    assert tw.i8_head_packed_bytes(1, 128) == 64 * 128
    for v, k in ((0, 128), (100, 96), (100, 0), (100, 64), (1 << 33, 128), (16, (1 << 20) + 128)):
        assert tw.i8_head_packed_bytes(v, k) == -1, (v, k)
    assert L.i8_head_pack(p, 100, 96, p, None) == E_SHAPE
    assert L.i8_head_pack(p, 0, 128, p, None) == E_SHAPE
    assert L.i8_head_pack(None, 100, 128, p, None) == E_NULL
    assert L.i8_head_pack(p, 100, 128, None, None) == E_NULL
    assert L.i8_head_pack(m, 100, 128, p, None) == E_ALIGN
    assert L.i8_head_pack(p, 100, 128, m, None) == E_ALIGN
    g, gi = L.i8_head_gemv_packed, L.i8_head_gemv_packed_i8
    assert g(p, p, 100, 96, p, 1, p, None) == E_SHAPE                      # K % 128
    assert g(p, p, 0, 128, p, 1, p, None) == E_SHAPE                       # V = 0
    assert g(p, p, 100, 128, p, 0, p, None) == E_SHAPE                     # M = 0
    assert g(p, p, 100, 128, p, 17, p, None) == E_SHAPE                    # M > 16
    assert g(p, p, 100, 8192, p, 16, p, None) == E_SHAPE                   # bf16 x of 16 x 8192 exceeds LDS
    assert gi(p, p, 100, 8192, p, p, 16, p, None, None) != E_SHAPE         # int8 x of 16 x 8192 fits ...
    assert gi(p, p, 100, 8192, p, None, 16, p, None, None) == E_NULL       # ... (s_x missing here)
    assert gi(p, p, 100, 16384, p, p, 16, p, None, None) == E_SHAPE        # 16 x 16384 int8 does not
    assert g(None, p, 100, 128, p, 1, p, None) == E_NULL
    assert g(p, None, 100, 128, p, 1, p, None) == E_NULL
    assert g(p, p, 100, 128, None, 1, p, None) == E_NULL
    assert g(p, p, 100, 128, p, 1, None, None) == E_NULL
    assert g(m, p, 100, 128, p, 1, p, None) == E_ALIGN
    assert g(p, p, 100, 128, m, 1, p, None) == E_ALIGN
    assert g(p, p, 100, 128, p, 1, ctypes.c_void_p(0x10002), None) == E_ALIGN   # logits
    assert gi(p, p, 100, 128, m, p, 1, p, None, None) == E_ALIGN
    assert gi(p, p, 100, 128, p, p, 1, p, ctypes.c_void_p(0x10002), None) == E_ALIGN   # acc_dbg


def test_packed_head_argmax_argument_errors():
    L = tw.lib()
    p, m = ALIGNED, MISALIGNED
    f, fi = L.i8_head_argmax_packed, L.i8_head_argmax_packed_i8
    assert f(p, p, 100, 96, p, 1, p, p, None, p, None) == E_SHAPE          # K % 128
    assert f(p, p, 0, 128, p, 1, p, p, None, p, None) == E_SHAPE           # V = 0
    assert f(p, p, 100, 128, p, 0, p, p, None, p, None) == E_SHAPE         # M = 0
    assert f(p, p, 100, 128, p, 17, p, p, None, p, None) == E_SHAPE        # M > 16
    assert f(p, p, 100, 8192, p, 16, p, p, None, p, None) == E_SHAPE       # bf16 x exceeds LDS
    assert fi(p, p, 100, 8192, p, None, 16, p, p, None, p, None) == E_NULL  # int8 fits; s_x missing
    assert f(p, p, 100, 128, p, 1, p, p, None, None, None) == E_NULL       # workspace
    assert f(None, p, 100, 128, p, 1, p, p, None, p, None) == E_NULL
    assert f(p, p, 100, 128, p, 1, None, p, None, p, None) == E_NULL       # idx
    assert f(m, p, 100, 128, p, 1, p, p, None, p, None) == E_ALIGN
    assert f(p, p, 100, 128, p, 1, p, p, ctypes.c_void_p(0x10002), p, None) == E_ALIGN   # logits
    assert fi(p, p, 100, 128, p, p, 1, p, p, None, ctypes.c_void_p(0x10004), None) == E_ALIGN   # workspace % 8


def test_fv5b_packed_head_argument_errors():
    L = tw.lib()
    p, m = ALIGNED, MISALIGNED
    g, gi = L.fv5b_head_gemv_packed, L.fv5b_head_gemv_packed_i8
    f, fi = L.fv5b_head_argmax_packed, L.fv5b_head_argmax_packed_i8
    assert g(p, p, 100, 128, p, 1, p, None) == E_SHAPE                     # K % 256
    assert g(p, p, 0, 256, p, 1, p, None) == E_SHAPE
    assert g(p, p, 100, 256, p, 17, p, None) == E_SHAPE
    assert g(p, p, 100, 8192, p, 16, p, None) == E_SHAPE                   # bf16 x exceeds LDS
    assert g(None, p, 100, 256, p, 1, p, None) == E_NULL
    assert g(p, None, 100, 256, p, 1, p, None) == E_NULL
    assert g(m, p, 100, 256, p, 1, p, None) == E_ALIGN
    assert gi(p, p, 100, 256, p, None, 1, p, None, None) == E_NULL         # s_x
    assert gi(p, p, 100, 256, p, p, 1, p, ctypes.c_void_p(0x10002), None) == E_ALIGN   # acc_dbg
    assert f(p, p, 100, 128, p, 1, p, p, None, p, None) == E_SHAPE
    assert f(p, p, 100, 256, p, 1, None, p, None, p, None) == E_NULL       # idx
    assert f(p, p, 100, 256, p, 1, p, p, None, None, None) == E_NULL       # workspace
    assert fi(p, p, 100, 256, p, p, 1, p, p, None, ctypes.c_void_p(0x10004), None) == E_ALIGN
