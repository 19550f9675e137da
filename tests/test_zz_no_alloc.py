"""The allocation-free head argmax (i8_head_argmax_noalloc) through the C ABI
against the workspace entry point (i8_head_argmax) it shares its kernels
with: index, value and logits bit for bit, on two calls in a row, the
second with a smaller input (the library's key array keeps the first call's
keys, which the second must not see)."""
import ctypes

import numpy as np
import pytest

from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(v, k, m, seed):
    import torch
    rng = np.random.default_rng(seed)
    w, rs = synth.gen_head(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    return (torch.from_numpy(w).cuda(), torch.from_numpy(rs).cuda(),
            torch.from_numpy(x.view(np.int16)).cuda())


def _noalloc(L, W, rs, x, logits):
    import torch
    v, k = W.shape
    m = x.shape[0]
    idx = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((m,), -7.0, dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rc = L.i8_head_argmax_noalloc(p(W), p(rs), v, k, p(x), m, p(idx), p(val), p(logits), s)
    assert rc == 0, L.tern_strerror(rc)
    return idx, val


def test_noalloc_matches_workspace_entry_point():
    import torch
    import ternary_weight_decode_amd as tw
    L = tw.lib()
    # first the full 8B head at M = 3, then a smaller head (fewer row tiles, M = 1)
    for (v, k, m, seed) in [(151936, 4096, 3, 31), (20011, 1024, 1, 32)]:
        W, rs, x = _inputs(v, k, m, seed)
        lg_a = torch.empty((m, v), dtype=torch.float32, device="cuda")
        lg_b = torch.full((m, v), 5.0, dtype=torch.float32, device="cuda")
        idx_a, val_a = tw.i8_head_argmax(W, rs, x, logits=lg_a)
        idx_b, val_b = _noalloc(L, W, rs, x, lg_b)
        torch.cuda.synchronize()
        assert np.array_equal(idx_b.cpu().numpy(), idx_a.cpu().numpy())
        assert np.array_equal(val_b.cpu().numpy().view(np.uint32), val_a.cpu().numpy().view(np.uint32))
        assert np.array_equal(lg_b.cpu().numpy().view(np.uint32), lg_a.cpu().numpy().view(np.uint32))
        # and the choice is the greedy argmax of those logits (lowest index among equal values)
        lg = lg_a.cpu().numpy()
        assert np.array_equal(idx_a.cpu().numpy(), np.argmax(lg + np.float32(0.0), axis=1).astype(np.int32))


def test_noalloc_without_logits_and_limit():
    import torch
    import ternary_weight_decode_amd as tw
    L = tw.lib()
    W, rs, x = _inputs(4099, 2048, 16, 33)
    idx_a, val_a = tw.i8_head_argmax(W, rs, x)
    idx_b, val_b = _noalloc(L, W, rs, x, None)
    torch.cuda.synchronize()
    assert np.array_equal(idx_b.cpu().numpy(), idx_a.cpu().numpy())
    assert np.array_equal(val_b.cpu().numpy().view(np.uint32), val_a.cpu().numpy().view(np.uint32))
    # beyond the key array (ceil(V/16) * M > 262144): rejected on the host, nothing launched
    p = ctypes.c_void_p(W.data_ptr())
    assert L.i8_head_argmax_noalloc(p, p, 16 * 262144 + 16, 128, p, 1, p, p, None, None) == 2
