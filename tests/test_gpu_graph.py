"""The library's calls inside a captured hipGraph (the benchmark replays the
token as one): a graph holding every decode-path call is replayed several
times, with the program's own eager work and synchronisations between the
replays, and every replay must reproduce the eager results bit for bit (all
kernels are deterministic).  The eager results are tied to the oracle."""
import numpy as np
import pytest

import oracle
from oracle import fv5, fv5b
from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tw():
    import torch
    import ternary_weight_decode_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def test_decode_calls_replay_in_a_graph(tw):
    import torch
    rng = np.random.default_rng(21)
    n, k = 6144, 4096
    t = synth.gen_ternary(rng, n, k)
    s = synth.gen_scales(rng, n, k // 128)
    packed = tw.tern_pack(dev(t), dev(s))
    lv = synth.gen_levels5(rng, 4096, k)
    lo, hi = synth.gen_scales5(rng, 4096, k // 256)
    p5 = tw.tern5_pack(dev(lv), dev(lo), dev(hi))
    v = 20000
    w, rs = synth.gen_head(rng, rng, v, k)
    wb, sb = synth.gen_head_blocks(rng, rng, v, k)
    W, RS, WB, SB = dev(w), dev(rs), dev(wb), dev(sb)
    x1 = dev(synth.gen_x_bf16(rng, 1, k))
    x8 = dev(synth.gen_x_bf16(rng, 8, k))
    ids = dev(np.array([5, 19999, 0, 123], np.int32))
    # prefill: 300 activation rows; the 512-row weight gives a small grid, so K is split in
    # two halves (clear, atomic partial sums, row scaling), the 6144-row one is not
    n2, mp = 512, 300
    t2 = synth.gen_ternary(rng, n2, k)
    s2 = synth.gen_scales(rng, n2, k // 128)
    packed2 = tw.tern_pack(dev(t2), dev(s2))
    xp = dev(synth.gen_x_bf16(rng, mp, k))
    assert tw.tern_prefill_config(n2, k, mp)["split"] == 1 and tw.tern_prefill_config(n, k, mp)["split"] == 0
    ws = tw.i8_head_argmax_workspace(v, 8)
    ws_b = tw.i8_head_argmax_workspace(v, 1)

    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    out = {
        "q": torch.empty((8, k), dtype=torch.int8, device="cuda"), "sx": f32(8),
        "y1": f32(1, n), "y8": f32(8, n), "y8i": f32(8, n), "y5": f32(1, 4096), "y5i": f32(8, 4096),
        "idx": torch.empty(8, dtype=torch.int32, device="cuda"), "val": f32(8), "logits": f32(8, v),
        "idxb": torch.empty(1, dtype=torch.int32, device="cuda"), "valb": f32(1),
        "emb": f32(4, k), "embh": torch.empty((4, k), dtype=torch.bfloat16, device="cuda"),
        "qp": torch.empty((mp, k), dtype=torch.int8, device="cuda"), "sxp": f32(mp),
        "yp": f32(mp, n2), "yp2": f32(mp, n),
    }

    def step():
        tw.tern_quantize_i8(x8, q=out["q"], s_x=out["sx"])
        tw.tern_gemv(packed, n, k, x1, y=out["y1"])
        tw.tern_gemv(packed, n, k, x8, y=out["y8"])
        tw.tern_gemv_i8(packed, n, k, out["q"], out["sx"], y=out["y8i"])
        tw.tern5_gemv(p5, 4096, k, x1, y=out["y5"])
        tw.tern5_gemv_i8(p5, 4096, k, out["q"], out["sx"], y=out["y5i"])
        i, vv = tw.i8_head_argmax_i8(W, RS, out["q"], out["sx"], workspace=ws, logits=out["logits"])
        out["idx"].copy_(i)
        out["val"].copy_(vv)
        i, vv = tw.fv5b_head_argmax(WB, SB, x1, workspace=ws_b)
        out["idxb"].copy_(i)
        out["valb"].copy_(vv)
        tw.fv5b_embed(WB, SB, ids, out=out["emb"], out_bf16=out["embh"])
        tw.tern_quantize_i8(xp, q=out["qp"], s_x=out["sxp"])
        tw.tern_gemm_prefill(packed2, n2, k, out["qp"], out["sxp"], y=out["yp"])
        tw.tern_gemm_prefill(packed, n, k, out["qp"], out["sxp"], y=out["yp2"])

    step()
    torch.cuda.synchronize()
    eager = {key: t_.clone() for key, t_ in out.items()}

    # the eager results against the oracle
    q, sx = eager["q"].cpu().numpy(), eager["sx"].cpu().numpy()
    x8_bits = x8.view(torch.int16).cpu().numpy().view(np.uint16)
    q0, sx0 = oracle.quantize_i8(x8_bits)
    assert np.array_equal(q, q0) and np.array_equal(sx, sx0)
    y64, _ = oracle.gemv_bf16(oracle.pack(t, s), n, k, x1.view(torch.int16).cpu().numpy().view(np.uint16))
    assert oracle.rel_l2(eager["y1"].cpu().numpy(), y64) < 1e-5
    acc, _, _ = oracle.head_i8(w, rs, q0, sx0)
    i0, v0 = oracle.greedy_argmax(oracle.head_i8_logits_f32(acc, rs, sx0))
    assert np.array_equal(eager["idx"].cpu().numpy(), i0)
    _, y5i, _ = fv5.gemv_i8_levels(lv, lo, hi, q0, sx0)
    assert oracle.rel_l2(eager["y5i"].cpu().numpy(), y5i) < 1e-5
    emb = fv5b.embed_f32(wb, sb, ids.cpu().numpy())
    assert np.array_equal(eager["emb"].cpu().numpy(), emb)
    qp0, sxp0 = oracle.quantize_i8(xp.view(torch.int16).cpu().numpy().view(np.uint16))
    _, yp64, _ = oracle.tern_i8(oracle.pack(t2, s2), n2, k, qp0, sxp0, want_acc=False)
    assert oracle.rel_l2(eager["yp"].cpu().numpy(), yp64) < 1e-5
    rows = np.arange(0, n, 97)
    _, yq64, _ = oracle.tern_i8(oracle.pack(t[rows], s[rows]), len(rows), k, qp0, sxp0, want_acc=False)
    assert oracle.rel_l2(eager["yp2"].cpu().numpy()[:, rows], yq64) < 1e-5

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t_ in out.values():
            t_.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, t_ in out.items():
            a, b = t_.cpu(), eager[key].cpu()
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (rep, key)
