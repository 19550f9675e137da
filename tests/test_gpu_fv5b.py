"""GPU parity of the block-scaled int8 head and the embedding rows
(FV5B-style) against the CPU oracle (oracle/fv5b.py) on the same seeded
inputs: int8 block sums and embedding rows (fp32 and bf16) bit for bit,
logits within a relative L2 error of 1e-5 of the fp64 oracle, and the fused
greedy argmax a valid maximum of the oracle's logits (the oracle's choice
wherever the top two differ by more than the fp32 error)."""
import numpy as np
import pytest

import oracle
from oracle import fv5b
from ternary_weight_decode_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


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


def host(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def inputs(v, k, m, seed):
    rng = np.random.default_rng(seed)
    w, s = synth.gen_head_blocks(rng, rng, v, k)
    x = synth.gen_x_bf16(rng, m, k)
    q = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.005, 0.05, m).astype(np.float32)
    return w, s, x, q, sx


def test_golden_head_and_embedding(tw):
    from test_oracle_fv5b import golden_head_acts, golden_tensors, read_golden
    ex = read_golden()
    e = ex["head"]
    w, s = golden_tensors(e)
    x, q, sx = golden_head_acts(e["K"])
    assert host(tw.fv5b_head_gemv(dev(w), dev(s), dev(x)))[0].tolist() == e["y_bf16"]
    import torch
    acc = torch.empty((1, e["V"], e["K"] // 256), dtype=torch.int32, device="cuda")
    y = host(tw.fv5b_head_gemv_i8(dev(w), dev(s), dev(q), dev(sx), acc=acc))
    assert y[0].tolist() == e["y_i8"]
    assert {r: host(acc)[0, r].tolist() for r in e["acc"]} == e["acc"]
    e = ex["embed"]
    w, s = golden_tensors(e)
    f, b = tw.fv5b_embed(dev(w), dev(s), dev(np.array(e["ids"], np.int32)))
    f, b = host(f), host(b).view(np.uint16)
    want_f = np.zeros(f.shape, np.uint32)
    want_b = np.zeros(b.shape, np.uint16)
    for (m, k, bits) in e["f32"]:
        want_f[m, k] = bits
    for (m, k, bits) in e["bf16"]:
        want_b[m, k] = bits
    assert np.array_equal(f.view(np.uint32), want_f) and np.array_equal(b, want_b)


HEAD = [(300, 512, 1), (5003, 1024, 3), (20000, 4096, 16), (151936, 4096, 1), (151936, 1024, 4)]


@pytest.mark.parametrize("v,k,m", HEAD)
def test_head_bf16(tw, v, k, m):
    w, s, x, _, _ = inputs(v, k, m, seed=v + k + m)
    y = host(tw.fv5b_head_gemv(dev(w), dev(s), dev(x)))
    y64, _ = fv5b.head_bf16(w, s, x)
    assert oracle.rel_l2(y, y64) < TOL


@pytest.mark.parametrize("v,k,m", HEAD)
def test_head_i8_block_sums_exact(tw, v, k, m):
    import torch
    w, s, _, q, sx = inputs(v, k, m, seed=2 * v + k + m)
    acc = torch.empty((m, v, k // 256), dtype=torch.int32, device="cuda")
    y = host(tw.fv5b_head_gemv_i8(dev(w), dev(s), dev(q), dev(sx), acc=acc))
    acc64, y64, _ = fv5b.head_i8(w, s, q, sx)
    assert np.array_equal(host(acc).astype(np.int64), acc64)
    assert oracle.rel_l2(y, y64) < TOL


def check_argmax(idx, val, y64):
    for r in range(y64.shape[0]):
        top = np.sort(y64[r])[::-1]
        tol = 1e-5 * np.abs(y64[r]).max()
        assert y64[r, idx[r]] >= top[0] - tol, (r, idx[r])
        assert abs(val[r] - y64[r, idx[r]]) <= tol
        if top[0] - top[1] > 2 * tol:
            assert idx[r] == int(np.argmax(y64[r]))


@pytest.mark.parametrize("v,k,m", [(300, 512, 1), (151936, 4096, 1), (20000, 4096, 16)])
def test_head_argmax_valid(tw, v, k, m):
    import torch
    w, s, x, q, sx = inputs(v, k, m, seed=3 * v + m)
    logits = torch.empty((m, v), dtype=torch.float32, device="cuda")
    idx, val = tw.fv5b_head_argmax(dev(w), dev(s), dev(x), logits=logits)
    y64, _ = fv5b.head_bf16(w, s, x)
    assert oracle.rel_l2(host(logits), y64) < TOL
    check_argmax(host(idx), host(val), y64)
    idx, val = tw.fv5b_head_argmax_i8(dev(w), dev(s), dev(q), dev(sx))
    _, y64i, _ = fv5b.head_i8(w, s, q, sx)
    check_argmax(host(idx), host(val), y64i)


def test_head_argmax_ties_take_the_lowest_row(tw):
    """Rows identical in W and S give identical logits: copies of the winning
    row at lower indices win, and a head of identical rows returns row 0."""
    v, k, m = 4099, 512, 2
    w, s, _, q, sx = inputs(v, k, m, seed=9)
    _, y64, _ = fv5b.head_i8(w, s, q, sx)
    win = np.argmax(y64, axis=1)
    w2, s2 = w.copy(), s.copy()
    for r, dup in zip(range(m), (17, 3001)):
        w2[dup], s2[dup] = w[win[r]], s[win[r]]
    idx, _ = tw.fv5b_head_argmax_i8(dev(w2), dev(s2), dev(q), dev(sx))
    _, y64b, _ = fv5b.head_i8(w2, s2, q, sx)
    want = [min(d, int(np.argmax(y64b[r]))) for r, d in zip(range(m), (17, 3001))]
    assert host(idx).tolist() == want
    same_w, same_s = np.repeat(w[:1], v, axis=0), np.repeat(s[:1], v, axis=0)
    idx, _ = tw.fv5b_head_argmax_i8(dev(same_w), dev(same_s), dev(q), dev(sx))
    assert host(idx).tolist() == [0, 0]


@pytest.mark.parametrize("v,k,m", [(1000, 256, 1), (151936, 4096, 7), (5000, 1024, 300)])
def test_embed_bit_exact(tw, v, k, m):
    rng = np.random.default_rng(v + m)
    w, s = synth.gen_head_blocks(rng, rng, v, k)
    ids = rng.integers(0, v, size=m).astype(np.int32)
    ids[::5] = ids[0]                          # repeated tokens
    if m > 2:
        ids[1], ids[2] = -1, v                 # outside [0, V): zero rows
    f, b = tw.fv5b_embed(dev(w), dev(s), dev(ids))
    assert np.array_equal(host(f).view(np.uint32), fv5b.embed_f32(w, s, ids).view(np.uint32))
    assert np.array_equal(host(b).view(np.uint16), fv5b.embed_bf16(w, s, ids))
    f_only, none = tw.fv5b_embed(dev(w), dev(s), dev(ids), bf16=False)
    assert none is None and np.array_equal(host(f_only), host(f))


def test_head_argmax_embed(tw):
    """Head + argmax + the chosen rows' embeddings in one call.  Each
    activation row gets a planted winner (a head row aligned with it), so the
    oracle's argmax is unambiguous; the gathered rows must equal the oracle's
    embedding of those indices bit for bit, and a table smaller than the
    winning index gives a zero row."""
    import torch
    v, k, m = 20000, 4096, 3
    rng = np.random.default_rng(77)
    w, s, x, _, _ = inputs(v, k, m, seed=78)
    winners = [17, 9001, 19999]
    xf = synth.bf16_bits_to_f32(x)
    for r, wi in enumerate(winners):
        w[wi] = np.clip(np.rint(100.0 * np.sign(xf[r])), -127, 127).astype(np.int8)
        s[wi] = 0.02
    y64, _ = fv5b.head_bf16(w, s, x)
    for r, wi in enumerate(winners):
        top = np.sort(y64[r])[::-1]
        assert int(np.argmax(y64[r])) == wi and top[0] - top[1] > 1e-3 * abs(top[0])
    ve, ke = 30000, 1024
    e, es = synth.gen_head_blocks(rng, rng, ve, ke)
    idx, val, emb, embh = tw.fv5b_head_argmax_embed(dev(w), dev(s), dev(x), dev(e), dev(es))
    assert host(idx).tolist() == winners
    want = fv5b.embed_f32(e, es, winners)
    assert np.array_equal(host(emb).view(np.uint32), want.view(np.uint32))
    assert np.array_equal(host(embh).view(np.uint16), fv5b.round_bf16(want))
    i2, v2 = tw.fv5b_head_argmax(dev(w), dev(s), dev(x))
    assert np.array_equal(host(i2), host(idx)) and np.array_equal(host(v2), host(val))
    # a table of 9001 rows: the first winner has a row, the others do not
    e_small, es_small = e[:9001].copy(), es[:9001].copy()
    _, _, emb2, _ = tw.fv5b_head_argmax_embed(dev(w), dev(s), dev(x), dev(e_small), dev(es_small), bf16=False)
    want2 = fv5b.embed_f32(e_small, es_small, winners)
    assert np.array_equal(host(emb2).view(np.uint32), want2.view(np.uint32))
    assert not want2[1:].any()
