"""The FV5B-style head and embedding oracle (oracle/fv5b.py) pinned to
things other than itself: hand-derived examples, brute force, the per-row
head oracle (plain C) where the formats coincide, and the bf16 rounding's
ties."""
import os

import numpy as np

import oracle
from oracle import fv5b
from ternary_weight_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fv5b_examples.txt")


def read_golden():
    ex, cur = {}, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] in ("head", "embed"):
            cur = {"V": int(tok[2]), "K": int(tok[4]), "w": [], "s": {}, "acc": {}, "f32": [], "bf16": []}
            ex[tok[0]] = cur
        elif tok[0] == "w":
            cur["w"].append((int(tok[1]), int(tok[2]), int(tok[3])))
        elif tok[0] == "s":
            cur["s"][int(tok[1])] = [float(t) for t in tok[2:]]
        elif tok[0] in ("y_bf16", "y_i8"):
            cur[tok[0]] = [float(t) for t in tok[1:]]
        elif tok[0] == "acc":
            cur["acc"][int(tok[1])] = [int(t) for t in tok[2:]]
        elif tok[0] == "ids":
            cur["ids"] = [int(t) for t in tok[1:]]
        elif tok[0] in ("f32", "bf16"):
            cur[tok[0]].append((int(tok[1]), int(tok[2]), int(tok[3], 16)))
    return ex


def golden_tensors(e):
    v, k = e["V"], e["K"]
    w = np.zeros((v, k), np.int8)
    for (r, c, val) in e["w"]:
        w[r, c] = val
    s = np.zeros((v, k // 256), np.float32)
    for r, vals in e["s"].items():
        s[r] = vals
    return w, s


def golden_head_acts(k):
    kk = np.arange(k)
    x = synth.f32_to_bf16_bits((kk % 7 - 3).astype(np.float32)[None, :])
    q = (kk % 5 - 2).astype(np.int8)[None, :]
    return x, q, np.array([0.5], np.float32)


def test_golden_head():
    e = read_golden()["head"]
    w, s = golden_tensors(e)
    x, q, sx = golden_head_acts(e["K"])
    y64, _ = fv5b.head_bf16(w, s, x)
    assert y64[0].tolist() == e["y_bf16"]
    acc, y64i, _ = fv5b.head_i8(w, s, q, sx)
    for r, vals in e["acc"].items():
        assert acc[0, r].tolist() == vals
    assert y64i[0].tolist() == e["y_i8"]


def test_golden_embed():
    e = read_golden()["embed"]
    w, s = golden_tensors(e)
    f = fv5b.embed_f32(w, s, e["ids"])
    b = fv5b.embed_bf16(w, s, e["ids"])
    listed = {(m, k) for (m, k, _) in e["f32"]}
    for (m, k, bits) in e["f32"]:
        assert f[m:m + 1, k].view(np.uint32)[0] == bits, (m, k)
    for (m, k, bits) in e["bf16"]:
        assert b[m, k] == bits, (m, k)
    mask = np.ones(f.shape, bool)
    for (m, k) in listed:
        mask[m, k] = False
    assert not f[mask].any() and not b[mask].any()


def test_head_vs_brute_force():
    rng = np.random.default_rng(1)
    v, k, m = 5, 512, 2
    w = rng.integers(-127, 128, size=(v, k)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, (v, k // 256)).astype(np.float32)
    x = synth.gen_x_bf16(rng, m, k)
    q = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.01, 0.1, m).astype(np.float32)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    want = np.zeros((m, v))
    want_i = np.zeros((m, v))
    for mm in range(m):
        for vv in range(v):
            tot, tot_i = 0.0, 0.0
            for b in range(k // 256):
                part, part_i = 0.0, 0
                for kk in range(256 * b, 256 * b + 256):
                    part += float(w[vv, kk]) * xf[mm, kk]
                    part_i += int(w[vv, kk]) * int(q[mm, kk])
                tot += float(s[vv, b]) * part
                tot_i += float(s[vv, b]) * part_i
            want[mm, vv] = tot
            want_i[mm, vv] = float(sx[mm]) * tot_i
    y, _ = fv5b.head_bf16(w, s, x)
    _, yi, _ = fv5b.head_i8(w, s, q, sx)
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)
    assert np.allclose(yi, want_i, rtol=1e-13, atol=1e-13)


def test_reduces_to_the_per_row_head():
    """With every block of a row sharing one scale, the block-scaled head is
    the per-row-scaled int8 head (the plain C oracle); the int8 block sums
    add up to its exact per-row sums."""
    rng = np.random.default_rng(2)
    v, k, m = 300, 1024, 3
    w, rs = synth.gen_head(rng, rng, v, k)
    s = np.repeat(rs[:, None], k // 256, axis=1)
    x = synth.gen_x_bf16(rng, m, k)
    y, _ = fv5b.head_bf16(w, s, x)
    y_row, _ = oracle.head_bf16(w, rs, x)
    assert oracle.rel_l2(y, y_row) < 1e-13
    q = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.01, 0.1, m).astype(np.float32)
    acc, yi, _ = fv5b.head_i8(w, s, q, sx)
    acc_row, yi_row, _ = oracle.head_i8(w, rs, q, sx)
    assert np.array_equal(acc.sum(axis=2), acc_row.astype(np.int64))
    assert oracle.rel_l2(yi, yi_row) < 1e-13


def test_rows_subset_and_embed_matches_head_rows():
    rng = np.random.default_rng(3)
    v, k = 40, 768
    w = rng.integers(-127, 128, size=(v, k)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, (v, k // 256)).astype(np.float32)
    x = synth.gen_x_bf16(rng, 2, k)
    rows = [0, 17, 39]
    assert np.array_equal(fv5b.head_bf16(w, s, x, rows)[0], fv5b.head_bf16(w, s, x)[0][:, rows])
    # a one-hot activation picks one dequantized weight per row: the head's
    # column k equals the embedding rows' element k (exact products)
    kk = 300
    onehot = np.zeros((1, k), np.uint16)
    onehot[0, kk] = 0x3F80
    col = fv5b.head_bf16(w, s, onehot)[0][0]
    emb = fv5b.embed_f32(w, s, np.arange(v))
    assert np.array_equal(col.astype(np.float32), emb[:, kk])


def test_round_bf16_ties_and_signs():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8), -(1 + 3 * 2 ** -8),
                     0.0, -0.0, 2 ** -130], np.float32)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xBF80, 0xBF82, 0x0000, 0x8000, 0x0008], np.uint16)   # 2^-130: bf16 subnormal 8 * 2^-133
    assert np.array_equal(fv5b.round_bf16(vals), want)
    # against the neighbour definition on random values: the result is a
    # nearest bf16 and never farther than half a bf16 step
    rng = np.random.default_rng(4)
    f = (rng.standard_normal(100000) * 10.0).astype(np.float32)
    b = fv5b.round_bf16(f)
    back = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    step = np.abs((((b.astype(np.uint32) | 1) << 16).view(np.float32)).astype(np.float64)
                  - (((b.astype(np.uint32) & ~np.uint32(1)) << 16).view(np.float32)).astype(np.float64))
    assert (np.abs(back - f.astype(np.float64)) <= step / 2 + 1e-300).all()
