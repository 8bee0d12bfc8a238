"""Pins of the oracle's grouped expert GEMM, SwiGLU + quant, combine and layer.

* grouped GEMM vs an fp64 pure-Python loop over (row, column, group, k) that extracts
  nibbles with its own bit operations and decodes e4m3 with torch;
* E=1, k=1 reduces to one dense GEMM (numpy matmul on separately dequantised operands);
* integer-valued operands with unit scales give exact integer results;
* SwiGLU: h(0) = 0 and silu against scipy's expit; combine: equal rows give the row back,
  k=1 with w=1 is a pure gather; the layer routes every (token, expert) pair exactly once.
"""

import numpy as np
import torch
from scipy.special import expit

from oracle.codec import e4m3_encode
from oracle.moe import combine, grouped_gemm, grouped_gemm_rows, moe_layer, swiglu
from oracle.quant import quant_group
from oracle.route import group_pairs
from synth import CONFIGS, moe_inputs

DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float64).numpy()


def _brute(a_codes, a_scales, w_packed, w_scales, offsets):
    R, K = a_codes.shape
    E, N, _ = w_packed.shape
    y = np.zeros((R, N))
    for e in range(E):
        for i in range(int(offsets[e]), int(offsets[e + 1])):
            for n in range(N):
                acc = 0.0
                for g in range(K // 128):
                    part = 0.0
                    for kk in range(g * 128, g * 128 + 128):
                        byte = int(w_packed[e, n, kk // 2])
                        nib = (byte >> 4) if kk % 2 else (byte & 15)
                        qv = nib - 16 if nib >= 8 else nib
                        part += DEC[a_codes[i, kk]] * qv
                    acc += float(a_scales[i, g]) * float(w_scales[e, n, g]) * part
                y[i, n] = acc
    return y


def _tiny(seed=0, R=12, K=256, N=6, E=3):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((R, K)).astype(np.float32)
    aq, as_ = quant_group(a)
    wp = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E, N, K // 128)).astype(np.float32)
    off = np.array([0, 5, 5, R], dtype=np.int32)  # expert 1 empty
    return aq, as_, wp, ws, off


def test_grouped_gemm_vs_triple_loop():
    aq, as_, wp, ws, off = _tiny()
    y, b = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    ref = _brute(aq, as_, wp, ws, off)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert np.all(b >= np.abs(y) - 1e-12)
    rows = np.array([0, 4, 5, 11])
    cols = np.array([0, 5, 2, 3])
    ys, bs = grouped_gemm_rows(aq, as_, wp, ws, off, rows, cols)
    assert np.allclose(ys, ref[rows, cols], rtol=1e-12, atol=1e-15)
    assert np.allclose(bs, b[rows, cols], rtol=1e-12)


def test_single_expert_is_dense_gemm():
    aq, as_, wp, ws, _ = _tiny(1, R=9, K=384, N=5, E=1)
    y = grouped_gemm(aq, as_, wp, ws, np.array([0, 9], np.int32))
    a = DEC[aq] * np.repeat(as_.astype(np.float64), 128, axis=1)
    lo = (wp & 15).astype(np.int64)
    hi = (wp >> 4).astype(np.int64)
    q = np.empty((5, 384), np.int64)
    q[:, 0::2] = lo[0]
    q[:, 1::2] = hi[0]
    q = np.where(q >= 8, q - 16, q)
    w = q * np.repeat(ws[0].astype(np.float64), 128, axis=1)
    assert np.allclose(y, np.matmul(a, w.T), rtol=1e-12, atol=1e-15)


def test_integer_operands_are_exact():
    rng = np.random.default_rng(2)
    ints = rng.integers(-8, 9, size=(6, 256)).astype(np.float64)
    aq = e4m3_encode(ints)
    as_ = np.ones((6, 2), np.float32)
    wp = rng.integers(0, 256, size=(2, 4, 128), dtype=np.uint8)
    ws = np.ones((2, 4, 2), np.float32)
    off = np.array([0, 2, 6], np.int32)
    y = grouped_gemm(aq, as_, wp, ws, off)
    assert np.array_equal(y, np.round(y))
    assert np.array_equal(y, _brute(aq, as_, wp, ws, off))


def test_swiglu_closed_forms():
    g = np.linspace(-20, 20, 101)
    u = np.linspace(3, -3, 101)
    h = swiglu(np.concatenate([g[:, None], u[:, None]], axis=1))[:, 0]
    assert np.allclose(h, g * expit(g) * u, rtol=1e-13, atol=1e-300)
    assert swiglu(np.zeros((1, 2)))[0, 0] == 0.0


def test_combine_special_cases():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((8, 5))
    # all k rows of each token equal -> out equals that row (weights sum to 1)
    T, k = 4, 2
    pos = np.array([0, 1, 2, 3, 4, 5, 6, 7])
    y_eq = np.repeat(y[::2], 2, axis=0)
    w = rng.uniform(0.1, 1, (T, k))
    w /= w.sum(axis=1, keepdims=True)
    assert np.allclose(combine(y_eq, pos, w), y[::2], rtol=1e-14)
    # k = 1, w = 1: a pure gather
    perm = rng.permutation(8)
    out = combine(y, perm, np.ones((8, 1)))
    assert np.array_equal(out, y[perm])


def test_layer_routes_every_pair_once():
    c = CONFIGS["moe_tiny"]
    inp = moe_inputs(c)
    r = moe_layer(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"],
                  inp["s_dn"], c.k)
    R = c.T * c.k
    pairs = set()
    for i, p in enumerate(r["sorted"]):
        t, j = divmod(int(p), c.k)
        e = int(r["ids"][t, j])
        assert r["offsets"][e] <= i < r["offsets"][e + 1]
        pairs.add((t, e))
    assert len(pairs) == R
    assert r["out"].shape == (c.T, c.H) and np.all(np.isfinite(r["out"]))
    assert np.array_equal(r["offsets"], group_pairs(r["ids"], c.E)[0])
