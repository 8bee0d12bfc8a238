"""Pins of the oracle's dense W8A8 projection.

* identity weight: W = I gives code 0x7E on the diagonal and s_w = 1/448, so the
  projection returns the dequantised activation (up to fp32 rounding of s_w * 448);
* numpy matmul on operands dequantised independently (torch's e4m3 decode) at
  M = 1, 16, 300 -- the shapes of FreeToken PR #389's "Testing" section;
* the per-tensor weight quantiser keeps the weight within e4m3 tolerance (the PR's
  "loader round trip within e4m3 tolerance").
"""

import numpy as np
import pytest
import torch

from oracle.dense import dense_w8a8, dense_w8a8_entries, quantize_weight
from oracle.quant import quant_tensor_bf16
from synth import CONFIGS, bf16_bits_from_f32, dense_inputs, f32_from_bf16_bits

DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float64).numpy()


def test_identity_weight():
    K = 256
    w = bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    wq, sw = quantize_weight(w)
    assert np.all(np.diag(wq) == 0x7E) and np.all(wq[~np.eye(K, dtype=bool)] == 0)
    assert sw == np.float32(1.0) / np.float32(448.0)
    x = bf16_bits_from_f32(np.random.default_rng(0).standard_normal((5, K)).astype(np.float32))
    qa, blk = quant_tensor_bf16(x)
    y = dense_w8a8(qa, blk[2], wq, sw)
    assert np.allclose(y, DEC[qa] * blk[2], rtol=1e-6)


@pytest.mark.parametrize("M", [1, 16, 300])
def test_vs_matmul(M):
    c = CONFIGS["dense_w8a8"]
    inp = dense_inputs(c, M=M)
    w = inp["w_qkv"][:64, :512]
    x = inp["x"][:, :512]
    wq, sw = quantize_weight(w)
    qa, blk = quant_tensor_bf16(x)
    y, b = dense_w8a8(qa, blk[2], wq, sw, with_bound=True)
    ref = np.matmul(DEC[qa] * float(blk[2]), (DEC[wq] * float(sw)).T)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    rows = np.arange(M) % M
    cols = np.arange(M) % 64
    ye, be = dense_w8a8_entries(qa, blk[2], wq, sw, rows, cols)
    assert np.allclose(ye, ref[rows, cols], rtol=1e-12, atol=1e-12)
    assert np.all(b >= np.abs(y) - 1e-12)


def test_weight_round_trip_within_e4m3_tolerance():
    c = CONFIGS["dense_w8a8"]
    w = dense_inputs(c, M=1)["w_o"][:256]
    wq, sw = quantize_weight(w)
    wf = f32_from_bf16_bits(w).astype(np.float64)
    deq = DEC[wq] * float(sw)
    sub = np.abs(wf) < 2.0 ** -6 * float(sw)
    tol = np.where(sub, 2.0 ** -10 * float(sw), 2.0 ** -4 * np.abs(wf)) * (1 + 1e-6)
    assert np.all(np.abs(deq - wf) <= tol + 1e-30)
