"""Pins of the oracle's dense W8A8 projection.

* identity weight: W = I gives code 0x7E on the diagonal and s_w = 1/448, so the
  projection returns the dequantised activation (up to fp32 rounding of s_w * 448);
* numpy matmul on operands dequantised independently (torch's e4m3 decode) at
  M = 1, 16, 300 -- the shapes of FreeToken PR #389's "Testing" section;
* the per-tensor weight quantiser keeps the weight within e4m3 tolerance (the PR's
  "loader round trip within e4m3 tolerance");
* row-wise variant: numpy matmul with each row's scale; equal row scales give the
  per-tensor projection; scaling one row's scale scales that output row only; brute force
  (Python float loops) on a tiny case;
* block-128 variant: the same sum taken as scaled per-group partial products; uniform
  scales reduce it to the row-wise projection; brute force across a block boundary.
"""

import numpy as np
import pytest
import torch

from oracle.dense import (dense_w8a8, dense_w8a8_entries, dense_w8a8_rowwise,
                          dense_w8a8_rowwise_entries, quantize_weight)
from oracle.quant import quant_row_bf16, quant_tensor_bf16
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


@pytest.mark.parametrize("M", [1, 16, 300])
def test_rowwise_vs_matmul_and_per_tensor(M):
    c = CONFIGS["dense_w8a8"]
    inp = dense_inputs(c, M=M)
    w = inp["w_qkv"][:64, :512]
    x = inp["x"][:, :512]
    wq, sw = quantize_weight(w)
    qa, sa = quant_row_bf16(x)
    y, b = dense_w8a8_rowwise(qa, sa, wq, sw, with_bound=True)
    ref = np.matmul(DEC[qa] * sa.astype(np.float64)[:, None], (DEC[wq] * float(sw)).T)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    rows = np.arange(M) % M
    cols = np.arange(M) % 64
    ye, be = dense_w8a8_rowwise_entries(qa, sa, wq, sw, rows, cols)
    assert np.allclose(ye, ref[rows, cols], rtol=1e-12, atol=1e-12)
    assert np.all(b >= np.abs(y) - 1e-12)
    # equal row scales: the per-tensor projection
    s0 = np.float32(0.0123)
    assert np.array_equal(dense_w8a8_rowwise(qa, np.full(M, s0, np.float32), wq, sw),
                          dense_w8a8(qa, s0, wq, sw))
    # one row's scale doubled: that output row doubles, the others stay
    s2 = sa.copy()
    s2[M // 2] *= 2
    y2 = dense_w8a8_rowwise(qa, s2, wq, sw)
    assert np.array_equal(y2[M // 2], 2 * y[M // 2])
    assert np.array_equal(np.delete(y2, M // 2, 0), np.delete(y, M // 2, 0))


def test_rowwise_brute_force():
    rng = np.random.default_rng(5)
    qa = rng.integers(0, 256, (3, 128)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0  # no NaN codes
    qw = rng.integers(0, 256, (5, 128)).astype(np.uint8)
    qw[(qw & 0x7F) == 0x7F] = 0
    sa = np.float32([0.5, 3.0, 1e-3])
    sw = np.float32(0.25)
    y = dense_w8a8_rowwise(qa, sa, qw, sw)
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for k in range(128):
                acc += float(DEC[qa[m, k]]) * float(DEC[qw[n, k]])
            assert abs(y[m, n] - float(sa[m]) * float(sw) * acc) <= 1e-12 * max(1.0, abs(acc))


def _block_case(M, N, K, seed):
    from oracle.quant import quant_block128_bf16, quant_group_bf16
    rng = np.random.default_rng(seed)
    x = bf16_bits_from_f32((rng.standard_normal((M, K)) * rng.uniform(0.1, 10, (M, 1))).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02 * rng.uniform(0.2, 5, (N, 1))).astype(np.float32))
    qa, sa = quant_group_bf16(x)
    qw, sw = quant_block128_bf16(w)
    return qa, sa, qw, sw


def test_block_gemm_group_partials():
    """Block-128 variant against a different order of the same sum: per-K-group partial
    products of the decoded codes (torch's e4m3 decode), each scaled by its row's group
    scale and its column's block scale, then summed over the groups."""
    from oracle.dense import block_gemm, block_gemm_entries
    M, N, K = 37, 200, 384
    qa, sa, qw, sw = _block_case(M, N, K, 3)
    y, b = block_gemm(qa, sa, qw, sw, with_bound=True)
    ref = np.zeros((M, N))
    for g in range(K // 128):
        part = DEC[qa[:, 128 * g:128 * (g + 1)]] @ DEC[qw[:, 128 * g:128 * (g + 1)]].T
        ref += part * sa[:, g:g + 1].astype(np.float64) * np.repeat(sw[:, g].astype(np.float64), 128)[:N][None, :]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)
    rows = np.arange(50) % M
    cols = (np.arange(50) * 7) % N
    ye, be = block_gemm_entries(qa, sa, qw, sw, rows, cols)
    assert np.allclose(ye, ref[rows, cols], rtol=1e-12, atol=1e-14)
    assert np.all(b >= np.abs(y) - 1e-12)


def test_block_gemm_uniform_scales_is_rowwise():
    from oracle.dense import block_gemm
    M, N, K = 9, 256, 256
    qa, _, qw, _ = _block_case(M, N, K, 4)
    sa_row = np.float32([0.5, 2, 3, 1e-3, 7, 0.25, 1, 1, 4])
    sa = np.repeat(sa_row[:, None], K // 128, axis=1)
    sw = np.full((2, 2), np.float32(0.125))
    assert np.allclose(block_gemm(qa, sa, qw, sw), dense_w8a8_rowwise(qa, sa_row, qw, np.float32(0.125)),
                       rtol=1e-13, atol=0)


def test_block_gemm_brute_force():
    from oracle.dense import block_gemm
    M, N, K = 2, 130, 256
    qa, sa, qw, sw = _block_case(M, N, K, 5)
    y = block_gemm(qa, sa, qw, sw)
    for m in range(M):
        for n in (0, 1, 127, 128, 129):
            acc = 0.0
            for k in range(K):
                acc += float(DEC[qa[m, k]]) * float(sa[m, k // 128]) * float(DEC[qw[n, k]]) * float(sw[n // 128, k // 128])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
