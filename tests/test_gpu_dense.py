"""fp8_dense_gemm (and the per-tensor quantiser feeding it) on the GPU vs the oracle,
and the row-wise variant fp8_dense_gemm_rowwise (FreeToken PR #389, "Limits").

Shapes: M = 1, 16, 300 (FreeToken PR #389, "Testing": the op against the dequantised
weight at M=1/16/300) and the full 2048 x 4096 x {6144, 4096} projections, sampled.
"""

import numpy as np
import pytest
import torch

from oracle.dense import (dense_w8a8, dense_w8a8_entries, dense_w8a8_rowwise,
                          dense_w8a8_rowwise_entries, quantize_weight)
from oracle.numeric import bf16_bits, round_bf16
from oracle.quant import quant_row_bf16, quant_tensor_bf16
from oracle.tol import check_close, gemm_bound
from synth import CONFIGS, bf16_bits_from_f32, dense_inputs
from tests.gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _gpu(x_bits, w_bits, out_dtype=torch.float32):
    import fp8_moe_prefill_amd as f
    wq, sw = f.quantize_weight(dev(w_bits))
    xq, blk = f.fp8_quant_act(dev(x_bits), 0)
    y = f.fp8_dense_gemm(xq, blk, wq, sw, out_dtype)
    torch.cuda.synchronize()
    return host(y), host(xq), host(blk), host(wq), host(sw)


@pytest.mark.parametrize("M", [1, 16, 300])
def test_small_m(M):
    inp = dense_inputs(CONFIGS["dense_w8a8"], M=M)
    w = inp["w_qkv"][:528]  # N = 528: a ragged last tile
    y, xq, blk, wq, sw = _gpu(inp["x"], w)
    rq, rblk = quant_tensor_bf16(inp["x"])
    rwq, rsw = quantize_weight(w)
    assert_bytes_equal(xq, rq, "activation codes")
    assert_bytes_equal(wq, rwq, "weight codes")
    assert sw[0] == rsw
    ref, b = dense_w8a8(rq, rblk[2], rwq, rsw, with_bound=True)
    check_close(y.astype(np.float64), ref, gemm_bound(b), f"dense M={M}")


def test_identity_weight():
    K = 512
    w = bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    x = bf16_bits_from_f32(np.random.default_rng(0).standard_normal((33, K)).astype(np.float32))
    y, xq, blk, wq, sw = _gpu(x, w)
    from oracle.codec import e4m3_decode
    ref = e4m3_decode(xq) * float(blk[2])
    assert np.allclose(y, ref, rtol=2e-7, atol=0)


def test_bf16_output_is_rounded_fp32_output():
    inp = dense_inputs(CONFIGS["dense_w8a8"], M=300)
    y32 = _gpu(inp["x"], inp["w_o"][:256], torch.float32)[0]
    y16 = _gpu(inp["x"], inp["w_o"][:256], torch.bfloat16)[0]
    assert_bytes_equal(y16, bf16_bits(round_bf16(y32.astype(np.float64))), "bf16 = RNE(fp32)")


@pytest.mark.parametrize("which", ["w_qkv", "w_o"])
def test_full_size_sampled(which):
    inp = dense_inputs(CONFIGS["dense_w8a8"])
    x = inp["x"] if which == "w_qkv" else inp["x_o"]
    y, xq, blk, wq, sw = _gpu(x, inp[which])
    rq, rblk = quant_tensor_bf16(x)
    assert_bytes_equal(xq, rq, "activation codes")
    rng = np.random.default_rng(5)
    rows = rng.integers(0, y.shape[0], 3000)
    cols = rng.integers(0, y.shape[1], 3000)
    ref, b = dense_w8a8_entries(rq, rblk[2], wq, sw[0], rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), f"dense {which}")


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("N,K", [(6656, 2560), (2560, 3072), (8192, 2560)])
def test_decode_shapes(M, N, K):
    """The decode shapes of FreeToken PR #389, "Why" (per-rank projections at M = 1, 8, 16):
    the small-M weight-streaming path, every output within the bound, bf16 = RNE(fp32)."""
    rng = np.random.default_rng(M * 7 + N + K)
    x = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    y, xq, blk, wq, sw = _gpu(x, w)
    rq, rblk = quant_tensor_bf16(x)
    rwq, rsw = quantize_weight(w)
    assert_bytes_equal(xq, rq, "activation codes")
    assert_bytes_equal(wq, rwq, "weight codes")
    ref, b = dense_w8a8(rq, rblk[2], rwq, rsw, with_bound=True)
    check_close(y, ref, gemm_bound(b), f"decode M={M} N={N} K={K}")
    yb = _gpu(x, w, torch.bfloat16)[0]
    assert_bytes_equal(yb, bf16_bits(round_bf16(y.astype(np.float64))), "bf16 = RNE(fp32)")


def _gpu_rowwise(x_bits, w_bits, out_dtype=torch.float32):
    import fp8_moe_prefill_amd as f
    wq, sw = f.quantize_weight(dev(w_bits))
    xq, sa = f.fp8_quant_act(dev(x_bits), f.QUANT_ROW)
    y = f.fp8_dense_gemm_rowwise(xq, sa, wq, sw, out_dtype)
    torch.cuda.synchronize()
    return host(y), host(xq), host(sa), host(wq), host(sw)


@pytest.mark.parametrize("M", [1, 8, 16, 300])
def test_rowwise_small_m(M):
    """Row-wise scales at M = 1 / 8 / 16 (the weight-streaming path) and 300 (tiles, ragged
    last row tile), N = 528 (ragged last column tile), on the outlier-channel activations."""
    inp = dense_inputs(CONFIGS["dense_w8a8"], M=M)
    w = inp["w_qkv"][:528]
    y, xq, sa, wq, sw = _gpu_rowwise(inp["x"], w)
    rq, rs = quant_row_bf16(inp["x"])
    assert_bytes_equal(xq, rq, "activation codes")
    assert_bytes_equal(sa.view(np.uint32), rs.view(np.uint32), "row scales")
    ref, b = dense_w8a8_rowwise(rq, rs, wq, sw[0], with_bound=True)
    check_close(y.astype(np.float64), ref, gemm_bound(b), f"rowwise M={M}")
    yb = _gpu_rowwise(inp["x"], w, torch.bfloat16)[0]
    assert_bytes_equal(yb, bf16_bits(round_bf16(y.astype(np.float64))), "bf16 = RNE(fp32)")


@pytest.mark.parametrize("which", ["w_qkv", "w_o"])
def test_rowwise_full_size_sampled(which):
    inp = dense_inputs(CONFIGS["dense_w8a8"])
    x = inp["x"] if which == "w_qkv" else inp["x_o"]
    y, xq, sa, wq, sw = _gpu_rowwise(x, inp[which])
    rq, rs = quant_row_bf16(x)
    assert_bytes_equal(xq, rq, "activation codes")
    assert_bytes_equal(sa.view(np.uint32), rs.view(np.uint32), "row scales")
    rng = np.random.default_rng(6)
    rows = rng.integers(0, y.shape[0], 3000)
    cols = rng.integers(0, y.shape[1], 3000)
    ref, b = dense_w8a8_rowwise_entries(rq, rs, wq, sw[0], rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), f"rowwise {which}")


def _gpu_block(x_bits, w_bits, out_dtype=torch.float32):
    import fp8_moe_prefill_amd as f
    wq, ws = f.fp8_quant_weight_block128(dev(w_bits))
    xq, xs = f.fp8_quant_act(dev(x_bits), 128)
    y = f.fp8_block_gemm(xq, xs, wq, ws, out_dtype)
    torch.cuda.synchronize()
    return host(y), host(xq), host(xs), host(wq), host(ws)


def _block_weight(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02 * rng.uniform(0.2, 5, (N, 1)) * rng.uniform(0.5, 2, (1, K))
    return bf16_bits_from_f32(w.astype(np.float32))


@pytest.mark.parametrize("M", [1, 8, 16, 300])
def test_block128_small_m(M):
    """Block-128 weights (memra-engine fp8_ffi docs): codes and block scales bit-exact; the
    GEMM at M = 1 / 8 / 16 (weight-streaming path) and 300 (tiles), N = 528 (a ragged last
    weight block of 16 rows), K = 4096, within the fp32 accumulation bound."""
    from oracle.dense import block_gemm
    from oracle.quant import quant_block128_bf16, quant_group_bf16
    inp = dense_inputs(CONFIGS["dense_w8a8"], M=M)
    w = _block_weight(528, 4096, M)
    y, xq, xs, wq, ws = _gpu_block(inp["x"], w)
    rq, rs = quant_group_bf16(inp["x"])
    rwq, rws = quant_block128_bf16(w)
    assert_bytes_equal(xq, rq, "activation codes")
    assert_bytes_equal(wq, rwq, "weight codes")
    assert_bytes_equal(ws.view(np.uint32), rws.view(np.uint32), "block scales")
    ref, b = block_gemm(rq, rs, rwq, rws, with_bound=True)
    check_close(y.astype(np.float64), ref, gemm_bound(b), f"block128 M={M}")
    yb = _gpu_block(inp["x"], w, torch.bfloat16)[0]
    assert_bytes_equal(yb, bf16_bits(round_bf16(y.astype(np.float64))), "bf16 = RNE(fp32)")


@pytest.mark.parametrize("which", ["w_qkv", "w_o"])
def test_block128_full_size_sampled(which):
    from oracle.dense import block_gemm_entries
    from oracle.quant import quant_group_bf16
    inp = dense_inputs(CONFIGS["dense_w8a8"])
    x = inp["x"] if which == "w_qkv" else inp["x_o"]
    y, xq, xs, wq, ws = _gpu_block(x, inp[which])
    rq, rs = quant_group_bf16(x)
    assert_bytes_equal(xq, rq, "activation codes")
    rng = np.random.default_rng(7)
    rows = rng.integers(0, y.shape[0], 3000)
    cols = rng.integers(0, y.shape[1], 3000)
    ref, b = block_gemm_entries(rq, rs, wq, ws, rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), f"block128 {which}")


def test_block128_quant_ragged_and_outliers():
    from oracle.quant import quant_block128_bf16
    w = _block_weight(200, 384, 11)
    w[150, 300] = 0x447A  # 1000.0 in bf16: the outlier sets its own block's scale only
    w[5] = 0x8000  # a -0 row
    import fp8_moe_prefill_amd as f
    q, s = f.fp8_quant_weight_block128(dev(w))
    torch.cuda.synchronize()
    rq, rs = quant_block128_bf16(w)
    assert_bytes_equal(host(q), rq, "codes")
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "block scales")


def test_big_tiles_sampled_and_equal_to_small_tiles():
    """4000 x 8000 x 256 per-tensor: enough 256 x 256 tiles for the one-workgroup-per-CU
    tiling (ragged in both M and N), sampled against the oracle with the last row and
    column included; its first 300 rows must equal, bit for bit, the same product over
    only those rows (128 x 128 tiles): both tilings run the same K steps per output."""
    import fp8_moe_prefill_amd as f
    rng = np.random.default_rng(21)
    M, N, K = 4000, 8000, 256
    x = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, sw = f.quantize_weight(dev(w))
    xq, blk = f.fp8_quant_act(dev(x), 0)
    y = f.fp8_dense_gemm(xq, blk, wq, sw, torch.float32)
    y_small = f.fp8_dense_gemm(xq[:300].contiguous(), blk, wq, sw, torch.float32)
    torch.cuda.synchronize()
    y, y_small = host(y), host(y_small)
    assert_bytes_equal(y[:300], y_small, "big tiles vs small tiles")
    rows = rng.integers(0, M, 3000)
    cols = rng.integers(0, N, 3000)
    rows[:3], cols[:3] = [M - 1, M - 1, 0], [N - 1, 0, N - 1]
    ref, b = dense_w8a8_entries(host(xq), host(blk)[2], host(wq), host(sw)[0], rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), "dense big tiles")


@pytest.mark.parametrize("rowwise", [False, True])
def test_wide_tiles_sampled_and_equal_to_small_tiles(rowwise):
    """1000 x 12176 x 256: 128 x 192 tiles fill the two workgroup slots of every CU in one
    round where 128 x 128 tiles would not, so the wide tiling runs (ragged in M and N: the
    last column tile holds 80 columns). Its first 640 rows must equal, bit for bit, the
    product over only those rows (128 x 128 tiles); bf16 output must be the rounded fp32
    output; sampled entries with the last row and column against the oracle."""
    import fp8_moe_prefill_amd as f
    rng = np.random.default_rng(31 + rowwise)
    M, N, K = 1000, 12176, 256
    x = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, sw = f.quantize_weight(dev(w))
    if rowwise:
        xq, sa = f.fp8_quant_act(dev(x), f.QUANT_ROW)
        gemm = lambda a, s, dt: f.fp8_dense_gemm_rowwise(a, s, wq, sw, dt)
        y = gemm(xq, sa, torch.float32)
        y_small = gemm(xq[:640].contiguous(), sa[:640].contiguous(), torch.float32)
        y16 = gemm(xq, sa, torch.bfloat16)
    else:
        xq, sa = f.fp8_quant_act(dev(x), 0)
        gemm = lambda a, dt: f.fp8_dense_gemm(a, sa, wq, sw, dt)
        y = gemm(xq, torch.float32)
        y_small = gemm(xq[:640].contiguous(), torch.float32)
        y16 = gemm(xq, torch.bfloat16)
    torch.cuda.synchronize()
    y, y_small, y16 = host(y), host(y_small), host(y16)
    assert_bytes_equal(y[:640], y_small, "wide tiles vs small tiles")
    assert_bytes_equal(y16, bf16_bits(round_bf16(y.astype(np.float64))), "bf16 = RNE(fp32)")
    rows = rng.integers(0, M, 3000)
    cols = rng.integers(0, N, 3000)
    rows[:4], cols[:4] = [M - 1, M - 1, 0, 639], [N - 1, 0, N - 1, N - 80]
    if rowwise:
        ref, b = dense_w8a8_rowwise_entries(host(xq), host(sa), host(wq), host(sw)[0], rows, cols)
    else:
        ref, b = dense_w8a8_entries(host(xq), host(sa)[2], host(wq), host(sw)[0], rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), "dense wide tiles")
