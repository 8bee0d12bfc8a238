"""fp8_quant_act on the GPU vs the oracle: e4m3 bytes and fp32 scales bit-exact."""

import numpy as np
import pytest
import torch

from oracle.quant import quant_group_bf16, quant_row_bf16, quant_tensor_bf16
from synth import CONFIGS, bf16_bits_from_f32, dense_inputs, moe_inputs
from tests.gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _run_group(x_bits):
    import fp8_moe_prefill_amd as f
    q, s = f.fp8_quant_act(dev(x_bits), 128)
    torch.cuda.synchronize()
    return host(q), host(s)


def _run_tensor(x_bits):
    import fp8_moe_prefill_amd as f
    q, blk = f.fp8_quant_act(dev(x_bits), 0)
    torch.cuda.synchronize()
    return host(q), host(blk)


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_group_mode_config_inputs(cfg):
    x = moe_inputs(CONFIGS[cfg])["x"]
    q, s = _run_group(x)
    rq, rs = quant_group_bf16(x)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), "scales")


def test_group_mode_every_bf16_value():
    """Every finite bf16 with |x| <= 448, in groups whose amax is exactly 448 (so the
    multiplier is 1 and the codes are the plain encodings), then the same values at
    several other group maxima."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    vals = v[keep]
    n = len(vals)
    per = 127
    G = (n + per - 1) // per
    G = (G + 7) // 8 * 8  # whole rows of 8 groups
    x = np.zeros((G, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(G * per, np.float32)
    flat[:n] = vals
    x[:, 1:] = flat.reshape(G, per)
    for amax in [448.0, 1.0, 3.0e-3, 600.0, 7.0]:
        xs = (x * np.float32(amax / 448.0)).astype(np.float32)
        xb = bf16_bits_from_f32(xs).reshape(-1, 1024)  # 8 groups per row
        q, s = _run_group(xb)
        rq, rs = quant_group_bf16(xb)
        assert_bytes_equal(q, rq, f"codes at amax {amax}")
        assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), f"scales at amax {amax}")


def test_group_mode_edge_values():
    x = np.zeros((3, 256), np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = np.linspace(-5, 5, 128)
    x[2, :] = 1e-30  # far below the floor
    xb = bf16_bits_from_f32(x)
    xb[1, :128] = 0x8000  # -0.0 exactly
    q, s = _run_group(xb)
    rq, rs = quant_group_bf16(xb)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), "scales")
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (33, 2048), (2, 8192)])
def test_group_mode_ragged_shapes(M, K):
    rng = np.random.default_rng(M * K)
    x = bf16_bits_from_f32((rng.standard_normal((M, K)) * rng.uniform(0.01, 50, (M, 1))).astype(np.float32))
    q, s = _run_group(x)
    rq, rs = quant_group_bf16(x)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), "scales")


@pytest.mark.parametrize("M,K", [(1, 128), (16, 4096), (300, 4096), (2048, 4096), (8, 8)])
def test_tensor_mode(M, K):
    """Per-tensor: the fused single-workgroup path (<= 64k elements) and the two-pass
    path, on the dense workload's outlier-channel activations."""
    x = dense_inputs(CONFIGS["dense_w8a8"], M=min(M, 2048))["x"][:M, :K]
    x = np.ascontiguousarray(x)
    q, blk = _run_tensor(x)
    rq, rblk = quant_tensor_bf16(x)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(blk.view(np.uint32), rblk.view(np.uint32), "scale block")


def test_tensor_mode_zero_input_floor():
    x = np.zeros((16, 4096), np.uint16)
    q, blk = _run_tensor(x)
    assert np.all(q == 0)
    assert blk[0] == 0.0 and blk[2] == np.float32(np.float32(1e-12) / np.float32(448.0))


def test_weights_quantise_like_oracle():
    w = dense_inputs(CONFIGS["dense_w8a8"], M=1)["w_o"]
    q, blk = _run_tensor(w)
    rq, rblk = quant_tensor_bf16(w)
    assert_bytes_equal(q, rq, "weight codes")
    assert_bytes_equal(blk.view(np.uint32), rblk.view(np.uint32), "weight scale block")


def test_nan_smoke():
    x = np.ones((2, 128), np.float32)
    xb = bf16_bits_from_f32(x)
    xb[0, 5] = 0x7FC0  # quiet NaN
    q, s = _run_group(xb)
    assert q[0, 5] == 0x7F
    rq, rs = quant_group_bf16(xb)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), "scales")


def test_repeat_runs_identical():
    x = moe_inputs(CONFIGS["moe_tiny"])["x"]
    a = _run_group(x)
    b = _run_group(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _run_row(x_bits):
    import fp8_moe_prefill_amd as f
    q, s = f.fp8_quant_act(dev(x_bits), f.QUANT_ROW)
    torch.cuda.synchronize()
    return host(q), host(s)


@pytest.mark.parametrize("M,K", [(1, 8), (1, 4096), (7, 200), (300, 4096), (2048, 4096),
                                 (5, 16384)])
def test_row_mode(M, K):
    """One scale per row (FreeToken PR #389, "Limits"): ragged K (not a multiple of 128),
    one-row and full 2048 x 4096 tensors, rows spanning 4 decades, an all-zero row, a -0
    row and an outlier channel confined to its row."""
    rng = np.random.default_rng(M + K)
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-5, 4, (M, 1)))).astype(np.float32)
    if M > 3:
        x[1] = 0.0
        x[2, K // 3] = 3000.0
    xb = bf16_bits_from_f32(x)
    if M > 3:
        xb[3] = 0x8000
    q, s = _run_row(xb)
    rq, rs = quant_row_bf16(xb)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s.view(np.uint32), rs.view(np.uint32), "scales")
    if M > 3:
        assert np.all(q[1] == 0) and np.all(q[3] == 0x80)


def _sum_bound(q):
    """fp32 summation of one group: error <= 8 * 2^-24 * sum |dec(code)| (depth-7 tree)."""
    from oracle.codec import e4m3_decode
    M, K = q.shape
    return 8 * 2.0 ** -24 * np.abs(e4m3_decode(q)).reshape(M, K // 128, 128).sum(-1)


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_group_mode_code_sums(cfg):
    """The optional per-(token, 128) code sums: the codes and scales are unchanged by asking
    for them, and each sum is the sum of that group's decoded codes (the oracle's codes,
    which the GPU's equal bit for bit), to fp32 summation accuracy."""
    import fp8_moe_prefill_amd as f
    from oracle.quant import code_sums
    x = moe_inputs(CONFIGS[cfg])["x"]
    q, s, sm = f.fp8_quant_act(dev(x), 128, with_sums=True)
    torch.cuda.synchronize()
    rq, rs = quant_group_bf16(x)
    assert_bytes_equal(host(q), rq, "codes")
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")
    err = np.abs(host(sm).astype(np.float64) - code_sums(rq))
    assert np.all(err <= _sum_bound(rq)), err.max()


def test_code_sums_extremes():
    """Groups at the format's edges: all +448 (sum 57344, above 2^15 so fp32 partial sums
    round), all zero, alternating signs, and one outlier per group."""
    import fp8_moe_prefill_amd as f
    from oracle.quant import code_sums
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    x[0] = 7.0
    x[1] = 0.0
    x[2, 0::2], x[2, 1::2] = 3.0, -3.0
    x[3:, ::128] = 1000.0
    xb = bf16_bits_from_f32(x)
    q, s, sm = f.fp8_quant_act(dev(xb), 128, with_sums=True)
    torch.cuda.synchronize()
    rq, _ = quant_group_bf16(xb)
    assert_bytes_equal(host(q), rq, "codes")
    ref = code_sums(rq)
    err = np.abs(host(sm).astype(np.float64) - ref)
    assert np.all(err <= _sum_bound(rq)), err.max()
    assert np.all(host(sm)[0] == 57344.0) and np.all(host(sm)[1] == 0.0)
