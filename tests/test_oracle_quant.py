"""Pins of the oracle's activation quantiser.

* invariant: in every group whose amax is above the floor the largest element maps to
  the largest code (|code| = 0x7E), because amax * fp32(448/amax) rounds to 448;
* special case: an all-zero group gives all 0x00 and s = fp32(1e-12)/448; -0.0 gives 0x80;
* closed-form error bound: |x - dec(q) * s| <= 2^-4 |x| in e4m3's normal range and
  <= 2^-10 s in the subnormal range (half a code spacing), up to fp32 scale rounding;
* library cross-check: torch computes x * inv in fp32 and casts with its own e4m3 encoder;
* per-tensor mode on a single group equals group mode; the scale block layout;
* row-wise mode: torch's fp32 multiply and e4m3 cast with each row's own amax; a single
  row equals per-tensor mode; rows a power of two apart share codes, scales exactly;
* block-128 weights: torch's cast with each 128 x 128 block's amax (ragged last row
  block); a single block equals per-tensor mode; blocks are independent.
"""

import numpy as np
import torch

from oracle.codec import e4m3_decode
from oracle.quant import AMAX_FLOOR, quant_group, quant_group_bf16, quant_row, quant_tensor
from synth import CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits, moe_inputs


def _x(seed=0, shape=(37, 512)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * np.exp(rng.uniform(-6, 4, (shape[0], 1)))
    return f32_from_bf16_bits(bf16_bits_from_f32(x.astype(np.float32)))


def test_max_element_maps_to_448():
    x = _x()
    q, s = quant_group(x)
    qg = q.reshape(x.shape[0], -1, 128)
    assert np.all(np.any((qg & 0x7F) == 0x7E, axis=2))
    assert np.all((qg & 0x7F) != 0x7F)  # no NaN codes from finite input


def test_zero_group_and_signed_zero():
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = np.linspace(-1, 1, 128, dtype=np.float32)
    q, s = quant_group(x)
    assert np.all(q[0] == 0x00) and np.all(q[1, :128] == 0x80)
    assert s[0, 0] == np.float32(np.float32(1e-12) / np.float32(448.0))
    assert s[0, 0] == s[1, 0] and AMAX_FLOOR == np.float32(1e-12)


def test_dequant_error_bound():
    x = _x(1, (64, 1024))
    q, s = quant_group(x)
    deq = e4m3_decode(q).reshape(64, 8, 128) * s[:, :, None].astype(np.float64)
    xx = x.reshape(64, 8, 128).astype(np.float64)
    err = np.abs(deq - xx)
    # x * inv is in the subnormal range when |x| < 2^-6 * s (approximately)
    sub = np.abs(xx) < (2.0 ** -6) * s[:, :, None]
    bound = np.where(sub, 2.0 ** -10 * s[:, :, None], 2.0 ** -4 * np.abs(xx))
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30)


def test_matches_torch_fp32_mul_and_cast():
    inp = moe_inputs(CONFIGS["moe_tiny"])
    q, s = quant_group_bf16(inp["x"])
    xt = torch.from_numpy(f32_from_bf16_bits(inp["x"]).copy()).reshape(64, -1, 128)
    amax = xt.abs().amax(dim=2, keepdim=True).clamp_min(1e-12)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    ref = torch.clamp(xt * inv, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(q, ref.reshape(64, -1).numpy())
    assert np.array_equal(s, (amax / 448.0).reshape(64, -1).numpy())


def test_per_tensor_block_and_single_group_equivalence():
    x = _x(2, (1, 128))
    qg, sg = quant_group(x)
    qt, blk = quant_tensor(x)
    assert np.array_equal(qg, qt) and blk[2] == sg[0, 0]
    assert blk[0] == np.abs(x).max() and blk[1] == np.float32(448.0) / blk[0] and blk[3] == 0


def test_per_tensor_outlier_channels_set_the_scale():
    inp_x = _x(3, (16, 256))
    inp_x[:, 5] *= 20
    q, blk = quant_tensor(inp_x)
    assert blk[0] == np.abs(inp_x).max()
    assert (q.reshape(-1) & 0x7F).max() == 0x7E


def test_nan_policy():
    x = _x(4, (2, 128))
    x[0, 3] = np.nan
    q, s = quant_group(x)
    assert q[0, 3] == 0x7F
    x2 = x.copy()
    x2[0, 3] = 0.0
    q2, s2 = quant_group(x2)
    assert s[0, 0] == s2[0, 0]  # NaN does not take part in amax


def test_row_wise_matches_torch_per_row_rule():
    # FreeToken PR #389 "Limits": row-wise scales; torch's own fp32 multiply and e4m3 cast
    # of every row with that row's amax
    x = _x(7, (37, 384))
    x[3, 5] = 300.0  # an outlier channel sets the scale of its own row only
    x[11] = 0.0      # an all-zero row takes the floor
    q, s = quant_row(x)
    xt = torch.from_numpy(x.copy())
    amax = xt.abs().amax(dim=1, keepdim=True).clamp_min(1e-12)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    ref = torch.clamp(xt * inv, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(q, ref.numpy())
    assert np.array_equal(s, (amax / 448.0).reshape(-1).numpy())
    assert s[3] == np.float32(300.0) / np.float32(448.0) and np.all(q[11] == 0)


def test_row_wise_single_row_is_per_tensor_and_rows_scale_exactly():
    x = _x(8, (1, 256))
    qr, sr = quant_row(x)
    qt, blk = quant_tensor(x)
    assert np.array_equal(qr, qt) and sr[0] == blk[2]
    # rows that differ by a power of two share their codes; their scales differ by it
    rows = np.concatenate([x * np.float32(2.0 ** j) for j in (-3, 0, 5)])
    q3, s3 = quant_row(rows)
    assert all(np.array_equal(q3[i], qt[0]) for i in range(3))
    assert np.array_equal(s3, blk[2] * np.float32([2.0 ** -3, 1.0, 2.0 ** 5]))


def test_block128_matches_torch_per_block_rule():
    # memra-engine fp8_ffi docs: the block-128 e4m3 weight class, one scale per 128 x 128
    # block; torch's fp32 multiply and e4m3 cast with each block's amax. N = 200: the last
    # row block has 72 rows.
    from oracle.quant import quant_block128
    w = _x(9, (200, 384)) * np.float32(0.05)
    w[150, 300] = 1000.0  # an outlier sets the scale of its own block only
    q, s = quant_block128(w)
    assert s.shape == (2, 3)
    wt = torch.from_numpy(np.vstack([w, np.zeros((56, 384), np.float32)]).copy())
    blocks = wt.reshape(2, 128, 3, 128).permute(0, 2, 1, 3)
    amax = blocks.abs().amax(dim=(2, 3), keepdim=True).clamp_min(1e-12)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    ref = torch.clamp(blocks * inv, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    ref = ref.permute(0, 2, 1, 3).reshape(256, 384)[:200]
    assert np.array_equal(q, ref.numpy())
    assert np.array_equal(s, (amax / 448.0).reshape(2, 3).numpy())
    assert s[1, 2] == np.float32(1000.0) / np.float32(448.0)


def test_block128_single_block_is_per_tensor_and_blocks_are_independent():
    from oracle.quant import quant_block128
    w = _x(10, (128, 256))
    q, s = quant_block128(w)
    for g in range(2):
        qt, blk = quant_tensor(w[:, 128 * g:128 * (g + 1)])
        assert np.array_equal(q[:, 128 * g:128 * (g + 1)], qt) and s[0, g] == blk[2]
    w2 = w.copy()
    w2[:, 128:] *= np.float32(2.0 ** 7)
    q2, s2 = quant_block128(w2)
    assert np.array_equal(q2, q) and s2[0, 0] == s[0, 0] and s2[0, 1] == s[0, 1] * 2 ** 7


def test_code_sums_closed_forms():
    """Sum of decoded codes per (row, 128 group): constant codes give 128 x value, a code
    beside its negation cancels, and a single nonzero code lands in its own (row, group)
    cell only (catches a transposed or mis-strided reshape)."""
    from oracle.quant import code_sums
    ones = np.full((3, 256), 0x38, np.uint8)  # e4m3 1.0
    assert np.array_equal(code_sums(ones), np.full((3, 2), 128.0))
    top = np.full((1, 128), 0x7E, np.uint8)  # e4m3 448 (largest finite)
    assert code_sums(top)[0, 0] == 448.0 * 128
    rng = np.random.default_rng(1)
    c = rng.integers(0, 0x7F, size=(4, 64), dtype=np.uint8)
    pair = np.empty((4, 128), np.uint8)
    pair[:, 0::2] = c
    pair[:, 1::2] = c | 0x80
    assert np.array_equal(code_sums(pair), np.zeros((4, 1)))
    for m, k, code, val in [(0, 5, 0x40, 2.0), (2, 300, 0xC8, -4.0), (1, 511, 0x01, 2.0 ** -9)]:
        q = np.zeros((3, 512), np.uint8)
        q[m, k] = code
        ref = np.zeros((3, 4))
        ref[m, k // 128] = val
        assert np.array_equal(code_sums(q), ref)


def test_code_sums_match_torch_float8_decode():
    import torch
    from oracle.quant import code_sums
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=(16, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0  # drop NaN codes
    t = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
    ref = t.reshape(16, 3, 128).sum(-1).numpy()
    assert np.allclose(code_sums(q), ref, rtol=0, atol=1e-9)
