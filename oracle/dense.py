"""Dense W8A8 projection -- oracle side (test infrastructure).

FreeToken PR #389, "What this adds": the projection weights are quantised at load time
to e4m3 with one fp32 scale per tensor, the activation gets one dynamic per-tensor
scale, and the product runs as an FP8 x FP8 GEMM. The memra-engine ``fp8_ffi`` module
text adds that the activation and weight scales are folded into one scalar applied to
the accumulator. So

    y[m, n] = (s_a * s_w) * sum_k dec(qa[m, k]) * dec(qw[n, k])

with both operands K-contiguous (a "TN" GEMM), computed here in float64.

Row-wise variant (FreeToken PR #389, "Limits": row-wise activation scales, measured there
against the per-tensor route): the activation carries one scale per row, so

    y[m, n] = (s_a[m] * s_w) * sum_k dec(qa[m, k]) * dec(qw[n, k]).

Block-128 variant (memra-engine fp8_ffi docs: the block-128 e4m3 weight class read in
place by a per-block FP8 tile): the weight carries one scale per 128 x 128 block. The
pages do not say how the activation is scaled on that path; reading: per (token, 128-wide
K group), as the grouped expert GEMM's activations (FP8 grouped-expert prefill note,
section 1), so both scales are constant inside each 128-wide K group and

    y[m, n] = sum_g s_a[m, g] * s_w[n // 128, g] * sum_{k in g} dec(qa[m, k]) * dec(qw[n, k]).
"""

from __future__ import annotations

import numpy as np

from .codec import e4m3_decode
from .quant import quant_tensor_bf16


def quantize_weight(w_bits: np.ndarray):
    """bf16 weight [N, K] -> (e4m3 codes [N, K], fp32 scale s_w): the per-tensor rule."""
    q, block = quant_tensor_bf16(w_bits)
    return q, np.float32(block[2])


def dense_w8a8(a_codes, a_scale, w_codes, w_scale, with_bound=False):
    a = e4m3_decode(a_codes) * float(a_scale)
    w = e4m3_decode(w_codes) * float(w_scale)
    y = a @ w.T
    if with_bound:
        return y, np.abs(a) @ np.abs(w).T
    return y


def dense_w8a8_entries(a_codes, a_scale, w_codes, w_scale, rows, cols):
    """Selected outputs y[rows[m], cols[m]] and bounds, one at a time."""
    y = np.empty(len(rows))
    b = np.empty(len(rows))
    for m, (i, n) in enumerate(zip(rows, cols)):
        a = e4m3_decode(a_codes[i]) * float(a_scale)
        w = e4m3_decode(w_codes[n]) * float(w_scale)
        y[m] = float(a @ w)
        b[m] = float(np.abs(a) @ np.abs(w))
    return y, b


def dense_w8a8_rowwise(a_codes, a_scales, w_codes, w_scale, with_bound=False):
    """Row-wise variant: a_scales is fp32 [M], one activation scale per row."""
    a = e4m3_decode(a_codes) * np.asarray(a_scales, dtype=np.float64)[:, None]
    w = e4m3_decode(w_codes) * float(w_scale)
    y = a @ w.T
    if with_bound:
        return y, np.abs(a) @ np.abs(w).T
    return y


def dense_w8a8_rowwise_entries(a_codes, a_scales, w_codes, w_scale, rows, cols):
    """Selected outputs of the row-wise variant and their bounds, one at a time."""
    y = np.empty(len(rows))
    b = np.empty(len(rows))
    for m, (i, n) in enumerate(zip(rows, cols)):
        a = e4m3_decode(a_codes[i]) * float(a_scales[i])
        w = e4m3_decode(w_codes[n]) * float(w_scale)
        y[m] = float(a @ w)
        b[m] = float(np.abs(a) @ np.abs(w))
    return y, b


def _block_dequant(a_codes, a_scales, w_codes, w_scales):
    G = 128
    a = e4m3_decode(a_codes) * np.repeat(np.asarray(a_scales, np.float64), G, axis=1)
    ws = np.repeat(np.repeat(np.asarray(w_scales, np.float64), G, axis=0), G, axis=1)
    w = e4m3_decode(w_codes) * ws[:w_codes.shape[0]]
    return a, w


def block_gemm(a_codes, a_scales, w_codes, w_scales, with_bound=False):
    """Block-128 variant: a_scales fp32 [M, K/128] (per token and K group), w_scales fp32
    [ceil(N/128), K/128] (per weight block). Both operands are dequantised with their
    scales, then multiplied in float64."""
    a, w = _block_dequant(a_codes, a_scales, w_codes, w_scales)
    y = a @ w.T
    if with_bound:
        return y, np.abs(a) @ np.abs(w).T
    return y


def block_gemm_entries(a_codes, a_scales, w_codes, w_scales, rows, cols):
    """Selected outputs of the block-128 variant and their bounds, one at a time."""
    G = 128
    y = np.empty(len(rows))
    b = np.empty(len(rows))
    for m, (i, n) in enumerate(zip(rows, cols)):
        a = e4m3_decode(a_codes[i]) * np.repeat(np.asarray(a_scales[i], np.float64), G)
        w = e4m3_decode(w_codes[n]) * np.repeat(np.asarray(w_scales[n // G], np.float64), G)
        y[m] = float(a @ w)
        b[m] = float(np.abs(a) @ np.abs(w))
    return y, b
