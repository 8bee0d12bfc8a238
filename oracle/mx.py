"""FP4 (E2M1) activations with shared power-of-two block scales -- oracle side (test
infrastructure).

The DeepGEMM issue "FP4 activations for fp8_fp4_mega_moe" (github.com/deepseek-ai/DeepGEMM
issue 338) proposes E2M1 activations, packed by a pre-dispatch kernel, to halve the
dispatch buffer and to run an MXF4 main loop. The pages give no packing formula; the
plainest reading of "E2M1" with an "MXF4" main loop is the OCP Microscaling (MX) v1.0
MXFP4 format, and that published definition is what this module states:

* blocks of 32 consecutive elements along K share one scale X = 2^e stored as E8M0
  (byte e + 127);
* e = floor(log2(max |v| over the block)) - 2 (2 is E2M1's largest exponent), clamped to
  the E8M0 range [-127, 127]; an all-zero block takes e = -127;
* each element is v / X rounded to the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (sign
  separate) to nearest, ties to the even code, magnitudes above 6 saturating to 6.

Readings where the spec leaves a choice to the implementation: NaN elements are skipped
by the block maximum and encode to +0 (E2M1 has no NaN); the sign of zero is kept
(-0 -> code 8). Codes are 4-bit: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
packed two per byte, the low nibble holding the even index along K (as the int4 bank).

The grouped GEMM with such activations is the grouped expert GEMM of ``moe.py`` with the
activation dequantised as code value x 2^e per 32-element block.
"""

from __future__ import annotations

import numpy as np

from .codec import bf16_to_f32
from .moe import dequant_bank

BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E8M0_BIAS = 127


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float64 values -> 4-bit codes: nearest grid point, ties to the even code, saturating
    at 6, sign kept on zero, NaN -> +0."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, np.abs(v))
    # distance to every grid point; the lowest code among the nearest is the even one at a
    # tie, since adjacent grid points have codes of opposite parity
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    code = np.where(a > 6.0, 7, code)
    sign = np.signbit(v) & ~nan
    return (code | np.where(sign, 8, 0)).astype(np.uint8)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent e of a block with maximum magnitude amax (float64)."""
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))) - 2, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quant_mxfp4(x: np.ndarray):
    """fp32 activations [M, K] (K % 32 == 0) -> (E2M1 codes uint8 [M, K], E8M0 scale bytes
    uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    assert K % BLOCK == 0
    xb = x.reshape(M, K // BLOCK, BLOCK)
    amax = np.where(np.isnan(xb), 0.0, np.abs(xb)).max(axis=2)
    e = block_exponent(amax)
    codes = e2m1_encode(xb / np.exp2(e)[:, :, None]).reshape(M, K)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def quant_mxfp4_bf16(x_bits: np.ndarray):
    return quant_mxfp4(bf16_to_f32(x_bits))


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1 codes [M, K] with E8M0 bytes [M, K/32] -> float64 [M, K]."""
    M, K = codes.shape
    v = e2m1_decode(codes).reshape(M, K // BLOCK, BLOCK)
    x = np.exp2(np.asarray(scales, np.float64) - E8M0_BIAS)
    return (v * x[:, :, None]).reshape(M, K)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[M, K] 4-bit codes -> [M, K/2] bytes, low nibble = even index."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def grouped_gemm_fp4act(a_codes, a_scales, w_packed, w_scales, offsets, with_bound=False):
    """Grouped expert GEMM with MXFP4 activations: a_codes [R, K] E2M1 codes, a_scales
    [R, K/32] E8M0 bytes, the int4 bank as in ``moe.grouped_gemm``. float64 [R, N]."""
    R, K = a_codes.shape
    E, N, _ = w_packed.shape
    y = np.zeros((R, N), dtype=np.float64)
    bound = np.zeros((R, N), dtype=np.float64) if with_bound else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = dequant_mxfp4(a_codes[lo:hi], a_scales[lo:hi])
        w = dequant_bank(w_packed[e], w_scales[e])
        y[lo:hi] = a @ w.T
        if with_bound:
            bound[lo:hi] = np.abs(a) @ np.abs(w).T
    return (y, bound) if with_bound else y


def grouped_gemm_fp4act_rows(a_codes, a_scales, w_packed, w_scales, offsets, rows, cols):
    """Selected outputs and bounds of ``grouped_gemm_fp4act``, one at a time."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    expert = np.searchsorted(np.asarray(offsets, np.int64), rows, side="right") - 1
    y = np.empty(len(rows))
    b = np.empty(len(rows))
    for m, (i, n, e) in enumerate(zip(rows, cols, expert)):
        a = dequant_mxfp4(a_codes[i:i + 1], a_scales[i:i + 1])[0]
        w = dequant_bank(w_packed[e, n:n + 1], w_scales[e, n:n + 1])[0]
        y[m] = float(np.dot(a, w))
        b[m] = float(np.dot(np.abs(a), np.abs(w)))
    return y, b


def moe_layer_mxfp4(x_bits, logits, w_gu, s_gu, w_dn, s_dn, k):
    """The MoE layer with MXFP4 activations into the gate|up GEMM (DeepGEMM issue 338's
    FP4 dispatch); every other stage as ``moe.moe_layer``: routing, the SwiGLU and its
    e4m3 requantisation, the down GEMM, the combine."""
    from .moe import combine, grouped_gemm, swiglu_quant
    from .numeric import round_bf16
    from .route import group_pairs, permute_rows, topk_route

    E = w_gu.shape[0]
    xq, xs = quant_mxfp4_bf16(x_bits)
    ids, w = topk_route(logits, k)
    offsets, sorted_, pos = group_pairs(ids, E)
    aq = permute_rows(xq, sorted_, k)
    as_ = permute_rows(xs, sorted_, k)
    y_gu = grouped_gemm_fp4act(aq, as_, w_gu, s_gu, offsets)
    hq, hs, h = swiglu_quant(y_gu)
    y_dn = grouped_gemm(hq, hs, w_dn, s_dn, offsets)
    y_dn_bf16 = round_bf16(y_dn)
    out = combine(y_dn_bf16, pos, w)
    return dict(xq=xq, xs=xs, ids=ids, w=w, offsets=offsets, sorted=sorted_, pos=pos,
                aq=aq, as_=as_, y_gu=y_gu, h=h, hq=hq, hs=hs, y_dn=y_dn,
                y_dn_bf16=y_dn_bf16, out=out)
