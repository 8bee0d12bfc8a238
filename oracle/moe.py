"""Grouped expert GEMM, SwiGLU + intermediate quantisation, weighted combine, and the
whole MoE layer -- oracle side (test infrastructure).

Source: "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1: one
grouped expert GEMM per layer over e4m3 activations and the resident packed-int4 expert
bank (dequantised to e4m3 without rounding, since -8..7 are exact in e4m3), with the
per-(token, group) activation scale and the per-group weight scale folded into the
accumulator. For expert e and its rows i,

    y[i, n] = sum_g  s_a[i, g] * s_w[e, n, g] * sum_{k in group g} dec(a[i, k]) * q[e, n, k]

computed here in float64 by dequantising both operands and multiplying (the same sum up
to rounding order).

Readings where the pages are silent:
* the expert FFN is SwiGLU with the gate|up projection fused into one [2I, H] bank,
  gate rows first: h = silu(gate) * up, silu(g) = g * sigmoid(g);
* h goes to e4m3 straight from fp32 (no bf16 round trip), per (row, 128 columns), with
  the same rule as the activation quantiser, and feeds the down GEMM;
* the down GEMM's rows are written in bf16; the combine weights them in fp32 order
  j = 0..k-1 and writes bf16.
"""

from __future__ import annotations

import numpy as np

from .codec import e4m3_decode, unpack_int4
from .quant import GROUP, quant_group, quant_group_bf16
from .route import group_pairs, permute_rows, topk_route


def dequant_act(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """e4m3 codes [R, K] with scales [R, K/group] -> float64 [R, K]."""
    R, K = codes.shape
    a = e4m3_decode(codes).reshape(R, K // group, group)
    return (a * np.asarray(scales, np.float64)[:, :, None]).reshape(R, K)


def dequant_bank(packed: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Packed int4 [N, K/2] with scales [N, K/group] -> float64 [N, K] (one expert)."""
    q = unpack_int4(packed).astype(np.float64)
    N, K = q.shape
    w = q.reshape(N, K // group, group) * np.asarray(scales, np.float64)[:, :, None]
    return w.reshape(N, K)


def grouped_gemm(a_codes, a_scales, w_packed, w_scales, offsets, with_bound=False):
    """y [R, N] float64 (and the bound B = sum_k |a_k w_k| if asked)."""
    R, K = a_codes.shape
    E, N, _ = w_packed.shape
    y = np.zeros((R, N), dtype=np.float64)
    bound = np.zeros((R, N), dtype=np.float64) if with_bound else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = dequant_act(a_codes[lo:hi], a_scales[lo:hi])
        w = dequant_bank(w_packed[e], w_scales[e])
        y[lo:hi] = a @ w.T
        if with_bound:
            bound[lo:hi] = np.abs(a) @ np.abs(w).T
    return (y, bound) if with_bound else y


def grouped_gemm_rows(a_codes, a_scales, w_packed, w_scales, offsets, rows, cols):
    """y[rows[m], cols[m]] and its bound, one output at a time (for full-size checks)."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    expert = np.searchsorted(np.asarray(offsets, np.int64), rows, side="right") - 1
    y = np.empty(len(rows))
    b = np.empty(len(rows))
    for m, (i, n, e) in enumerate(zip(rows, cols, expert)):
        a = dequant_act(a_codes[i:i + 1], a_scales[i:i + 1])[0]
        w = dequant_bank(w_packed[e, n:n + 1], w_scales[e, n:n + 1])[0]
        y[m] = float(np.dot(a, w))
        b[m] = float(np.dot(np.abs(a), np.abs(w)))
    return y, b


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu(y_gu: np.ndarray) -> np.ndarray:
    """[R, 2I] gate|up -> h [R, I] = silu(gate) * up, float64."""
    I = y_gu.shape[1] // 2
    return silu(y_gu[:, :I]) * y_gu[:, I:]


def swiglu_quant(y_gu: np.ndarray):
    """h in fp32, then e4m3 per (row, 128): (codes [R, I], scales [R, I/128], h fp32)."""
    h = swiglu(np.asarray(y_gu, np.float64)).astype(np.float32)
    q, s = quant_group(h)
    return q, s, h


def combine(y_perm: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_{j = 0..k-1} w[t, j] * y_perm[pos[t*k + j]], float64 [T, H]."""
    w = np.asarray(w, np.float64)
    T, k = w.shape
    y = np.asarray(y_perm, np.float64)
    pos = np.asarray(pos, np.int64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[pos[:, j]]
    return out


def moe_layer(x_bits, logits, w_gu, s_gu, w_dn, s_dn, k):
    """The whole MoE layer on bf16 input bits. Returns every stage (float64 outputs;
    the down GEMM's output is also given rounded to bf16, as the GPU writes it)."""
    from .numeric import round_bf16

    E = w_gu.shape[0]
    xq, xs = quant_group_bf16(x_bits)
    ids, w = topk_route(logits, k)
    offsets, sorted_, pos = group_pairs(ids, E)
    aq = permute_rows(xq, sorted_, k)
    as_ = permute_rows(xs, sorted_, k)
    y_gu = grouped_gemm(aq, as_, w_gu, s_gu, offsets)
    hq, hs, h = swiglu_quant(y_gu)
    y_dn = grouped_gemm(hq, hs, w_dn, s_dn, offsets)
    y_dn_bf16 = round_bf16(y_dn)
    out = combine(y_dn_bf16, pos, w)
    return dict(xq=xq, xs=xs, ids=ids, w=w, offsets=offsets, sorted=sorted_, pos=pos,
                aq=aq, as_=as_, y_gu=y_gu, h=h, hq=hq, hs=hs, y_dn=y_dn,
                y_dn_bf16=y_dn_bf16, out=out)
