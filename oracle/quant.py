"""Dynamic activation quantisation to e4m3 -- oracle side (test infrastructure).

Three granularities:

* per (token, 128-wide K group): the FP8 grouped-expert prefill note, section 1 (one
  dynamic scale for each token and K group, applied inside the fp32 accumulation); this
  feeds the grouped expert GEMMs;
* per tensor: FreeToken PR #389, "What this adds" (a dynamic per-tensor activation
  scale: an amax pass, then the cast), and the memra-engine ``fp8_ffi`` docs (module
  text: one scalar scale amax/448); this feeds the dense W8A8 projections and is also the
  load-time weight quantiser ("e4m3 with one fp32 scale each");
* per row (token): FreeToken PR #389, "Limits", measures row-wise activation scales as
  the alternative to the per-tensor one (one outlier channel in one row then sets the
  scale of that row only). The pages print no row-wise formula; reading: the per-tensor
  rule below applied to each row on its own;
* per 128 x 128 weight block: the memra-engine fp8_ffi docs name a block-128 e4m3 weight
  class (QT_F8_E4M3_BLK, "the Qwen-official FP8 class": e4m3 weights with their own grid
  of block scales, read in place by a per-block FP8 tile). Reading: one scale per
  (128-row, 128-column) block of the [N, K] weight, found by the same rule; the last
  row block may be shorter when N is not a multiple of 128.

Arithmetic, all in fp32 as the scale block of ``fp8_ffi``'s ``Fp8Scratch`` is fp32:
  amax  = max |x| over the group (exact; NaN elements are skipped)
  a     = max(amax, AMAX_FLOOR)
  s     = fp32(a / 448)        the dequantisation scale (correctly rounded division)
  inv   = fp32(448 / a)        the quantising multiplier ("quant mul" slot of Fp8Scratch)
  q     = e4m3(fp32(x * inv))
Readings: the floor constant is not printed on the pages (PR #389 "Testing" names a
zero-input scale floor without its value); 1e-12 is used. Quantising multiplies by the
reciprocal, as the scale block's "quant mul" slot implies, rather than dividing.
"""

from __future__ import annotations

import numpy as np

from .codec import bf16_to_f32, e4m3_encode

AMAX_FLOOR = np.float32(1e-12)
GROUP = 128


def _scale_pair(amax: np.ndarray):
    a = np.maximum(np.asarray(amax, dtype=np.float32), AMAX_FLOOR)
    s = (a / np.float32(448.0)).astype(np.float32)
    inv = (np.float32(448.0) / a).astype(np.float32)
    return a, s, inv


def _amax(x: np.ndarray, axis) -> np.ndarray:
    ax = np.abs(x)
    ax = np.where(np.isnan(ax), np.float32(0.0), ax)  # NaN is skipped (maxNum)
    return ax.max(axis=axis).astype(np.float32)


def quant_group(x: np.ndarray, group: int = GROUP):
    """fp32 activations [M, K] -> (e4m3 codes [M, K], fp32 scales [M, K/group])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % group == 0
    xg = x.reshape(M, K // group, group)
    _, s, inv = _scale_pair(_amax(xg, axis=2))
    prod = (xg * inv[:, :, None]).astype(np.float32)  # fp32 product, correctly rounded
    q = e4m3_encode(prod).reshape(M, K)
    return q, s


def quant_tensor(x: np.ndarray):
    """fp32 tensor -> (e4m3 codes, scale block [amax, inv, s, 0] as fp32[4])."""
    x = np.asarray(x, dtype=np.float32)
    amax = _amax(x.reshape(-1), axis=0)
    _, s, inv = _scale_pair(amax)
    q = e4m3_encode((x * inv).astype(np.float32))
    return q, np.array([amax, inv, s, 0.0], dtype=np.float32)


def quant_row(x: np.ndarray):
    """fp32 activations [M, K] -> (e4m3 codes [M, K], fp32 scales [M]): one scale per row
    (FreeToken PR #389, "Limits": row-wise scales), each row quantised by the per-tensor
    rule."""
    x = np.asarray(x, dtype=np.float32)
    _, s, inv = _scale_pair(_amax(x, axis=1))
    q = e4m3_encode((x * inv[:, None]).astype(np.float32))
    return q, s


def quant_block128(w: np.ndarray):
    """fp32 weight [N, K] (K % 128 == 0) -> (e4m3 codes [N, K], fp32 block scales
    [ceil(N/128), K/128]): each 128 x 128 block quantised by the per-tensor rule
    (memra-engine fp8_ffi docs, the block-128 e4m3 class)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % GROUP == 0
    NB, G = -(-N // GROUP), K // GROUP
    q = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((NB, G), dtype=np.float32)
    for nb in range(NB):
        for g in range(G):
            blk = w[nb * GROUP:(nb + 1) * GROUP, g * GROUP:(g + 1) * GROUP]
            _, s, inv = _scale_pair(_amax(blk.reshape(-1), axis=0))
            q[nb * GROUP:(nb + 1) * GROUP, g * GROUP:(g + 1) * GROUP] = e4m3_encode(
                (blk * inv).astype(np.float32))
            scales[nb, g] = s
    return q, scales


def code_sums(q: np.ndarray, group: int = GROUP) -> np.ndarray:
    """e4m3 codes [M, K] -> float64 [M, K/group]: the sum of the decoded (unscaled) codes in
    each group. Not a quantity the pages name: the library can emit it beside the codes so
    that a GEMM on an offset-coded int4 weight (w = u - 8 with u >= 0) recovers
    sum_k a_k w_k as sum_k a_k u_k - 8 sum_k a_k without forming the second sum itself.
    Definition only: decode, then add, in float64 (exact for any 128 e4m3 values)."""
    from .codec import e4m3_decode
    q = np.asarray(q, dtype=np.uint8)
    M, K = q.shape
    assert K % group == 0
    return e4m3_decode(q).reshape(M, K // group, group).sum(axis=2)


def quant_block128_bf16(w_bits: np.ndarray):
    return quant_block128(bf16_to_f32(w_bits))


def quant_row_bf16(x_bits: np.ndarray):
    return quant_row(bf16_to_f32(x_bits))


def quant_group_bf16(x_bits: np.ndarray, group: int = GROUP):
    return quant_group(bf16_to_f32(x_bits), group)


def quant_tensor_bf16(x_bits: np.ndarray):
    return quant_tensor(bf16_to_f32(x_bits))
