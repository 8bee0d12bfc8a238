"""Depth stack of L transformer layers with FP8 dense projections and FP8 grouped-expert
MoE, ending in LM-head logits -- oracle side (test infrastructure).

Source: "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1 (FP8
e4m3 q/k/v/o projections plus the grouped FP8 expert FFN; the parity gate is the cosine of
the final logits) and section 3 (depths L=8 and L=12). FreeToken PR #389, "Limits": the
LM head stays bf16.

Readings (the pages print no layer recipe):
* pre-norm blocks, RMSNorm with eps 1e-6 and unit gain, normalised activations stored
  in bf16;
* fused qkv projection [q (n_q*d) | k (n_kv*d) | v (n_kv*d)], no rotary embedding,
  grouped-query attention with query head h reading kv head h // (n_q/n_kv), causal,
  softmax scale 1/sqrt(d), output stored in bf16;
* residual adds are stored in bf16; the router is a bf16 GEMM with fp32 output over the
  normalised activations; the final RMSNorm feeds a bf16 LM head with fp32 logits.

The "bf16 path" is the same stack with the dense projections on the unquantised bf16
weights, no activation quantisation anywhere, and the experts on the int4 weights
dequantised exactly -- the analogue of the note's higher-precision baseline.
"""

from __future__ import annotations

import numpy as np

from .codec import bf16_to_f32
from .dense import dense_w8a8, quantize_weight
from .moe import combine, dequant_bank, swiglu
from .numeric import round_bf16
from .quant import quant_tensor
from .route import group_pairs, permute_rows, topk_route

EPS = 1e-6


def rmsnorm(x: np.ndarray) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row, float64 (unit gain)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)


def causal_gqa_attention(q, k, v, n_q, n_kv, d, with_bound=False):
    """q [T, n_q*d], k/v [T, n_kv*d] -> [T, n_q*d], float64.

    With ``with_bound`` also returns sum_s p[t, s] * |v[s]| per output element (the
    magnitude the attention weights' rounding errors scale with)."""
    T = q.shape[0]
    q = np.asarray(q, np.float64).reshape(T, n_q, d)
    k = np.asarray(k, np.float64).reshape(T, n_kv, d)
    v = np.asarray(v, np.float64).reshape(T, n_kv, d)
    out = np.empty((T, n_q, d))
    bound = np.empty((T, n_q, d)) if with_bound else None
    mask = np.tril(np.ones((T, T), dtype=bool))
    rep = n_q // n_kv
    for h in range(n_q):
        kv = h // rep
        s = (q[:, h, :] @ k[:, kv, :].T) / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
        if with_bound:
            bound[:, h, :] = p @ np.abs(v[:, kv, :])
    if with_bound:
        return out.reshape(T, n_q * d), bound.reshape(T, n_q * d)
    return out.reshape(T, n_q * d)


def _w8a8(x_bf16_vals, w_codes, w_scale):
    qa, blk = quant_tensor(np.asarray(x_bf16_vals, np.float32))
    return dense_w8a8(qa, blk[2], w_codes, w_scale)


def _route(logits, k, forced=None):
    """Top-k routing of one layer, or the given expert ids with their weights recomputed
    from these logits (the softmax over the k forced experts' logits)."""
    if forced is None:
        return topk_route(logits, k)
    ids = np.asarray(forced, np.int32)
    sel = np.take_along_axis(np.asarray(logits, np.float64), ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids, ex / ex.sum(axis=1, keepdims=True)


def _moe_fp8(hn_bf16_vals, logits, lay, k, forced=None):
    """The FP8 MoE layer of ``moe.moe_layer`` on already-bf16 activations (values)."""
    from .moe import grouped_gemm, swiglu_quant
    from .quant import quant_group

    E = lay["w_gu"].shape[0]
    xq, xs = quant_group(np.asarray(hn_bf16_vals, np.float32))
    ids, w = _route(logits, k, forced)
    offsets, sorted_, pos = group_pairs(ids, E)
    y_gu = grouped_gemm(permute_rows(xq, sorted_, k), permute_rows(xs, sorted_, k),
                        lay["w_gu"], lay["s_gu"], offsets)
    hq, hs, _ = swiglu_quant(y_gu)
    y_dn = round_bf16(grouped_gemm(hq, hs, lay["w_dn"], lay["s_dn"], offsets))
    return combine(y_dn, pos, w), ids


def _moe_bf16(hn_bf16_vals, logits, lay, k, forced=None):
    """Same routing; experts in float64 on the exactly dequantised int4 weights."""
    E = lay["w_gu"].shape[0]
    x = np.asarray(hn_bf16_vals, np.float64)
    ids, w = _route(logits, k, forced)
    out = np.zeros_like(x)
    for e in range(E):
        t, j = np.nonzero(ids == e)
        if len(t) == 0:
            continue
        wgu = dequant_bank(lay["w_gu"][e], lay["s_gu"][e])
        wdn = dequant_bank(lay["w_dn"][e], lay["s_dn"][e])
        h = round_bf16(swiglu(x[t] @ wgu.T))
        y = round_bf16(h @ wdn.T)
        np.add.at(out, t, w[t, j][:, None] * y)
    return out, ids


def stack_forward(inp: dict, n_q: int, n_kv: int, d: int, k: int, fp8: bool = True,
                  return_layers: bool = False, perturb=None, route_ids=None,
                  return_routes: bool = False, on_layer=None):
    """Run the stack on ``synth.stack_inputs`` data. Returns fp32 logits [T, V] (float64
    array of fp32-rounded values) and, if asked, the per-layer residual streams and the
    per-layer expert ids.

    Probes of the stack's sensitivity (none changes the arithmetic when left at None):
    ``perturb`` is applied to every dense projection output (q/k/v and o) before its bf16
    rounding; ``route_ids`` (one [T, k] array per layer) replaces the top-k choice of each
    layer's experts, the weights coming from that layer's own router logits.
    ``on_layer(li)`` is called after each layer (progress reports only)."""
    x = round_bf16(bf16_to_f32(inp["x0"]))
    nq = n_q * d
    nk = n_kv * d
    trace, routes = [], []
    pert = (lambda y: y) if perturb is None else perturb
    for li, lay in enumerate(inp["layers"]):
        hn = round_bf16(rmsnorm(x))
        if fp8:
            wq, sw = quantize_weight(lay["w_qkv"])
            qkv = round_bf16(pert(_w8a8(hn, wq, sw)))
        else:
            qkv = round_bf16(pert(hn @ bf16_to_f32(lay["w_qkv"]).astype(np.float64).T))
        att = round_bf16(causal_gqa_attention(qkv[:, :nq], qkv[:, nq:nq + nk],
                                              qkv[:, nq + nk:], n_q, n_kv, d))
        if fp8:
            wo, so = quantize_weight(lay["w_o"])
            o = round_bf16(pert(_w8a8(att, wo, so)))
        else:
            o = round_bf16(pert(att @ bf16_to_f32(lay["w_o"]).astype(np.float64).T))
        x = round_bf16(x + o)
        hn2 = round_bf16(rmsnorm(x))
        logits = (hn2 @ bf16_to_f32(lay["w_router"]).astype(np.float64).T).astype(np.float32)
        forced = None if route_ids is None else route_ids[li]
        moe, ids = (_moe_fp8 if fp8 else _moe_bf16)(hn2, logits, lay, k, forced)
        routes.append(ids)
        x = round_bf16(x + round_bf16(moe))
        if return_layers:
            trace.append(x.copy())
        if on_layer is not None:
            on_layer(li)
    hf = round_bf16(rmsnorm(x))
    out = (hf @ bf16_to_f32(inp["w_lm"]).astype(np.float64).T).astype(np.float32).astype(np.float64)
    res = (out,)
    if return_layers:
        res += (trace,)
    if return_routes:
        res += (routes,)
    return res if len(res) > 1 else out
