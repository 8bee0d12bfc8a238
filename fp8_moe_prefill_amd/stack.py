"""Depth stack of L prefill layers composed from the C-ABI calls.

"FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", sections 1 and 3: L = 8
and L = 12 layers, each with e4m3 W8A8 q/k/v/o projections around a bf16 causal
attention core and an MoE block whose experts run as the FP8 grouped GEMM over the
resident int4 bank, gated on the cosine of the final logits. FreeToken PR #389,
"Limits": the LM head stays bf16.

Block recipe (the pages print none; the plain pre-norm reading, unit RMSNorm gains, eps
1e-6, residual stream in bf16):

    hn  = rmsnorm(x)                         fp8moe_rmsnorm (fused with the previous add)
    qkv = W8A8(hn)        [q | k | v]        fp8_quant_act(per tensor) + fp8_dense_gemm
    att = attention(qkv)  causal, GQA        fp8moe_causal_attention
    o   = W8A8(att)                          fp8_quant_act(per tensor) + fp8_dense_gemm
    x   = x + o;  hn2 = rmsnorm(x)           fp8moe_rmsnorm (residual add fused)
    logits_r = hn2 . W_router^T  (fp32)      fp8moe_bf16_gemm
    m   = MoE(hn2, logits_r)                 the five MoE-layer calls
    x   = x + m                              fused into the next rmsnorm
    out = rmsnorm(x) . W_lm^T  (fp32)        fp8moe_rmsnorm + fp8moe_bf16_gemm

Every buffer is allocated once by ``StackRunner``; ``run`` only enqueues library calls on
the current stream (no host sync).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from .layer import ExpertBank, MoELayerRunner, quantize_weight


@dataclass
class StackLayer:
    """Device weights of one layer: e4m3 W8A8 projections with their per-tensor scales,
    the bf16 router and the packed expert bank."""

    w_qkv: torch.Tensor  # e4m3 [(n_q + 2 n_kv) d, H]
    s_qkv: torch.Tensor  # fp32 [1]
    w_o: torch.Tensor    # e4m3 [H, n_q d]
    s_o: torch.Tensor    # fp32 [1]
    w_router: torch.Tensor  # bf16 [E, H]
    bank: ExpertBank


@dataclass
class DepthStack:
    layers: list
    w_lm: torch.Tensor  # bf16 [V, H]
    n_q: int
    n_kv: int
    head_dim: int
    k: int

    @property
    def H(self) -> int:
        return self.w_lm.shape[1]

    @property
    def V(self) -> int:
        return self.w_lm.shape[0]

    @staticmethod
    def from_host(inp: dict, n_q: int, n_kv: int, head_dim: int, k: int, device) -> "DepthStack":
        """Host weights (bf16 bit patterns as uint16, canonical int4 banks) -> device; the
        dense projections are quantised to e4m3 per tensor on the device (load time)."""

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
                torch.bfloat16)

        layers = []
        for lay in inp["layers"]:
            wq, sq = quantize_weight(bf16(lay["w_qkv"]))
            wo, so = quantize_weight(bf16(lay["w_o"]))
            layers.append(StackLayer(wq, sq, wo, so, bf16(lay["w_router"]),
                                     ExpertBank.from_host(lay, device)))
        return DepthStack(layers, bf16(inp["w_lm"]), n_q, n_kv, head_dim, k)


class StackRunner:
    """The whole stack over T tokens with preallocated buffers. ``run(x0)`` returns the
    fp32 logits [T, V] (overwritten by the next call).

    ``keep``: a list that receives, per layer, a dict of copies of the intermediates (for
    parity checks; the copies are torch device copies outside the timed path), and a last
    dict with the final residual stream and normalised activations; ``keep_layers``
    restricts the full records to those layer indices (a layer right after a recorded one
    keeps only its input "x", the others None).
    ``events``: optional dict of (start, end) torch.cuda.Event pairs keyed by "layer" and
    "lm_head", recorded around those parts."""

    def __init__(self, stack: DepthStack, T: int, device):
        s = stack
        dev = torch.device(device)
        H, d = s.H, s.head_dim
        bank = s.layers[0].bank
        self.stack, self.T = s, T
        bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
        nqkv = (s.n_q + 2 * s.n_kv) * d
        self.x = torch.empty((T, H), dtype=bf, device=dev)
        self.hn = torch.empty((T, H), dtype=bf, device=dev)
        self.qa = torch.empty((T, max(H, s.n_q * d)), dtype=u8, device=dev)
        self.blk = torch.empty(4, dtype=f32, device=dev)
        self.qws = torch.empty(max(_lib.workspace_bytes(_lib.OP_QUANT_ACT, T, max(H, s.n_q * d), 0),
                                   256), dtype=u8, device=dev)
        self.qkv = torch.empty((T, nqkv), dtype=bf, device=dev)
        self.att = torch.empty((T, s.n_q * d), dtype=bf, device=dev)
        self.aws = torch.empty(_lib.workspace_bytes(_lib.OP_ATTENTION, T, s.n_kv, d),
                               dtype=u8, device=dev)
        self.o = torch.empty((T, H), dtype=bf, device=dev)
        self.logits_r = torch.empty((T, bank.E), dtype=f32, device=dev)
        self.moe = MoELayerRunner(T, H, bank.E, s.k, bank.I, dev)
        self.logits = torch.empty((T, s.V), dtype=f32, device=dev)

    def _w8a8(self, x, wq, sw, out, stream):
        T, K = x.shape
        qa = self.qa.view(-1)[:T * K].view(T, K)
        _lib.fp8_quant_act(x, 0, q=qa, scales=self.blk, ws=self.qws, stream=stream)
        _lib.fp8_dense_gemm(qa, self.blk, wq, sw, out=out, stream=stream)

    def run(self, x0: torch.Tensor, keep=None, keep_layers=None, events=None, stream=None):
        s = self.stack
        ev = events or {}
        x_in = x0
        all_keep = keep
        for li, lay in enumerate(s.layers):
            keep = all_keep if keep_layers is None or li in keep_layers else None
            if "layer" in ev:
                ev["layer"][0][li].record()
            if li == 0:
                _lib.rmsnorm(x0, y=self.hn, stream=stream)
            else:
                # x = x + moe (previous layer), then this layer's first norm
                _lib.rmsnorm(self.x, delta=self.moe.out, x_out=self.x, y=self.hn, stream=stream)
            if keep is not None:
                rec = dict(x=x_in.clone(), hn=self.hn.clone())
            elif all_keep is not None:
                # a layer after a recorded one keeps its input (the recorded layer's output)
                after = li - 1 in keep_layers
                all_keep.append(dict(x=x_in.clone()) if after else None)
            self._w8a8(self.hn, lay.w_qkv, lay.s_qkv, self.qkv, stream)
            _lib.causal_attention(self.qkv, s.n_q, s.n_kv, s.head_dim, out=self.att,
                                  ws=self.aws, stream=stream)
            self._w8a8(self.att, lay.w_o, lay.s_o, self.o, stream)
            # x = x + o, hn2 = rmsnorm(x)
            _lib.rmsnorm(x_in, delta=self.o, x_out=self.x, y=self.hn, stream=stream)
            x_in = self.x
            _lib.bf16_gemm(self.hn, lay.w_router, out=self.logits_r, stream=stream)
            if keep is not None:
                rec.update(qkv=self.qkv.clone(), att=self.att.clone(), o=self.o.clone(),
                           x_mid=self.x.clone(), hn2=self.hn.clone(),
                           logits_r=self.logits_r.clone())
            self.moe.run(self.hn, self.logits_r, lay.bank, stream=stream)
            if keep is not None:
                rt = self.moe.route
                rec.update(ids=rt["ids"].clone(), weights=rt["weights"].clone(),
                           offsets=rt["offsets"].clone(), pos=rt["pos"].clone(),
                           sorted=rt["sorted"].clone(), xq=self.moe.xq.clone(),
                           xs=self.moe.xs.clone(), hq=self.moe.hq.clone(),
                           hs=self.moe.hs.clone(), y=self.moe.y.clone(),
                           moe=self.moe.out.clone())
                keep.append(rec)
            if "layer" in ev:
                ev["layer"][1][li].record()
        keep = all_keep
        if "lm_head" in ev:
            ev["lm_head"][0].record()
        _lib.rmsnorm(self.x, delta=self.moe.out, x_out=self.x, y=self.hn, stream=stream)
        if keep is not None:
            keep.append(dict(x=self.x.clone(), hf=self.hn.clone()))
        _lib.bf16_gemm(self.hn, s.w_lm, out=self.logits, stream=stream)
        if "lm_head" in ev:
            ev["lm_head"][1].record()
        return self.logits
