"""Composition of the C-ABI calls into the MoE prefill layer and a W8A8 projection.

"FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1: the MoE layer
runs the activation quantiser, the routing/grouping, ONE grouped gate|up GEMM (SwiGLU and
the e4m3 requantisation fused in its epilogue), ONE grouped down GEMM, and the weighted
combine -- five launches families per layer, no per-token dispatch, no host sync.
FreeToken PR #389, "What this adds": a W8A8 projection is a per-tensor activation
quantisation followed by an FP8 x FP8 GEMM with the folded scalar scale.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class ExpertBank:
    """Resident expert weights of one MoE layer (device tensors), in the layout the grouped
    GEMM streams (see ``pack_expert_bank``).

    w_gu: bank bytes [E, 2I, H/2] (gate rows 0..I-1, up rows I..2I-1), s_gu fp32
    [E, H/128, 2I]; w_dn: bank bytes [E, H, I/2], s_dn fp32 [E, I/128, H].
    """

    w_gu: torch.Tensor
    s_gu: torch.Tensor
    w_dn: torch.Tensor
    s_dn: torch.Tensor

    @property
    def E(self) -> int:
        return self.w_gu.shape[0]

    @property
    def I(self) -> int:
        return self.w_gu.shape[1] // 2

    @property
    def H(self) -> int:
        return self.w_dn.shape[1]

    act: str = "e4m3"

    @staticmethod
    def from_canonical(w_gu, s_gu, w_dn, s_dn, stream=None, act: str = "e4m3") -> "ExpertBank":
        """Canonical device tensors (packed int4 [E, N, K/2], low nibble = even k; scales
        [E, N, K/128]) -> the packed layout (one-time, at load). ``act="mxfp4"``: the
        gate|up bank in the K order of the MXFP4-activation GEMM (the down GEMM's
        activations stay e4m3)."""
        if act not in ("e4m3", "mxfp4"):
            raise ValueError(f"act must be 'e4m3' or 'mxfp4', got {act!r}")
        gu = _lib.pack_expert_bank(w_gu, s_gu, stream=stream, mxfp4=act == "mxfp4")
        dn = _lib.pack_expert_bank(w_dn, s_dn, stream=stream)
        return ExpertBank(gu[0], gu[1], dn[0], dn[1], act)

    @staticmethod
    def from_host(d: dict, device, act: str = "e4m3") -> "ExpertBank":
        """Canonical host arrays w_gu, s_gu, w_dn, s_dn -> a packed bank on ``device``."""
        t = [torch.from_numpy(d[n]).to(device) for n in ("w_gu", "s_gu", "w_dn", "s_dn")]
        return ExpertBank.from_canonical(*t, act=act)


def moe_layer(x: torch.Tensor, logits: torch.Tensor, bank: ExpertBank, k: int,
              keep: bool = False, stream=None):
    """bf16 activations [T, H] and fp32 router logits [T, E] -> bf16 [T, H].

    With ``keep`` the intermediate tensors are returned too (for parity checks)."""
    T = x.shape[0]
    R = T * k
    # gate|up gathers its rows from token order through `sorted`, and with them each row's
    # per-token scales (and code sums) straight from the quantiser's output
    if bank.act == "mxfp4":  # MXFP4 activations into gate|up (bank packed for them)
        rt = _lib.moe_route_permute(logits, k, stream=stream)
        xq, xs = _lib.mxfp4_quant_act(x, stream=stream)
        xsum = None
        hq, hs, hsum = _lib.mxfp4_grouped_expert_gemm(
            xq, xs.view(torch.float32), bank.w_gu, bank.s_gu, rt["offsets"], R,
            _lib.EPI_SWIGLU_QUANT, sorted_=rt["sorted"], k_route=k, stream=stream,
            with_sums=True)
    else:
        # the quantiser also emits each (token, 128) group's code sum; the grouped GEMMs
        # take those in place of forming them from the tiles. Quantiser and routing in one
        # call (the quantiser beside the top-k)
        xq, xs, xsum, rt = _lib.quant_route(x, logits, k, stream=stream)
        hq, hs, hsum = _lib.fp8_grouped_expert_gemm(
            xq, xs, bank.w_gu, bank.s_gu, rt["offsets"], R, _lib.EPI_SWIGLU_QUANT,
            sorted_=rt["sorted"], k_route=k, stream=stream, a_sums=xsum, with_sums=True)
    y = _lib.fp8_grouped_expert_gemm(hq, hs, bank.w_dn, bank.s_dn, rt["offsets"], R,
                                     _lib.EPI_STORE, out_dtype=torch.bfloat16, stream=stream,
                                     a_sums=hsum)
    out = _lib.moe_unpermute_combine(y, rt["pos"], rt["weights"], torch.bfloat16, stream=stream)
    if keep:
        return out, dict(xq=xq, xs=xs, xsum=xsum, hq=hq, hs=hs, hsum=hsum, y=y, **rt)
    return out


def quantize_weight(w: torch.Tensor, stream=None):
    """Load-time per-tensor e4m3 weight (PR #389): bf16 [N, K] -> (codes, s_w [1] fp32)."""
    q, blk = _lib.fp8_quant_act(w, 0, stream=stream)
    return q, blk[2:3].clone()


def w8a8_linear(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                out_dtype=torch.bfloat16, stream=None):
    """bf16 [M, K] activations -> dynamic per-tensor e4m3 -> W8A8 GEMM -> [M, N]."""
    xq, blk = _lib.fp8_quant_act(x, 0, stream=stream)
    return _lib.fp8_dense_gemm(xq, blk, wq, w_scale, out_dtype, stream=stream)


class MoELayerRunner:
    """One MoE layer with every intermediate buffer allocated once (for serving loops and
    timing): call ``run(x, logits, bank)`` repeatedly; outputs are overwritten in place.

    Every launch goes to one stream (``stream``, else the current one). The optional
    ``events`` dict of (start, end) torch.cuda.Event pairs, keyed by stage name (see
    ``STAGES``), is recorded around the corresponding launches on that stream.

    With e4m3 activations the quantiser and the routing go through one call
    (``fp8moe_quant_route``: the quantiser and the top-k share a launch; stage
    "quant_route") unless ``fuse_quant_route`` is False; the outputs are the same bytes."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, device, act: str = "e4m3",
                 fuse_quant_route: bool = True):
        R = T * k
        self.T, self.H, self.E, self.k, self.I, self.R = T, H, E, k, I, R
        self.act = act
        self.fused = fuse_quant_route and act != "mxfp4"
        self.STAGES = (("quant_route",) if self.fused else ("quant", "route")) + (
            "gate_up", "down", "combine")
        dev = torch.device(device)
        u8, f32, i32 = torch.uint8, torch.float32, torch.int32
        if act == "mxfp4":  # codes [T, H/2]; E8M0 bytes [T, H/32] = [T, H/128] words
            self.xq = torch.empty((T, H // 2), dtype=u8, device=dev)
            self.xs = torch.empty((T, H // 32), dtype=u8, device=dev)
        else:
            self.xq = torch.empty((T, H), dtype=u8, device=dev)
            self.xs = torch.empty((T, H // _lib.GROUP), dtype=f32, device=dev)
            self.xsum = torch.empty((T, H // _lib.GROUP), dtype=f32, device=dev)
        self.route = dict(ids=torch.empty((T, k), dtype=i32, device=dev),
                          weights=torch.empty((T, k), dtype=f32, device=dev),
                          offsets=torch.empty(E + 1, dtype=i32, device=dev),
                          sorted=torch.empty(R, dtype=i32, device=dev),
                          pos=torch.empty(R, dtype=i32, device=dev))
        nws = _lib.workspace_bytes(_lib.OP_ROUTE_PERMUTE, T, E, k)
        self.ws = torch.empty(max(nws, 256), dtype=u8, device=dev)
        self.hq = torch.empty((R, I), dtype=u8, device=dev)
        self.hs = torch.empty((I // _lib.GROUP, R), dtype=f32, device=dev)
        self.hsum = torch.empty((I // _lib.GROUP, R), dtype=f32, device=dev)
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def run(self, x, logits, bank: ExpertBank, events=None, stream=None):
        ev = events or {}
        main = torch.cuda.current_stream() if stream is None else stream

        def mark(name, i):  # on the stream the layer's kernels are launched on
            if name in ev:
                ev[name][i].record(main)

        rt = self.route
        mx = self.act == "mxfp4"
        if bank.act != self.act:
            raise ValueError(f"bank packed for {bank.act} activations, runner for {self.act}")
        if self.fused:
            mark("quant_route", 0)
            _lib.quant_route(x, logits, self.k, q=self.xq, scales=self.xs, sums=self.xsum,
                             out=rt, ws=self.ws, stream=stream)
            mark("quant_route", 1)
        else:
            mark("quant", 0)
            if mx:
                _lib.mxfp4_quant_act(x, q=self.xq, scales=self.xs, stream=stream)
            else:
                _lib.fp8_quant_act(x, _lib.GROUP, q=self.xq, scales=self.xs, sums=self.xsum,
                                   stream=stream)
            mark("quant", 1)
            mark("route", 0)
            _lib.moe_route_permute(logits, self.k, out=rt, ws=self.ws, stream=stream)
            mark("route", 1)
        mark("gate_up", 0)
        self.run_gate_up(bank, stream=stream)
        mark("gate_up", 1)
        mark("down", 0)
        _lib.fp8_grouped_expert_gemm(self.hq, self.hs, bank.w_dn, bank.s_dn, rt["offsets"],
                                     self.R, _lib.EPI_STORE, out=self.y, stream=stream,
                                     a_sums=self.hsum)
        mark("down", 1)
        mark("combine", 0)
        _lib.moe_unpermute_combine(self.y, rt["pos"], rt["weights"], out=self.out,
                                   stream=stream)
        mark("combine", 1)
        return self.out

    def run_gate_up(self, bank: ExpertBank, stream=None):
        """The gate|up stage alone (grouped GEMM + SwiGLU + requantisation) on the
        quantised activations and routing the last ``run`` left in this runner."""
        rt = self.route
        # rows gathered from token order through `sorted`, with their per-token scales
        # (and code sums) straight from the quantiser's output
        if self.act == "mxfp4":
            _lib.mxfp4_grouped_expert_gemm(
                self.xq, self.xs.view(torch.float32), bank.w_gu, bank.s_gu, rt["offsets"],
                self.R, _lib.EPI_SWIGLU_QUANT, sorted_=rt["sorted"], k_route=self.k,
                out=self.hq, out_scales=self.hs, out_sums=self.hsum, stream=stream)
        else:
            _lib.fp8_grouped_expert_gemm(
                self.xq, self.xs, bank.w_gu, bank.s_gu, rt["offsets"], self.R,
                _lib.EPI_SWIGLU_QUANT, sorted_=rt["sorted"], k_route=self.k, out=self.hq,
                out_scales=self.hs, out_sums=self.hsum, stream=stream, a_sums=self.xsum)
