"""Seeded sweep of the grouped expert GEMM over many small shapes, against the oracle.

Each case draws an expert count, a ragged row count per expert (empty experts, single
rows, exact and partial 128-row tiles), K (1..12 groups), N, the epilogue, the row source
(grouped rows, or rows gathered from token order through `sorted` with k = 1..6) and
whether the code sums are given. STORE outputs are checked element by element within the
GEMM bound; the SwiGLU epilogue's codes and scales against the oracle's SwiGLU of the same
kernel's fp32 accumulators (run with the same inputs)."""

import numpy as np
import pytest
import torch

from oracle.moe import grouped_gemm
from oracle.quant import code_sums, quant_group
from oracle.route import group_pairs, permute_rows, topk_route
from oracle.tol import check_close, gemm_bound
from tests.gpu_util import dev, host
from tests.test_gpu_grouped_gemm import _swiglu_check

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 5, 8, 17, 64]))
    K = 128 * int(rng.integers(1, 13))
    swiglu = bool(rng.integers(0, 2))
    N = 256 * int(rng.integers(1, 4)) if swiglu else 64 * int(rng.integers(1, 9))
    gather = bool(rng.integers(0, 2)) and E >= 2
    sums = bool(rng.integers(0, 2))
    if gather:
        k = int(rng.integers(1, min(6, E) + 1))
        T = int(rng.integers(1, 90))
        x = (rng.standard_normal((T, K)) * rng.uniform(0.01, 20, (T, 1))).astype(np.float32)
        logits = rng.standard_normal((T, E)).astype(np.float32)
        xq, xs = quant_group(x)
        ids, _ = topk_route(logits, k)
        off, sorted_, _ = group_pairs(ids, E)
        aq, as_ = permute_rows(xq, sorted_, k), permute_rows(xs, sorted_, k)
        src = (xq, xs, sorted_, k)
    else:
        counts = rng.choice([0, 1, 5, 127, 128, 129, 200], size=E)
        R = int(counts.sum())
        x = (rng.standard_normal((R, K)) * rng.uniform(0.01, 20, (R, 1))).astype(np.float32)
        aq, as_ = quant_group(x)
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        src = None
    wp = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.002, 0.03, size=(E, N, K // 128)).astype(np.float32)
    return dict(E=E, K=K, N=N, swiglu=swiglu, sums=sums, aq=aq, as_=as_, off=off, src=src,
                wp=wp, ws=ws)


@pytest.mark.parametrize("seed", range(32))
def test_grouped_gemm_sweep(seed):
    import fp8_moe_prefill_amd as f
    c = _case(seed)
    aq, as_, off = c["aq"], c["as_"], c["off"]
    R = aq.shape[0]
    w, s = f.pack_expert_bank(dev(c["wp"]), dev(c["ws"]))
    if c["src"] is None:
        args = (dev(aq), dev(np.ascontiguousarray(as_.T)), w, s, dev(off), R)
        kw = dict(a_sums=dev(np.ascontiguousarray(code_sums(aq).T.astype(np.float32)))
                  if c["sums"] else None)
    else:
        xq, xs, sorted_, k = c["src"]
        args = (dev(xq), dev(xs), w, s, dev(off), R)
        kw = dict(sorted_=dev(sorted_), k_route=k,
                  a_sums=dev(code_sums(xq).astype(np.float32)) if c["sums"] else None)
    y = f.fp8_grouped_expert_gemm(*args, f.EPI_STORE, torch.float32, **kw)
    torch.cuda.synchronize()
    ref, b = grouped_gemm(aq, as_, c["wp"], c["ws"], off, with_bound=True)
    check_close(host(y).astype(np.float64), ref, gemm_bound(b),
                f"sweep {seed}: E={c['E']} K={c['K']} N={c['N']} R={R}")
    if c["swiglu"] and R > 0:
        hq, hs = f.fp8_grouped_expert_gemm(*args, f.EPI_SWIGLU_QUANT, **kw)
        torch.cuda.synchronize()
        _swiglu_check(host(hq), np.ascontiguousarray(host(hs).T), host(y))


@pytest.mark.parametrize("seed", range(12))
def test_moe_layer_sweep(seed):
    """The whole layer (moe_layer: quantise with code sums, route, gate|up + SwiGLU, down,
    combine) on seeded random shapes, checked stage by stage as the layer tests do:
    quantiser bytes and routing indices bit-exact, the down GEMM and the combine on the
    GPU's own intermediates within their bounds, the output against the oracle's layer."""
    import fp8_moe_prefill_amd as f
    from oracle.moe import combine, moe_layer
    from oracle.numeric import cosine
    from oracle.tol import half_ulp_bf16
    from synth import moe_inputs
    from synth.inputs import MoEConfig
    from tests.gpu_util import assert_bytes_equal, bf16_values
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.choice([1, 2, 3, 8, 16, 33]))
    c = MoEConfig(name=f"sweep{seed}", T=int(rng.integers(1, 300)),
                  H=128 * int(rng.choice([1, 2, 4, 8])), E=E,
                  k=int(rng.integers(1, min(E, 8) + 1)), I=128 * int(rng.integers(1, 5)),
                  zipf_s=float(rng.choice([0.0, 1.2])), seed=seed)
    inp = moe_inputs(c)
    bank = f.ExpertBank.from_host(inp, "cuda:0")
    out, st = f.moe_layer(dev(inp["x"]), dev(inp["logits"]), bank, c.k, keep=True)
    torch.cuda.synchronize()
    ref = moe_layer(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"],
                    inp["s_dn"], c.k)
    what = f"{c}"
    for n in ("xq", "ids", "offsets", "sorted", "pos"):
        assert_bytes_equal(host(st[n]), ref[n], f"{n} ({what})")
    hq, hs = host(st["hq"]), np.ascontiguousarray(host(st["hs"]).T)
    y_ref, b = grouped_gemm(hq, hs, inp["w_dn"], inp["s_dn"], ref["offsets"], with_bound=True)
    y = bf16_values(st["y"])
    check_close(y, y_ref, gemm_bound(b) + half_ulp_bf16(y_ref), f"down ({what})")
    w = host(st["weights"]).astype(np.float64)
    o_ref = combine(y, host(st["pos"]), w)
    mag = combine(np.abs(y), host(st["pos"]), w)
    check_close(bf16_values(out), o_ref, 1e-6 * mag + half_ulp_bf16(o_ref), f"combine ({what})")
    assert cosine(bf16_values(out), ref["out"]) > 0.999, what


@pytest.mark.parametrize("seed", range(18))
def test_dense_w8a8_sweep(seed):
    """The W8A8 projection on seeded random shapes, for each scale granularity in turn
    (per tensor, per row, block-128 weights with per-(row, 128) activations): M from 1 to
    400 (the M <= 16 weight-streaming branch and the tiled one), ragged N (a multiple of
    16), K from 128 to 2048. Quantiser bytes bit-exact; outputs within the GEMM bound; the
    bf16 output equal to the rounded fp32 output."""
    import fp8_moe_prefill_amd as f
    from oracle.dense import block_gemm, dense_w8a8, dense_w8a8_rowwise, quantize_weight
    from oracle.numeric import bf16_bits, round_bf16
    from oracle.quant import (quant_block128_bf16, quant_group_bf16, quant_row_bf16,
                              quant_tensor_bf16)
    from synth import bf16_bits_from_f32
    from tests.gpu_util import assert_bytes_equal
    rng = np.random.default_rng(3000 + seed)
    mode = ("tensor", "row", "block")[seed % 3]
    M = int(rng.choice([1, 2, 7, 16])) if rng.integers(0, 2) else int(rng.integers(17, 400))
    N = 16 * int(rng.integers(1, 50))
    K = 128 * int(rng.integers(1, 17))
    x = rng.standard_normal((M, K)) * rng.uniform(0.1, 10, (M, 1))
    x[:, rng.integers(0, K, 3)] *= 20.0  # a few outlier channels
    xb = bf16_bits_from_f32(x.astype(np.float32))
    wb = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    what = f"{mode} M={M} N={N} K={K}"
    ys = {}
    for dt in (torch.float32, torch.bfloat16):
        if mode == "tensor":
            wq, sw = f.quantize_weight(dev(wb))
            xq, sa = f.fp8_quant_act(dev(xb), 0)
            y = f.fp8_dense_gemm(xq, sa, wq, sw, dt)
        elif mode == "row":
            wq, sw = f.quantize_weight(dev(wb))
            xq, sa = f.fp8_quant_act(dev(xb), f.QUANT_ROW)
            y = f.fp8_dense_gemm_rowwise(xq, sa, wq, sw, dt)
        else:
            wq, sw = f.fp8_quant_weight_block128(dev(wb))
            xq, sa = f.fp8_quant_act(dev(xb), 128)
            y = f.fp8_block_gemm(xq, sa, wq, sw, dt)
        torch.cuda.synchronize()
        ys[dt] = host(y)
    if mode == "tensor":
        rq, rblk = quant_tensor_bf16(xb)
        rwq, rsw = quantize_weight(wb)
        ref, b = dense_w8a8(rq, rblk[2], rwq, rsw, with_bound=True)
    elif mode == "row":
        rq, rs = quant_row_bf16(xb)
        rwq, rsw = quantize_weight(wb)
        ref, b = dense_w8a8_rowwise(rq, rs, rwq, rsw, with_bound=True)
    else:
        rq, rs = quant_group_bf16(xb)
        rwq, rws = quant_block128_bf16(wb)
        assert_bytes_equal(host(sw).view(np.uint32), rws.view(np.uint32), f"block scales ({what})")
        ref, b = block_gemm(rq, rs, rwq, rws, with_bound=True)
    assert_bytes_equal(host(xq), rq, f"activation codes ({what})")
    assert_bytes_equal(host(wq), rwq, f"weight codes ({what})")
    y32 = ys[torch.float32].astype(np.float64)
    check_close(y32, ref, gemm_bound(b), what)
    assert_bytes_equal(ys[torch.bfloat16], bf16_bits(round_bf16(y32)), f"bf16 = RNE(fp32) ({what})")


@pytest.mark.parametrize("seed", range(8))
def test_moe_layer_mxfp4_sweep(seed):
    """The layer with MXFP4 activations into gate|up on seeded random shapes: FP4 codes,
    E8M0 bytes and routing bit-exact, the down GEMM on the GPU's own intermediates within
    its bound, the output against the oracle's MXFP4 layer."""
    import fp8_moe_prefill_amd as f
    from oracle.mx import moe_layer_mxfp4, unpack_fp4
    from oracle.numeric import cosine
    from oracle.tol import half_ulp_bf16
    from synth import moe_inputs
    from synth.inputs import MoEConfig
    from tests.gpu_util import assert_bytes_equal, bf16_values
    rng = np.random.default_rng(4000 + seed)
    E = int(rng.choice([1, 3, 8, 16, 33]))
    c = MoEConfig(name=f"mxsweep{seed}", T=int(rng.integers(1, 300)),
                  H=128 * int(rng.choice([1, 2, 4, 8])), E=E,
                  k=int(rng.integers(1, min(E, 8) + 1)), I=128 * int(rng.integers(1, 5)),
                  zipf_s=float(rng.choice([0.0, 1.2])), seed=seed)
    inp = moe_inputs(c)
    bank = f.ExpertBank.from_host(inp, "cuda:0", act="mxfp4")
    out, st = f.moe_layer(dev(inp["x"]), dev(inp["logits"]), bank, c.k, keep=True)
    torch.cuda.synchronize()
    ref = moe_layer_mxfp4(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"],
                          inp["s_dn"], c.k)
    what = f"{c}"
    assert_bytes_equal(unpack_fp4(host(st["xq"])), ref["xq"], f"codes ({what})")
    assert_bytes_equal(host(st["xs"]), ref["xs"], f"E8M0 scales ({what})")
    for n in ("ids", "offsets", "sorted", "pos"):
        assert_bytes_equal(host(st[n]), ref[n], f"{n} ({what})")
    hq, hs = host(st["hq"]), np.ascontiguousarray(host(st["hs"]).T)
    y_ref, b = grouped_gemm(hq, hs, inp["w_dn"], inp["s_dn"], ref["offsets"], with_bound=True)
    y = bf16_values(st["y"])
    check_close(y, y_ref, gemm_bound(b) + half_ulp_bf16(y_ref), f"down ({what})")
    assert cosine(bf16_values(out), ref["out"]) > 0.999, what


@pytest.mark.parametrize("seed", range(10))
def test_causal_attention_sweep(seed):
    """Causal GQA attention of the depth stack on seeded random shapes: ragged T from 1 to
    300 (partial 64-key blocks and 16-query blocks), head layouts with 1, 2 and 4 query
    heads per kv head, two logit scales; within the derived bound of the existing attention
    test, token 0 exactly its own value row."""
    from tests.test_gpu_stack import test_attention_bound
    rng = np.random.default_rng(5000 + seed)
    n_kv = int(rng.choice([1, 2, 4]))
    n_q = n_kv * int(rng.choice([1, 2, 4]))
    T = int(rng.integers(1, 301))
    std = float(rng.choice([0.5, 3.0]))
    test_attention_bound(T, n_q, n_kv, std)


@pytest.mark.parametrize("seed", range(6))
def test_big_tile_gemm_sweep(seed):
    """The 256 x 256 TN tiling (taken when it gives every CU two tiles) on seeded ragged
    shapes, e4m3 per-tensor and bf16 in turn: sampled outputs within the GEMM bound, the
    last row and column included, and the first rows equal bit for bit to the same product
    over only those rows (which takes the 128 x 128 tiling)."""
    import fp8_moe_prefill_amd as f
    from oracle.dense import dense_w8a8_entries
    from synth import bf16_bits_from_f32
    from tests.gpu_util import assert_bytes_equal
    rng = np.random.default_rng(6000 + seed)
    bf16 = seed % 2 == 1
    M = int(rng.integers(2049, 4100))
    n_min = 256 * -(-512 // ((M + 255) // 256))  # enough 256-column tiles for 512 in all
    N = n_min + (16 * int(rng.integers(0, 100)) if not bf16 else int(rng.integers(1, 1500)))
    K = 128 * int(rng.integers(1, 5))
    assert ((M + 255) // 256) * ((N + 255) // 256) >= 512
    x = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    m0 = int(rng.integers(1, 300))
    if bf16:
        y = host(f.bf16_gemm(dev(x), dev(w)))
        y0 = host(f.bf16_gemm(dev(x[:m0]), dev(w)))
    else:
        wq, sw = f.quantize_weight(dev(w))
        xq, blk = f.fp8_quant_act(dev(x), 0)
        y = host(f.fp8_dense_gemm(xq, blk, wq, sw, torch.float32))
        y0 = host(f.fp8_dense_gemm(xq[:m0].contiguous(), blk, wq, sw, torch.float32))
    torch.cuda.synchronize()
    what = f"{'bf16' if bf16 else 'e4m3'} M={M} N={N} K={K}"
    assert_bytes_equal(y[:m0], y0, f"big vs small tiles ({what})")
    r = rng.integers(0, M, 2000)
    c = rng.integers(0, N, 2000)
    r[:3], c[:3] = [M - 1, M - 1, 0], [N - 1, 0, N - 1]
    if bf16:
        from oracle.codec import bf16_to_f32
        A = bf16_to_f32(x[r]).astype(np.float64)
        W = bf16_to_f32(w[c]).astype(np.float64)
        ref = np.einsum("ik,ik->i", A, W)
        b = np.einsum("ik,ik->i", np.abs(A), np.abs(W))
    else:
        ref, b = dense_w8a8_entries(host(xq), host(blk)[2], host(wq), host(sw)[0], r, c)
    check_close(y[r, c].astype(np.float64), ref, gemm_bound(b), what)
