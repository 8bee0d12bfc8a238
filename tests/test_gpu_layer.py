"""The whole MoE layer (quantise, route, gate|up + SwiGLU + requantise, down, combine)
through the C ABI vs the oracle.

Stage by stage on identical inputs: quantiser bytes and routing indices bit-exact; the
down GEMM and the combine checked on the GPU's own intermediate codes, so the strict
bounds apply; the final output additionally compared to the oracle's end-to-end result
through the element bound of the combine (each row's own rounding included).
"""

import numpy as np
import pytest
import torch

from oracle.moe import combine, grouped_gemm, grouped_gemm_rows, moe_layer
from oracle.numeric import cosine
from oracle.quant import quant_group_bf16
from oracle.route import group_pairs, topk_route
from oracle.tol import check_close, gemm_bound, half_ulp_bf16
from synth import CONFIGS, moe_inputs
from tests.gpu_util import assert_bytes_equal, bf16_values, dev, host

pytestmark = pytest.mark.gpu


def _gpu_layer(cfg, T=None):
    import fp8_moe_prefill_amd as f
    c = CONFIGS[cfg]
    inp = moe_inputs(c, T=T)
    bank = f.ExpertBank.from_host(inp, "cuda:0")
    out, st = f.moe_layer(dev(inp["x"]), dev(inp["logits"]), bank, c.k, keep=True)
    torch.cuda.synchronize()
    return c, inp, out, st


@pytest.mark.parametrize("cfg,T", [("moe_tiny", None), ("moe_prefill", 1), ("moe_prefill", 16)])
def test_layer_all_outputs(cfg, T):
    """The tiny layer, and the config-3 layer at decode token counts (one or two rows per
    expert: the grouped GEMM's few-rows regime)."""
    c, inp, out, st = _gpu_layer(cfg, T=T)
    ref = moe_layer(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"],
                    inp["s_dn"], c.k)
    assert_bytes_equal(host(st["xq"]), ref["xq"], "xq")
    assert_bytes_equal(host(st["ids"]), ref["ids"], "ids")
    assert_bytes_equal(host(st["offsets"]), ref["offsets"], "offsets")
    assert_bytes_equal(host(st["sorted"]), ref["sorted"], "sorted")
    assert_bytes_equal(host(st["pos"]), ref["pos"], "pos")
    # down GEMM on the GPU's own intermediate codes
    hq, hs = host(st["hq"]), np.ascontiguousarray(host(st["hs"]).T)
    y_ref, b = grouped_gemm(hq, hs, inp["w_dn"], inp["s_dn"], ref["offsets"], with_bound=True)
    y = bf16_values(st["y"])
    check_close(y, y_ref, gemm_bound(b) + half_ulp_bf16(y_ref), "down (bf16 out)")
    # combine on the GPU's own rows and weights
    o_ref = combine(y, host(st["pos"]), host(st["weights"]).astype(np.float64))
    mag = combine(np.abs(y), host(st["pos"]), host(st["weights"]).astype(np.float64))
    check_close(bf16_values(out), o_ref, 1e-6 * mag + half_ulp_bf16(o_ref), "combine")
    # end to end: the oracle's layer output vs the GPU's
    assert cosine(bf16_values(out), ref["out"]) > 0.999


@pytest.mark.parametrize("cfg", ["moe_prefill", "moe_skewed"])
def test_full_layer_sampled(cfg):
    c, inp, out, st = _gpu_layer(cfg)
    xq, xs = quant_group_bf16(inp["x"])
    assert_bytes_equal(host(st["xq"]), xq, "xq")
    assert_bytes_equal(host(st["xs"]).view(np.uint32), xs.view(np.uint32), "xs")
    ids, w = topk_route(inp["logits"], c.k)
    off, sorted_, pos = group_pairs(ids, c.E)
    assert_bytes_equal(host(st["ids"]), ids, "ids")
    assert_bytes_equal(host(st["offsets"]), off, "offsets")
    assert_bytes_equal(host(st["sorted"]), sorted_, "sorted")
    assert_bytes_equal(host(st["pos"]), pos, "pos")
    if cfg == "moe_skewed":
        assert (np.diff(off) == 0).sum() >= 1
    # down GEMM, sampled, on the GPU's intermediate codes
    hq, hs = host(st["hq"]), np.ascontiguousarray(host(st["hs"]).T)
    y = st["y"]
    R = c.T * c.k
    rng = np.random.default_rng(21)
    rows = rng.integers(0, R, 2000)
    cols = rng.integers(0, c.H, 2000)
    yr, b = grouped_gemm_rows(hq, hs, inp["w_dn"], inp["s_dn"], off, rows, cols)
    ys = y[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].float().cpu().numpy()
    check_close(ys.astype(np.float64), yr, gemm_bound(b) + half_ulp_bf16(yr), "down sampled")
    # combine on sampled tokens
    toks = rng.integers(0, c.T, 64)
    yv = bf16_values(y)
    o = bf16_values(out)
    wv = host(st["weights"]).astype(np.float64)
    p = host(st["pos"]).reshape(c.T, c.k)
    for t in toks:
        ref = sum(wv[t, j] * yv[p[t, j]] for j in range(c.k))
        mag = sum(abs(wv[t, j]) * np.abs(yv[p[t, j]]) for j in range(c.k))
        check_close(o[t], ref, 1e-6 * mag + half_ulp_bf16(ref), "combine sampled")


def test_layer_repeat_runs_identical():
    _, _, out1, st1 = _gpu_layer("moe_prefill", T=512)
    _, _, out2, st2 = _gpu_layer("moe_prefill", T=512)
    for n in ("xq", "hq", "hs", "y", "sorted", "pos"):
        a, b = host(st1[n]), host(st2[n])
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), n
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("cfg,T", [("moe_tiny", None), ("moe_prefill", 16), ("moe_prefill", None)])
def test_layer_mxfp4_activations(cfg, T):
    """The layer with MXFP4 activations into gate|up (DeepGEMM issue 338's FP4 dispatch):
    codes, scale bytes and routing bit-exact; the down GEMM and the combine on the GPU's own
    intermediates within their bounds; the output against the oracle's MXFP4 layer."""
    import fp8_moe_prefill_amd as f
    from oracle.mx import moe_layer_mxfp4, unpack_fp4
    c = CONFIGS[cfg]
    inp = moe_inputs(c, T=T)
    bank = f.ExpertBank.from_host(inp, "cuda:0", act="mxfp4")
    out, st = f.moe_layer(dev(inp["x"]), dev(inp["logits"]), bank, c.k, keep=True)
    torch.cuda.synchronize()
    ref = moe_layer_mxfp4(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"],
                          inp["s_dn"], c.k)
    assert_bytes_equal(unpack_fp4(host(st["xq"])), ref["xq"], "codes")
    assert_bytes_equal(host(st["xs"]), ref["xs"], "E8M0 scales")
    for key in ("ids", "offsets", "sorted", "pos"):
        assert_bytes_equal(host(st[key]), ref[key], key)
    hq, hs = host(st["hq"]), np.ascontiguousarray(host(st["hs"]).T)
    if cfg == "moe_tiny":
        y_ref, b = grouped_gemm(hq, hs, inp["w_dn"], inp["s_dn"], ref["offsets"], with_bound=True)
        y = bf16_values(st["y"])
        check_close(y, y_ref, gemm_bound(b) + half_ulp_bf16(y_ref), "down (bf16 out)")
    else:
        rng = np.random.default_rng(21)
        rows = rng.integers(0, hq.shape[0], 2000)
        cols = rng.integers(0, c.H, 2000)
        y_ref, b = grouped_gemm_rows(hq, hs, inp["w_dn"], inp["s_dn"], ref["offsets"], rows, cols)
        y = bf16_values(st["y"])[rows, cols]
        check_close(y, y_ref, gemm_bound(b) + half_ulp_bf16(y_ref), "down sampled")
    assert cosine(bf16_values(out), ref["out"]) > 0.999


def test_layer_on_side_stream_while_current_stream_allocates():
    """moe_layer(stream=s) with torch's current stream allocating and writing memory
    while s still runs: the layer's temporaries (quantised rows, routing, intermediate
    codes, down-GEMM rows) belong to s, so the current stream cannot be handed them before
    s is done with them; the output equals the one computed on the current stream."""
    import fp8_moe_prefill_amd as f
    c = CONFIGS["moe_prefill"]
    inp = moe_inputs(c, T=1024)
    bank = f.ExpertBank.from_host(inp, "cuda:0")
    x, lg = dev(inp["x"]), dev(inp["logits"])
    ref = f.moe_layer(x, lg, bank, c.k)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(f.moe_layer(x, lg, bank, c.k, stream=s))
        # the current stream takes and overwrites memory at once (not ordered after s)
        junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda:0") for _ in range(48)]
        del junk
    s.synchronize()
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def _skewed_rows(off, rng):
    """Rows of the skewed layer to sample: the last row of every non-empty expert, the
    first and last rows of each of expert 0's 128-row tiles and around its last partial
    tile, and random rows."""
    rows = [int(off[e + 1]) - 1 for e in range(len(off) - 1) if off[e + 1] > off[e]]
    lo, hi = int(off[0]), int(off[1])
    for m in range(lo, hi, 128):
        rows += [m, min(m + 127, hi - 1)]
    rows += list(range(max(lo, hi - 20), hi))
    rows += rng.integers(0, int(off[-1]), 400).tolist()
    return np.unique(np.array(rows, np.int64))


def test_skewed_layer_gate_up_swiglu_and_tokens():
    """The skewed large layer (16384 tokens, hidden 4096, 128 Zipf-routed experts with
    empty ones, I = 1536): gate|up fp32 outputs on sampled rows (every expert's last row,
    expert 0's ~16k rows at every tile boundary) within the element bound; the fused SwiGLU
    codes and scales on those rows against the oracle's SwiGLU of the GPU's own
    accumulators; and the layer output of sampled tokens against the oracle layer run on
    those tokens (a token's output depends on its own row and routing only)."""
    import fp8_moe_prefill_amd as f
    from fp8_moe_prefill_amd import _lib
    from oracle.moe import moe_layer as oracle_layer
    from oracle.route import permute_rows
    from tests.test_gpu_grouped_gemm import _swiglu_check
    c = CONFIGS["moe_skewed"]
    inp = moe_inputs(c)
    bank = f.ExpertBank.from_host(inp, "cuda:0")
    x, lg = dev(inp["x"]), dev(inp["logits"])
    out, st = f.moe_layer(x, lg, bank, c.k, keep=True)
    R = c.T * c.k
    y32 = _lib.fp8_grouped_expert_gemm(st["xq"], st["xs"], bank.w_gu, bank.s_gu, st["offsets"],
                                       R, _lib.EPI_STORE, torch.float32, sorted_=st["sorted"],
                                       k_route=c.k, a_sums=st["xsum"])
    torch.cuda.synchronize()
    off = host(st["offsets"]).astype(np.int64)
    ids, _ = topk_route(inp["logits"], c.k)
    off_ref, sorted_, _ = group_pairs(ids, c.E)
    assert_bytes_equal(off.astype(np.int32), off_ref, "offsets")
    assert (np.diff(off) == 0).sum() >= 1 and np.diff(off).max() > 16000
    rng = np.random.default_rng(5)
    rows = _skewed_rows(off, rng)
    xq, xs = quant_group_bf16(inp["x"])
    aq, as_ = permute_rows(xq, sorted_, c.k), permute_rows(xs, sorted_, c.k)
    # gate|up: 8 random columns and the first/last gate and up columns of each sampled row
    N = 2 * c.I
    cols = np.concatenate([rng.integers(0, N, (len(rows), 8)),
                           np.tile([0, c.I - 1, c.I, N - 1], (len(rows), 1))], axis=1)
    rr = np.repeat(rows, cols.shape[1])
    cc = cols.reshape(-1)
    yr, b = grouped_gemm_rows(aq, as_, inp["w_gu"], inp["s_gu"], off_ref, rr, cc)
    y_rows = y32[torch.from_numpy(rows).cuda()].cpu().numpy()
    yg = y_rows[np.repeat(np.arange(len(rows)), cols.shape[1]), cc].astype(np.float64)
    check_close(yg, yr, gemm_bound(b), "skewed gate|up sampled")
    # the fused SwiGLU + requantisation on those rows
    hq = host(st["hq"])[rows]
    hs = np.ascontiguousarray(host(st["hs"])[:, rows].T)
    _swiglu_check(hq, hs, y_rows)
    # end to end on sampled tokens: mostly tokens routed among the popular experts, plus
    # tokens reaching the highest-index non-empty expert
    last_e = int(np.nonzero(np.diff(off) > 0)[0].max())
    popular = np.nonzero(ids.max(axis=1) < 20)[0]
    rare = np.nonzero((ids == last_e).any(axis=1))[0]
    toks = np.unique(np.concatenate([rng.choice(popular, 40, replace=False), rare[:4]]))
    ref = oracle_layer(inp["x"][toks], inp["logits"][toks], inp["w_gu"], inp["s_gu"],
                       inp["w_dn"], inp["s_dn"], c.k)
    got = bf16_values(out)[toks]
    assert cosine(got, ref["out"]) > 0.999
    for i in range(len(toks)):
        assert cosine(got[i], ref["out"][i]) > 0.99
