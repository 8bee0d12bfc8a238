"""MXFP4 activations (DeepGEMM issue 338: FP4 E2M1 activations into the grouped expert
GEMM) on the GPU vs the oracle.

* mxfp4_quant_act: E2M1 codes and E8M0 scale bytes bit-exact, on random rows spanning
  many decades, every rounding midpoint, zero / -0 / NaN / subnormal blocks, ragged K;
* mxfp4_grouped_expert_gemm (bank from fp8moe_pack_expert_bank_mxfp4): fp32 outputs
  within |gpu - oracle| <= 1e-3 * sum_k |a_k w_k| + 1e-6; bf16 = RNE(fp32); rows gathered
  through `sorted` equal a GEMM on the permuted copy, bit for bit; the SwiGLU epilogue
  against the oracle's SwiGLU on the GPU's own fp32 gate|up; the 4096-token layer's
  gate|up sampled.
"""

import numpy as np
import pytest
import torch

from oracle.moe import swiglu
from oracle.mx import grouped_gemm_fp4act, grouped_gemm_fp4act_rows, quant_mxfp4, quant_mxfp4_bf16, unpack_fp4
from oracle.numeric import bf16_bits, round_bf16
from oracle.route import group_pairs, permute_rows, topk_route
from oracle.tol import check_close, gemm_bound
from synth import CONFIGS, bf16_bits_from_f32, moe_inputs
from tests.gpu_util import assert_bytes_equal, dev, host
from tests.test_gpu_grouped_gemm import _swiglu_check

pytestmark = pytest.mark.gpu


def _lib():
    import fp8_moe_prefill_amd as f
    return f


def _quant(x_bits):
    f = _lib()
    q, s = f.mxfp4_quant_act(dev(x_bits))
    torch.cuda.synchronize()
    return unpack_fp4(host(q)), host(s)


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (64, 2048), (3, 4160)])
def test_quant_random_rows(M, K):
    rng = np.random.default_rng(M * K)
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-20, 20, (M, K // 32)).repeat(32, 1)))
    xb = bf16_bits_from_f32(x.astype(np.float32))
    q, s = _quant(xb)
    rq, rs = quant_mxfp4_bf16(xb)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s, rs, "scale bytes")


def test_quant_midpoints_and_special_blocks():
    """Every E2M1 midpoint (ties to the even code) and its neighbours, at several block
    scales; an all-zero block, a -0 block, a block with NaN, a block of bf16 subnormals."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.5, 1.0, 3.0])
    rows = []
    for e in (-3, 0, 7, 40, -60):
        for sgn in (1, -1):
            blk = np.zeros(32, np.uint16)
            blk[0] = bf16_bits_from_f32(np.float32([4.0 * 2.0 ** e]))[0]  # scale 2^e exactly
            mb = bf16_bits_from_f32((sgn * mids * 2.0 ** e).astype(np.float32))
            blk[1:1 + len(mids)] = mb
            blk[14:14 + len(mids)] = mb - 1  # one bf16 step toward zero
            blk[26:32] = mb[:6] + 1          # one bf16 step away from zero
            rows.append(blk)
    xb = np.array(rows, np.uint16).reshape(-1, 64)
    extra = np.zeros((4, 64), np.uint16)
    extra[1, :] = 0x8000                  # -0
    extra[2, :32] = bf16_bits_from_f32(np.linspace(-3, 3, 32).astype(np.float32))
    extra[2, 5] = 0x7FC0                  # NaN: skipped by the max, encodes to +0
    extra[3, :] = np.arange(1, 65, dtype=np.uint16)  # bf16 subnormals
    xb = np.vstack([xb, extra])
    q, s = _quant(xb)
    rq, rs = quant_mxfp4_bf16(xb)
    assert_bytes_equal(q, rq, "codes")
    assert_bytes_equal(s, rs, "scale bytes")
    n = xb.shape[0]
    assert np.all(q[n - 4] == 0) and np.all(q[n - 3] == 8) and q[n - 2, 5] == 0


def _mx_problem(counts, K, N, seed):
    rng = np.random.default_rng(seed)
    R, E = int(sum(counts)), len(counts)
    x = (rng.standard_normal((R, K)) * rng.uniform(0.01, 30, (R, 1))).astype(np.float32)
    codes, sc = quant_mxfp4(x)
    wp = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E, N, K // 128)).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return codes, sc, wp, ws, off


def _words_gm(sc_rows):
    """[R, K/32] E8M0 bytes of the grouped rows -> [K/128, R] 32-bit words, group-major."""
    w = np.ascontiguousarray(sc_rows).view(np.uint32)  # [R, K/128]
    return dev(np.ascontiguousarray(w.T).view(np.int32))


def _mx_gemm(codes, sc, wp, ws, off, epilogue=0, out_dtype=torch.float32, sorted_=None,
             k_route=1, R=None):
    """sc: the E8M0 bytes [rows, K/32] of the rows of `codes` -- grouped rows without
    `sorted_` (passed group-major), token rows with it (passed per token, as the quantiser
    writes them)."""
    from oracle.mx import pack_fp4
    f = _lib()
    R = codes.shape[0] if R is None else R
    w, s = f.pack_expert_bank(dev(wp), dev(ws), mxfp4=True)
    words = (_words_gm(sc) if sorted_ is None
             else dev(np.ascontiguousarray(sc).view(np.uint32).view(np.int32)))
    r = f.mxfp4_grouped_expert_gemm(dev(pack_fp4(codes)), words, w, s, dev(off),
                                    R, epilogue, out_dtype,
                                    sorted_=None if sorted_ is None else dev(sorted_),
                                    k_route=k_route)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("counts,K,N", [
    ([0, 37, 130, 1, 200], 256, 512),
    ([128, 128], 128, 256),
    ([300], 384, 64),
    ([5, 0, 0, 261, 17, 64, 0, 9], 1024, 320),
    ([1] * 16 + [2] * 16, 2048, 1536),      # decode-like: every m-tile tiny
])
def test_store_f32_within_bound(counts, K, N):
    codes, sc, wp, ws, off = _mx_problem(counts, K, N, seed=K + N)
    y = host(_mx_gemm(codes, sc, wp, ws, off)).astype(np.float64)
    ref, b = grouped_gemm_fp4act(codes, sc, wp, ws, off, with_bound=True)
    check_close(y, ref, gemm_bound(b), "mxfp4 grouped gemm fp32")


def test_bf16_output_is_rounded_fp32_output():
    codes, sc, wp, ws, off = _mx_problem([40, 0, 300, 77], 512, 256, seed=3)
    y32 = host(_mx_gemm(codes, sc, wp, ws, off)).astype(np.float64)
    y16 = host(_mx_gemm(codes, sc, wp, ws, off, out_dtype=torch.bfloat16))
    assert_bytes_equal(y16, bf16_bits(round_bf16(y32)), "bf16 = RNE(fp32)")


def _routed(cfg):
    c = CONFIGS[cfg]
    inp = moe_inputs(c)
    codes, sc = quant_mxfp4_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, _ = group_pairs(ids, c.E)
    return c, inp, codes, sc, off, sorted_


def test_gather_equals_permuted_copy_and_oracle():
    c, inp, codes, sc, off, sorted_ = _routed("moe_tiny")
    R = c.T * c.k
    ac = permute_rows(codes, sorted_, c.k)
    asc = permute_rows(sc, sorted_, c.k)
    yg = host(_mx_gemm(codes, sc, inp["w_gu"], inp["s_gu"], off, sorted_=sorted_, k_route=c.k, R=R))
    yp = host(_mx_gemm(ac, asc, inp["w_gu"], inp["s_gu"], off))
    assert_bytes_equal(yg.view(np.uint32), yp.view(np.uint32), "gather vs permuted")
    ref, b = grouped_gemm_fp4act(ac, asc, inp["w_gu"], inp["s_gu"], off, with_bound=True)
    check_close(yp.astype(np.float64), ref, gemm_bound(b), "tiny gate|up mxfp4")


def test_route_gathers_the_scale_words():
    """moe_route_permute's scale gather, fed the quantiser's E8M0 bytes viewed as 32-bit
    words, yields the group-major words of the grouped rows."""
    f = _lib()
    c = CONFIGS["moe_tiny"]
    inp = moe_inputs(c)
    q, s = f.mxfp4_quant_act(dev(inp["x"]))
    rt = f.moe_route_permute(dev(inp["logits"]), c.k, xs=s.view(torch.float32))
    torch.cuda.synchronize()
    _, rs = quant_mxfp4_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    _, sorted_, _ = group_pairs(ids, c.E)
    want = np.ascontiguousarray(permute_rows(rs, sorted_, c.k)).view(np.uint32).T
    assert_bytes_equal(host(rt["xs_perm"]).view(np.uint32), np.ascontiguousarray(want), "xs_perm words")


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_swiglu_quant_epilogue(cfg):
    c, inp, codes, sc, off, sorted_ = _routed(cfg)
    R = c.T * c.k
    hq, hs = _mx_gemm(codes, sc, inp["w_gu"], inp["s_gu"], off, epilogue=1, sorted_=sorted_,
                      k_route=c.k, R=R)
    y32 = _mx_gemm(codes, sc, inp["w_gu"], inp["s_gu"], off, sorted_=sorted_, k_route=c.k, R=R)
    _swiglu_check(host(hq), np.ascontiguousarray(host(hs).T), host(y32))


def test_gate_up_full_size_sampled():
    c, inp, codes, sc, off, sorted_ = _routed("moe_prefill")
    R = c.T * c.k
    ac = permute_rows(codes, sorted_, c.k)
    asc = permute_rows(sc, sorted_, c.k)
    y = host(_mx_gemm(codes, sc, inp["w_gu"], inp["s_gu"], off, sorted_=sorted_, k_route=c.k, R=R))
    rng = np.random.default_rng(13)
    rows = rng.integers(0, R, 4000)
    cols = rng.integers(0, 2 * c.I, 4000)
    rows[:64] = off[1:65] - 1
    ref, b = grouped_gemm_fp4act_rows(ac, asc, inp["w_gu"], inp["s_gu"], off, rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), "mxfp4 gate|up sampled")
