"""fp8_grouped_expert_gemm on the GPU vs the oracle.

The bank is the oracle's canonical one, put into the kernel's layout on the device by
fp8moe_pack_expert_bank; activation scales go in group-major ([K/128, R], grouped row
order), the SwiGLU epilogue's scales come back group-major.

Floating outputs: |gpu - oracle| <= 1e-3 * sum_k |a_k w_k| + 1e-6 per element (fp32
output); the bf16 output equals the fp32 output rounded to nearest even, bit for bit.
SwiGLU + requantisation: checked against the oracle's SwiGLU applied to the GPU's own fp32
gate/up accumulators (same kernel, same accumulation order), where a code may differ only
by one step and only next to a rounding midpoint.
"""

import numpy as np
import pytest
import torch

from oracle.codec import e4m3_decode, e4m3_encode
from oracle.moe import grouped_gemm, grouped_gemm_rows, swiglu
from oracle.numeric import bf16_bits
from oracle.numeric import round_bf16
from oracle.quant import quant_group, quant_group_bf16
from oracle.route import group_pairs, permute_rows, topk_route
from oracle.tol import check_close, gemm_bound
from synth import CONFIGS, moe_inputs
from tests.gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _lib():
    import fp8_moe_prefill_amd as f
    return f


def _problem(counts, K, N, seed=0, scale_spread=True):
    rng = np.random.default_rng(seed)
    R = int(sum(counts))
    E = len(counts)
    x = rng.standard_normal((R, K)).astype(np.float32)
    if scale_spread:
        x *= rng.uniform(0.01, 30, (R, 1)).astype(np.float32)
    aq, as_ = quant_group(x)
    wp = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E, N, K // 128)).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return aq, as_, wp, ws, off


def _bank(wp, ws):
    f = _lib()
    return f.pack_expert_bank(dev(wp), dev(ws))


def _gm(scales_rows):
    """[R, K/128] scales in grouped row order -> the group-major device layout."""
    return dev(np.ascontiguousarray(scales_rows.T))


def _gemm(aq, as_, wp, ws, off, out_dtype=torch.float32, sorted_=None, k_route=1,
          R=None):
    """STORE-mode grouped GEMM. as_: [rows, K/128] scales of the rows of aq -- the grouped
    rows without `sorted_` (passed group-major), the token rows with it (passed as they
    are)."""
    f = _lib()
    R = aq.shape[0] if R is None else R
    w, s = _bank(wp, ws)
    y = f.fp8_grouped_expert_gemm(dev(aq), _gm(as_) if sorted_ is None else dev(as_), w, s,
                                  dev(off), R,
                                  f.EPI_STORE, out_dtype,
                                  sorted_=None if sorted_ is None else dev(sorted_),
                                  k_route=k_route)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("counts,K,N", [
    ([0, 37, 130, 1, 200], 256, 512),      # empty, ragged, single-row experts
    ([128, 128], 128, 256),                 # exact tiles, one K group
    ([300], 384, 64),                       # one expert, one 64-column group
    ([5, 0, 0, 261, 17, 64, 0, 9], 1024, 320),  # N not a multiple of the 256-wide tile
])
def test_store_f32_within_bound(counts, K, N):
    aq, as_, wp, ws, off = _problem(counts, K, N, seed=K + N)
    y = host(_gemm(aq, as_, wp, ws, off)).astype(np.float64)
    ref, b = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    check_close(y, ref, gemm_bound(b), "grouped gemm fp32")


def test_bf16_output_is_rounded_fp32_output():
    aq, as_, wp, ws, off = _problem([40, 0, 300, 77], 512, 256, seed=3)
    y32 = host(_gemm(aq, as_, wp, ws, off, torch.float32)).astype(np.float64)
    y16 = host(_gemm(aq, as_, wp, ws, off, torch.bfloat16))
    assert_bytes_equal(y16, bf16_bits(round_bf16(y32)), "bf16 = RNE(fp32)")


def test_integer_operands_exact():
    """Integer activations (exact in e4m3) with unit scales: every partial sum is an
    integer below 2^24, so the fp32 result must be exact."""
    rng = np.random.default_rng(4)
    R, K, N = 200, 512, 128
    aq = e4m3_encode(rng.integers(-16, 17, size=(R, K)).astype(np.float64))
    as_ = np.ones((R, K // 128), np.float32)
    wp = rng.integers(0, 256, size=(3, N, K // 2), dtype=np.uint8)
    ws = np.ones((3, N, K // 128), np.float32)
    off = np.array([0, 60, 61, R], np.int32)
    y = host(_gemm(aq, as_, wp, ws, off)).astype(np.float64)
    ref = grouped_gemm(aq, as_, wp, ws, off)
    assert np.array_equal(y, ref)


def test_on_the_fly_gather_equals_permuted_copy():
    """Rows gathered from token order through `sorted` give the same bits as a GEMM on
    the explicitly permuted activations."""
    c = CONFIGS["moe_tiny"]
    inp = moe_inputs(c)
    xq, xs = quant_group_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, _ = group_pairs(ids, c.E)
    R = c.T * c.k
    aq = permute_rows(xq, sorted_, c.k)
    as_ = permute_rows(xs, sorted_, c.k)
    y_gather = host(_gemm(xq, xs, inp["w_gu"], inp["s_gu"], off, sorted_=sorted_, k_route=c.k,
                          R=R))
    y_perm = host(_gemm(aq, as_, inp["w_gu"], inp["s_gu"], off))
    assert_bytes_equal(y_gather.view(np.uint32), y_perm.view(np.uint32), "gather vs permuted")
    ref, b = grouped_gemm(aq, as_, inp["w_gu"], inp["s_gu"], off, with_bound=True)
    check_close(y_perm.astype(np.float64), ref, gemm_bound(b), "tiny gate|up")


def _swiglu_check(hq, hs, y_gu32):
    """Codes/scales of the SwiGLU epilogue vs the oracle's SwiGLU on the GPU's own fp32
    gate|up accumulators."""
    h = swiglu(y_gu32.astype(np.float64)).astype(np.float32)
    rq, rs = quant_group(h)
    # scales: exact unless the amax element's h differs in its last bits (fp32 silu)
    ds = np.abs(hs.astype(np.float64) - rs) / rs
    assert ds.max() <= 4e-6, ds.max()
    same = hq == rq
    # fewer than 1e-4 of the codes may differ (an fp32 discrepancy of about 1e-6 relative
    # against a code spacing of 2^-4 flags about 2e-5 of them), each one only by the
    # rounding-boundary rule below
    miss = 1.0 - same.mean()
    assert miss < 1e-4, miss
    if not same.all():
        i = np.nonzero(~same)
        # adjacent codes only (same sign; code indices one apart)
        def idx(c):  # position on the signed code line; +0 and -0 coincide
            c = c.astype(np.int64)
            return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
        assert np.all(np.abs(idx(hq[i]) - idx(rq[i])) <= 1)
        # and the oracle's pre-quantisation value sits next to the midpoint of the two
        G = hs.shape[1]
        hg = h.reshape(h.shape[0], G, 128)
        amax = np.maximum(np.abs(hg).max(axis=2), np.float32(1e-12)).astype(np.float32)
        inv = (np.float32(448.0) / amax).astype(np.float32)
        u = (hg * inv[:, :, None]).astype(np.float32).reshape(h.shape)[i].astype(np.float64)
        mid = 0.5 * (e4m3_decode(hq[i]) + e4m3_decode(rq[i]))
        assert np.all(np.abs(np.abs(u) - np.abs(mid)) <= 1e-5 * np.abs(u) + 1e-9)


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_swiglu_quant_epilogue(cfg):
    c = CONFIGS[cfg]
    inp = moe_inputs(c)
    f = _lib()
    xq, xs = quant_group_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, _ = group_pairs(ids, c.E)
    R = c.T * c.k
    w, s = _bank(inp["w_gu"], inp["s_gu"])
    args = (dev(xq), dev(xs), w, s, dev(off), R)
    hq, hs = f.fp8_grouped_expert_gemm(*args, f.EPI_SWIGLU_QUANT, sorted_=dev(sorted_),
                                       k_route=c.k)
    y32 = f.fp8_grouped_expert_gemm(*args, f.EPI_STORE, torch.float32, sorted_=dev(sorted_),
                                    k_route=c.k)
    torch.cuda.synchronize()
    assert tuple(hs.shape) == (c.I // 128, R)
    _swiglu_check(host(hq), np.ascontiguousarray(host(hs).T), host(y32))


def test_gate_up_full_size_sampled():
    """Gate|up GEMM of the 4096-token, 64-expert layer (fp32 out) on 4000 sampled outputs,
    each computed by the oracle one at a time."""
    c = CONFIGS["moe_prefill"]
    inp = moe_inputs(c)
    xq, xs = quant_group_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, _ = group_pairs(ids, c.E)
    R = c.T * c.k
    aq = permute_rows(xq, sorted_, c.k)
    as_ = permute_rows(xs, sorted_, c.k)
    y = host(_gemm(xq, xs, inp["w_gu"], inp["s_gu"], off, sorted_=sorted_, k_route=c.k, R=R))
    rng = np.random.default_rng(11)
    rows = rng.integers(0, R, 4000)
    cols = rng.integers(0, 2 * c.I, 4000)
    rows[:64] = off[1:65] - 1  # last row of every expert
    ref, b = grouped_gemm_rows(aq, as_, inp["w_gu"], inp["s_gu"], off, rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), "gate|up sampled")


def test_down_full_size_sampled():
    """Down GEMM (K = 768) of the same layer on the GPU's own intermediate codes."""
    c = CONFIGS["moe_prefill"]
    inp = moe_inputs(c)
    f = _lib()
    rng = np.random.default_rng(12)
    R = c.T * c.k
    counts = np.bincount(rng.integers(0, c.E, R), minlength=c.E)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    h = (rng.standard_normal((R, c.I)) * rng.uniform(0.1, 10, (R, 1))).astype(np.float32)
    hq, hs = quant_group(h)
    y = host(_gemm(hq, hs, inp["w_dn"], inp["s_dn"], off, torch.float32))
    rows = rng.integers(0, R, 4000)
    cols = rng.integers(0, c.H, 4000)
    ref, b = grouped_gemm_rows(hq, hs, inp["w_dn"], inp["s_dn"], off, rows, cols)
    check_close(y[rows, cols].astype(np.float64), ref, gemm_bound(b), "down sampled")


def test_repeat_runs_identical():
    aq, as_, wp, ws, off = _problem([100, 3, 250], 256, 256, seed=9)
    a = host(_gemm(aq, as_, wp, ws, off))
    b = host(_gemm(aq, as_, wp, ws, off))
    assert_bytes_equal(a.view(np.uint32), b.view(np.uint32), "repeat")


def test_pack_expert_bank_layout():
    """The packed bank holds exactly the canonical int4 values at the documented
    positions, and the scales are transposed (decoded here from the header's description
    of the layout, independently of the kernels)."""
    f = _lib()
    rng = np.random.default_rng(5)
    E, N, K = 3, 128, 384
    wp = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E, N, K // 128)).astype(np.float32)
    pw, ps = f.pack_expert_bank(dev(wp), dev(ws))
    torch.cuda.synchronize()
    pw, ps = host(pw).reshape(-1), host(ps)
    from oracle.codec import unpack_int4
    q = unpack_int4(wp)  # [E, N, K] canonical values
    G = K // 128
    got = np.empty_like(q)
    for e in range(E):
        for c in range(N // 16):
            for g in range(G):
                blk = pw[((e * (N // 16) + c) * G + g) * 1024:][:1024]
                for h in range(4):
                    for i in range(16):
                        b16 = blk[16 * (16 * h + i):][:16]
                        for j in range(4):
                            for b in range(4):
                                byte = int(b16[4 * j + b])
                                k0 = 128 * g + 32 * h + 8 * j
                                for kk, nib in ((k0 + b, byte & 15), (k0 + 4 + b, byte >> 4)):
                                    n = 64 * (c // 4) + 4 * i + c % 4
                                    got[e, n, kk] = nib - 16 if nib >= 8 else nib
    assert np.array_equal(got, q)
    assert np.array_equal(ps, np.transpose(ws, (0, 2, 1)))


def _sums_gm(aq):
    """Oracle code sums of the grouped rows, group-major fp32 on the device."""
    from oracle.quant import code_sums
    return _gm(code_sums(aq).astype(np.float32))


@pytest.mark.parametrize("counts,K,N", [
    ([0, 37, 130, 1, 200], 256, 512),
    ([5, 0, 0, 261, 17, 64, 0, 9], 1024, 320),
])
def test_store_with_given_code_sums(counts, K, N):
    """a_sums in place of the in-kernel sums: within the same bound of the oracle. (Not bit
    for bit the result without them: the sum the kernel forms on the matrix core is not
    always the exact sum of the 128 codes, the given one is.)"""
    f = _lib()
    aq, as_, wp, ws, off = _problem(counts, K, N, seed=K + N + 1)
    w, s = _bank(wp, ws)
    args = (dev(aq), _gm(as_), w, s, dev(off), aq.shape[0], f.EPI_STORE, torch.float32)
    y1 = host(f.fp8_grouped_expert_gemm(*args, a_sums=_sums_gm(aq)))
    torch.cuda.synchronize()
    ref, b = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    check_close(y1.astype(np.float64), ref, gemm_bound(b), "grouped gemm with a_sums")


def test_integer_operands_exact_with_given_sums():
    """The exactness case above with the sums given: every term is an integer, so the
    result must be exact."""
    f = _lib()
    rng = np.random.default_rng(4)
    R, K, N = 200, 512, 128
    aq = e4m3_encode(rng.integers(-16, 17, size=(R, K)).astype(np.float64))
    as_ = np.ones((R, K // 128), np.float32)
    wp = rng.integers(0, 256, size=(3, N, K // 2), dtype=np.uint8)
    ws = np.ones((3, N, K // 128), np.float32)
    off = np.array([0, 60, 61, R], np.int32)
    w, s = _bank(wp, ws)
    y = host(f.fp8_grouped_expert_gemm(dev(aq), _gm(as_), w, s, dev(off), R, f.EPI_STORE,
                                       torch.float32, a_sums=_sums_gm(aq)))
    torch.cuda.synchronize()
    assert np.array_equal(y.astype(np.float64), grouped_gemm(aq, as_, wp, ws, off))


def test_wrong_code_sums_change_the_result():
    """The kernel really reads a_sums: sums off by one unit shift the outputs (the offset
    term of the int4 weights), so the result differs from the one with the right sums."""
    f = _lib()
    aq, as_, wp, ws, off = _problem([200, 56], 256, 256, seed=21)
    w, s = _bank(wp, ws)
    args = (dev(aq), _gm(as_), w, s, dev(off), aq.shape[0], f.EPI_STORE, torch.float32)
    from oracle.quant import code_sums
    bad = _gm((code_sums(aq) + 1.0).astype(np.float32))
    y0 = host(f.fp8_grouped_expert_gemm(*args, a_sums=_sums_gm(aq)))
    y1 = host(f.fp8_grouped_expert_gemm(*args, a_sums=bad))
    torch.cuda.synchronize()
    assert not np.array_equal(y0, y1)


@pytest.mark.parametrize("cfg", ["moe_tiny", "moe_prefill"])
def test_swiglu_epilogue_code_sums(cfg):
    """Gate|up with given input sums and the SwiGLU epilogue's optional output sums: the
    codes and scales pass the SwiGLU check against the same kernel's fp32 accumulators
    (also run with the given sums); each output sum is the sum of the decoded output codes
    of its (row, 128 group) to fp32 summation accuracy; and the down GEMM fed those sums
    stays within the bound of the oracle on those codes."""
    c = CONFIGS[cfg]
    inp = moe_inputs(c)
    f = _lib()
    from oracle.codec import e4m3_decode
    from oracle.quant import code_sums
    xq, xs = quant_group_bf16(inp["x"])
    ids, _ = topk_route(inp["logits"], c.k)
    off, sorted_, _ = group_pairs(ids, c.E)
    R = c.T * c.k
    w, s = _bank(inp["w_gu"], inp["s_gu"])
    args = (dev(xq), dev(xs), w, s, dev(off), R)
    kw = dict(sorted_=dev(sorted_), k_route=c.k, a_sums=dev(code_sums(xq).astype(np.float32)))
    hq, hs, hsum = f.fp8_grouped_expert_gemm(*args, f.EPI_SWIGLU_QUANT, **kw, with_sums=True)
    y32 = f.fp8_grouped_expert_gemm(*args, f.EPI_STORE, torch.float32, **kw)
    torch.cuda.synchronize()
    codes = host(hq)
    _swiglu_check(codes, np.ascontiguousarray(host(hs).T), host(y32))
    ref = code_sums(codes).T
    err = np.abs(host(hsum).astype(np.float64) - ref)
    bound = 8 * 2.0 ** -24 * np.abs(e4m3_decode(codes)).reshape(R, -1, 128).sum(-1).T
    assert np.all(err <= bound), err.max()
    wd, sd = _bank(inp["w_dn"], inp["s_dn"])
    y = host(f.fp8_grouped_expert_gemm(hq, hs, wd, sd, dev(off), R, f.EPI_STORE, torch.float32,
                                       a_sums=hsum))
    torch.cuda.synchronize()
    hs_rows = np.ascontiguousarray(host(hs).T)
    rng = np.random.default_rng(13)
    rows = rng.integers(0, R, 3000)
    cols = rng.integers(0, c.H, 3000)
    dref, db = grouped_gemm_rows(codes, hs_rows, inp["w_dn"], inp["s_dn"], off, rows, cols)
    check_close(y[rows, cols].astype(np.float64), dref, gemm_bound(db), "down with given sums")


@pytest.mark.parametrize("k", [3, 6])
def test_gather_with_k_not_a_power_of_two(k):
    """Rows, scales and code sums gathered through `sorted` with k = 3 and 6 (pair id / k by
    division, not a shift): bit for bit the GEMM on explicitly permuted copies, for STORE and
    for the SwiGLU epilogue."""
    f = _lib()
    from oracle.quant import code_sums
    rng = np.random.default_rng(30 + k)
    T, H, E, I = 50, 256, 8, 256
    x = (rng.standard_normal((T, H)) * rng.uniform(0.1, 10, (T, 1))).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    xq, xs = quant_group(x)
    ids, _ = topk_route(logits, k)
    off, sorted_, _ = group_pairs(ids, E)
    R = T * k
    wp = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E, 2 * I, H // 128)).astype(np.float32)
    w, s = _bank(wp, ws)
    aq, as_ = permute_rows(xq, sorted_, k), permute_rows(xs, sorted_, k)
    sums_tok = dev(code_sums(xq).astype(np.float32))
    sums_grp = _sums_gm(aq)
    for epi in (f.EPI_STORE, f.EPI_SWIGLU_QUANT):
        g = f.fp8_grouped_expert_gemm(dev(xq), dev(xs), w, s, dev(off), R, epi, torch.float32,
                                      sorted_=dev(sorted_), k_route=k, a_sums=sums_tok)
        p = f.fp8_grouped_expert_gemm(dev(aq), _gm(as_), w, s, dev(off), R, epi, torch.float32,
                                      a_sums=sums_grp)
        torch.cuda.synchronize()
        for a, b in (zip(g, p) if epi == f.EPI_SWIGLU_QUANT else [(g, p)]):
            assert_bytes_equal(host(a).view(np.uint8), host(b).view(np.uint8), f"epi {epi}")
    y = host(f.fp8_grouped_expert_gemm(dev(xq), dev(xs), w, s, dev(off), R, f.EPI_STORE,
                                       torch.float32, sorted_=dev(sorted_), k_route=k))
    torch.cuda.synchronize()
    ref, b = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    check_close(y.astype(np.float64), ref, gemm_bound(b), f"gather k={k}")


@pytest.mark.parametrize("counts,K,N", [
    ([17, 0, 23], 16384, 64),                     # the largest K the entry point takes
    ([0] * 500 + [3] + [0] * 400 + [130] + [0] * 121 + [1], 256, 128),  # E = 1024
])
def test_limits_of_k_and_expert_count(counts, K, N):
    """At the documented limits: K = 16384 (128 groups streamed per tile) and E = 1024
    experts, nearly all empty, with a ragged tail in the few that have rows."""
    assert len(counts) in (3, 1024)
    aq, as_, wp, ws, off = _problem(counts, K, N, seed=K + len(counts))
    y = host(_gemm(aq, as_, wp, ws, off)).astype(np.float64)
    ref, b = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    check_close(y, ref, gemm_bound(b), f"grouped gemm K={K} E={len(counts)}")


def _pad_experts(wp, ws, off, pad):
    """The same problem with `pad` empty experts appended (never read: no rows)."""
    wp_p = np.concatenate([wp, np.zeros((pad,) + wp.shape[1:], wp.dtype)])
    ws_p = np.concatenate([ws, np.ones((pad,) + ws.shape[1:], ws.dtype)])
    off_p = np.concatenate([off, np.full(pad, off[-1], np.int32)])
    return wp_p, ws_p, off_p


def _all_outputs(f, args, a_sums, **kw):
    y32 = f.fp8_grouped_expert_gemm(*args, f.EPI_STORE, torch.float32, a_sums=a_sums, **kw)
    y16 = f.fp8_grouped_expert_gemm(*args, f.EPI_STORE, torch.bfloat16, a_sums=a_sums, **kw)
    hq, hs, hsum = f.fp8_grouped_expert_gemm(*args, f.EPI_SWIGLU_QUANT, a_sums=a_sums,
                                             with_sums=True, **kw)
    torch.cuda.synchronize()
    return [host(t) for t in (y32, y16, hq, hs, hsum)]


ROWS16_PER_EXPERT = 16  # the launcher takes the 16-row-unit kernel when R <= 16 E


@pytest.mark.parametrize("sums", [False, True])
def test_rows16_kernel_equals_tile_kernel(sums):
    """A few routed rows per expert (R <= 16 E) take the kernel of 16-row units; the same
    problem with its trailing empty experts dropped (R > 16 E) takes the 128-row-tile
    kernel. Both form every output with the same MFMAs, seeds and fold, so the fp32, bf16
    and SwiGLU outputs (codes, scales, code sums) must agree bit for bit; the fp32 output is
    also checked against the oracle. Experts of 37 and 35 rows span three units each, the
    last ragged."""
    f = _lib()
    counts = [5, 37, 1, 35]  # R = 78 > 16 * 4; with one empty expert more, 78 <= 80
    K, N = 512, 512
    aq, as_, wp, ws, off = _problem(counts, K, N, seed=77)
    R = int(sum(counts))
    assert R > ROWS16_PER_EXPERT * len(counts) and R <= ROWS16_PER_EXPERT * (len(counts) + 1)
    wp_p, ws_p, off_p = _pad_experts(wp, ws, off, 1)
    a_sums = _sums_gm(aq) if sums else None
    outs = []
    for wpx, wsx, offx in ((wp, ws, off), (wp_p, ws_p, off_p)):
        w, s = _bank(wpx, wsx)
        outs.append(_all_outputs(f, (dev(aq), _gm(as_), w, s, dev(offx), R), a_sums))
    for name, a, b in zip(("fp32", "bf16", "codes", "scales", "code sums"), *outs):
        assert_bytes_equal(a.view(np.uint8), b.view(np.uint8), f"16-row units vs tiles: {name}")
    ref, bnd = grouped_gemm(aq, as_, wp, ws, off, with_bound=True)
    check_close(outs[1][0].astype(np.float64), ref, gemm_bound(bnd), "16-row units fp32")


def test_rows16_kernel_gather_equals_tile_kernel():
    """The same comparison with the rows gathered from token order through `sorted` and
    per-token scales and code sums (the layer's gate|up call): 25 tokens, top-4 of 6
    experts (R = 100 > 96), then of the same 6 plus one empty expert (100 <= 112)."""
    f = _lib()
    rng = np.random.default_rng(78)
    T, k, E0, K, N = 25, 4, 6, 384, 256
    assert T * k > ROWS16_PER_EXPERT * E0 and T * k <= ROWS16_PER_EXPERT * (E0 + 1)
    x = (rng.standard_normal((T, K)) * rng.uniform(0.1, 10, (T, 1))).astype(np.float32)
    xq, xs = quant_group(x)
    ids = np.stack([rng.permutation(E0)[:k] for _ in range(T)]).astype(np.int32)
    from oracle.quant import code_sums
    xsum = code_sums(xq).astype(np.float32)
    wp = rng.integers(0, 256, size=(E0, N, K // 2), dtype=np.uint8)
    ws = rng.uniform(0.005, 0.02, size=(E0, N, K // 128)).astype(np.float32)
    outs = []
    for E in (E0, E0 + 1):
        off, sorted_, _ = group_pairs(ids, E)
        wpx, wsx, _ = _pad_experts(wp, ws, off[:E0 + 1], E - E0)
        w, s = _bank(wpx, wsx)
        outs.append(_all_outputs(f, (dev(xq), dev(xs), w, s, dev(off), T * k), dev(xsum),
                                 sorted_=dev(sorted_), k_route=k))
    for name, a, b in zip(("fp32", "bf16", "codes", "scales", "code sums"), *outs):
        assert_bytes_equal(a.view(np.uint8), b.view(np.uint8), f"gather, 16-row units vs tiles: {name}")
