"""Pins of the oracle's MXFP4 activations (DeepGEMM issue 338, FP4 E2M1 activations; the
OCP MX v1.0 MXFP4 definition).

* E2M1 table: the 16 codes decode to the closed-form values (bit 3 sign, 2 exponent bits
  with bias 1, 1 mantissa bit); every grid value encodes to its own code;
* rounding: every midpoint between adjacent grid values goes to the even code, values just
  off a midpoint go to the nearer one; magnitudes above 6 saturate; -0 keeps its sign;
* block scale: amax in [2^k, 2^(k+1)) gives e = k - 2, so the block's largest element
  lands on 4 or 6; an all-zero block takes the smallest scale; a block multiplied by 2^j
  keeps its codes and moves its scale byte by j;
* closed-form error bound per element: half the grid spacing, X/4 below 2X, X/2 below
  4X, X below 6X, and under 2X in the saturated range;
* the grouped GEMM with such activations equals the e4m3 grouped GEMM (pinned on its own)
  on activations whose values both formats hold exactly.
"""

import numpy as np

from oracle.codec import e4m3_decode
from oracle.moe import grouped_gemm
from oracle.mx import (block_exponent, dequant_mxfp4, e2m1_decode, e2m1_encode,
                       grouped_gemm_fp4act, pack_fp4, quant_mxfp4, unpack_fp4)

TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_and_round_trip():
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        mag = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert e2m1_decode(np.array([c]))[0] == sign * mag == sign * TABLE[c & 7]
    assert np.array_equal(e2m1_encode(np.array(TABLE)), np.arange(8))
    assert np.array_equal(e2m1_encode(-np.array(TABLE[1:])), np.arange(9, 16))


def test_e2m1_rounding_ties_saturation_sign():
    mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for v, code in mids:
        assert e2m1_encode(np.array([v]))[0] == code, v
        assert e2m1_encode(np.array([-v]))[0] == code | 8, v
        up = np.nextafter(v, np.inf)
        dn = np.nextafter(v, -np.inf)
        hi = min(c for c in range(8) if TABLE[c] > v)
        lo = max(c for c in range(8) if TABLE[c] < v)
        assert e2m1_encode(np.array([up]))[0] == hi and e2m1_encode(np.array([dn]))[0] == lo
    assert list(e2m1_encode(np.array([6.0, 6.5, 7.99, 1e30, -1e30]))) == [7, 7, 7, 7, 15]
    assert list(e2m1_encode(np.array([-0.0, 0.0, np.nan]))) == [8, 0, 0]


def test_block_scale_rule():
    for k in range(-20, 20):
        for frac in (1.0, 1.5, 1.999):
            assert block_exponent(np.array([frac * 2.0 ** k]))[0] == k - 2
    assert block_exponent(np.array([0.0]))[0] == -127
    assert block_exponent(np.array([2.0 ** -140]))[0] == -127
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((50, 256)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    codes, sc = quant_mxfp4(x)
    blocks = np.abs(x.astype(np.float64)).reshape(50, 8, 32)
    top = np.take_along_axis(codes.reshape(50, 8, 32), blocks.argmax(2)[:, :, None], 2)[:, :, 0]
    nz = blocks.max(2) > 0
    assert np.all(np.isin(top[nz] & 7, [6, 7]))  # the largest element lands on 4 or 6
    assert sc[3, 0] == 0 and np.all(codes[3, :32] == 0)
    # scale equivariance: a block times 2^j keeps its codes, its scale byte moves by j
    x2 = x.copy()
    x2[:, 64:96] *= np.float32(2.0 ** 5)
    c2, s2 = quant_mxfp4(x2)
    assert np.array_equal(c2, codes)
    ok = nz[:, 2]
    assert np.array_equal(s2[ok, 2].astype(int), sc[ok, 2].astype(int) + 5)


def test_error_bound_and_packing():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-4, 4, (40, 1)))).astype(np.float32)
    codes, sc = quant_mxfp4(x)
    dq = dequant_mxfp4(codes, sc)
    X = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    xd = x.astype(np.float64)
    v = np.abs(xd) / X
    tol = X * np.select([v <= 2, v <= 4, v <= 6], [0.25, 0.5, 1.0], 2.0)
    assert np.all(np.abs(xd - dq) <= tol)
    assert np.array_equal(unpack_fp4(pack_fp4(codes)), codes)
    assert pack_fp4(np.array([[1, 2, 15, 0]]))[0].tolist() == [0x21, 0x0F]


def test_grouped_gemm_equals_e4m3_path_on_shared_values():
    """E2M1 values are all exact in e4m3: with unit scales on both sides the two grouped
    GEMMs must agree to rounding."""
    rng = np.random.default_rng(2)
    R, K, N, E = 40, 256, 48, 3
    codes = rng.integers(0, 16, (R, K)).astype(np.uint8)
    sc = np.full((R, K // 32), 127, np.uint8)
    vals = e2m1_decode(codes)
    enc = {float(e4m3_decode(np.array([c]))[0]): c for c in range(0x7F)}
    enc.update({-v: c | 0x80 for v, c in list(enc.items()) if v > 0})
    enc[-0.0] = 0x80
    e4 = np.vectorize(lambda v: enc[float(v)])(vals).astype(np.uint8)
    w_packed = rng.integers(0, 256, (E, N, K // 2)).astype(np.uint8)
    w_scales = rng.uniform(0.01, 0.1, (E, N, K // 128)).astype(np.float32)
    offsets = np.array([0, 13, 13, 40])
    y4 = grouped_gemm_fp4act(codes, sc, w_packed, w_scales, offsets)
    y8 = grouped_gemm(e4, np.ones((R, K // 128), np.float32), w_packed, w_scales, offsets)
    assert np.allclose(y4, y8, rtol=1e-12, atol=1e-12)
    # a power-of-two block scale multiplies that block's contribution exactly
    sc2 = sc.copy()
    sc2[:, 1] = 130
    codes2 = codes.copy()
    codes2[:, 32:64] = 0
    y_hi = grouped_gemm_fp4act(codes, sc2, w_packed, w_scales, offsets) - grouped_gemm_fp4act(codes2, sc2, w_packed, w_scales, offsets)
    y_lo = grouped_gemm_fp4act(codes, sc, w_packed, w_scales, offsets) - grouped_gemm_fp4act(codes2, sc, w_packed, w_scales, offsets)
    assert np.allclose(y_hi, 8 * y_lo, rtol=1e-12, atol=1e-12)


def test_layer_with_exactly_representable_activations():
    """Activations that MXFP4 holds exactly (E2M1 values times one power of two per
    32-block, each block's maximum 4 or 6 times it): the codes decode back to the input
    bit for bit, the gate|up GEMM equals the routed input times the dequantised bank (no
    quantisation at all), and the routing equals the e4m3 layer's."""
    from oracle.moe import dequant_bank, moe_layer
    from oracle.mx import moe_layer_mxfp4
    from synth import CONFIGS, bf16_bits_from_f32, moe_inputs
    c = CONFIGS["moe_tiny"]
    inp = moe_inputs(c)
    rng = np.random.default_rng(3)
    vals = np.array(TABLE)[rng.integers(0, 8, (c.T, c.H))] * rng.choice([-1, 1], (c.T, c.H))
    vals[:, ::32] = rng.choice([4.0, 6.0], (c.T, c.H // 32))
    pw = np.exp2(rng.integers(-6, 7, (c.T, c.H // 32))).repeat(32, axis=1)
    x = (vals * pw).astype(np.float32)
    xb = bf16_bits_from_f32(x)
    a = moe_layer_mxfp4(xb, inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"], inp["s_dn"], c.k)
    assert np.array_equal(dequant_mxfp4(a["xq"], a["xs"]), x.astype(np.float64))
    xp = x.astype(np.float64)[a["sorted"] // c.k]
    for e in range(c.E):
        lo, hi = a["offsets"][e], a["offsets"][e + 1]
        want = xp[lo:hi] @ dequant_bank(inp["w_gu"][e], inp["s_gu"][e]).T
        assert np.allclose(a["y_gu"][lo:hi], want, rtol=1e-12, atol=1e-9)
    b = moe_layer(xb, inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"], inp["s_dn"], c.k)
    for key in ("ids", "offsets", "sorted", "pos"):
        assert np.array_equal(a[key], b[key])
