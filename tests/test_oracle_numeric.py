"""Pins of the oracle's numeric helpers (round_bf16, half_ulp_bf16) against torch's own
fp32 -> bf16 conversion and against the bf16 grid read off the bit patterns.

* round_bf16 on fp32 values equals torch's round-to-nearest-even cast, bit for bit, over
  random fp32 bit patterns of the normal range, exact ties (lower 16 bits 0x8000, both
  parities of the kept LSB), values just below a power of two that round up into the next
  binade, negatives and zero (the sign of zero is kept);
* round_bf16 on float64 values equals the nearer of the two bf16 neighbours (ties to the
  even one), found by brute force from the bit grid;
* half_ulp_bf16(b) is half the distance from a bf16 value b to the next one away from
  zero, read off the bit patterns (b and b + 1 ulp), for every normal bf16 exponent.
"""

import numpy as np
import torch

from oracle.numeric import round_bf16
from oracle.tol import half_ulp_bf16


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.to(torch.float32).numpy().astype(np.float64)


def _normal_f32_bits(rng, n):
    # exponent field 1..253 keeps the value and its bf16 rounding in the normal range
    sign = rng.integers(0, 2, n, dtype=np.uint32) << np.uint32(31)
    exp = rng.integers(1, 254, n, dtype=np.uint32) << np.uint32(23)
    man = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    return sign | exp | man


def test_round_bf16_matches_torch_cast_on_fp32():
    rng = np.random.default_rng(0)
    bits = _normal_f32_bits(rng, 200_000)
    x = bits.view(np.float32)
    got = round_bf16(x.astype(np.float64))
    ref = _torch_bf16(x)
    assert np.array_equal(got, ref)


def test_round_bf16_ties_to_even():
    rng = np.random.default_rng(1)
    hi = _normal_f32_bits(rng, 50_000) & np.uint32(0xFFFF0000)
    tie = hi | np.uint32(0x8000)  # exactly half way between two bf16 values
    x = tie.view(np.float32)
    got = round_bf16(x.astype(np.float64))
    assert np.array_equal(got, _torch_bf16(x))
    # the result has an even kept mantissa: bit 16 of the pattern is clear
    gbits = got.astype(np.float32).view(np.uint32)
    assert np.all((gbits >> np.uint32(16)) & np.uint32(1) == 0)
    # below the tie rounds down, above rounds up
    lo = (tie - np.uint32(1)).view(np.float32)
    up = (tie + np.uint32(1)).view(np.float32)
    assert np.array_equal(round_bf16(lo.astype(np.float64)), hi.view(np.float32).astype(np.float64))
    nxt = (hi + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    assert np.array_equal(round_bf16(up.astype(np.float64)), nxt)


def test_round_bf16_binade_crossing_signs_and_zero():
    e = np.arange(-120, 120)
    below = np.nextafter(np.ldexp(1.0, e).astype(np.float32), np.float32(0))  # just below 2^e
    for sgn in (1.0, -1.0):
        x = (sgn * below).astype(np.float32)
        got = round_bf16(x.astype(np.float64))
        assert np.array_equal(got, _torch_bf16(x))
        assert np.array_equal(got, sgn * np.ldexp(1.0, e))  # rounds up into the next binade
    z = round_bf16(np.array([0.0, -0.0]))
    assert z[0] == 0 and z[1] == 0 and not np.signbit(z[0]) and np.signbit(z[1])


def test_round_bf16_float64_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20_000) * np.exp2(rng.integers(-60, 60, 20_000))
    got = round_bf16(x)
    # the two bf16 neighbours of x from the truncated fp32 bit pattern
    f = x.astype(np.float32)
    b = f.view(np.uint32) & np.uint32(0xFFFF0000)
    cand = np.stack([(b - np.uint32(0x10000)).view(np.float32), b.view(np.float32),
                     (b + np.uint32(0x10000)).view(np.float32),
                     (b + np.uint32(0x20000)).view(np.float32)], 1).astype(np.float64)
    cb = cand.astype(np.float32).view(np.uint32)
    d = np.abs(cand - x[:, None])
    best = d.min(axis=1, keepdims=True)
    # among the nearest candidates take the even one (bit 16 clear)
    ok = (d == best) & (((cb >> np.uint32(16)) & np.uint32(1)) == 0)
    ok |= (d == best) & ((d == best).sum(axis=1, keepdims=True) == 1)
    ref = cand[np.arange(len(x)), ok.argmax(axis=1)]
    assert np.array_equal(got, ref)


def test_half_ulp_bf16_from_bit_grid():
    rng = np.random.default_rng(3)
    exp = np.arange(1, 254, dtype=np.uint32)
    man = rng.integers(0, 128, exp.size, dtype=np.uint32)
    for sign in (0, 1):
        bits16 = (np.uint32(sign) << np.uint32(15)) | (exp << np.uint32(7)) | man
        b = (bits16 << np.uint32(16)).view(np.float32).astype(np.float64)
        nxt = ((bits16 + np.uint32(1)) << np.uint32(16)).view(np.float32).astype(np.float64)
        assert np.array_equal(half_ulp_bf16(b), np.abs(nxt - b) / 2)
        # closed form 2^(e - 127 - 8) for the biased exponent e
        assert np.array_equal(half_ulp_bf16(b), np.ldexp(1.0, exp.astype(np.int64) - 127 - 8))
    assert half_ulp_bf16(np.array([0.0]))[0] == 0.0
