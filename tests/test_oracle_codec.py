"""Pins of the oracle's number formats against things other than itself.

* e4m3 decode: torch's float8_e4m3fn (an independent library implementation) on all 256
  codes, and the format's fixed points (max 448, min subnormal 2^-9, NaN codes).
* e4m3 encode: a brute-force nearest-code search (ties to the even code, saturation at
  448) over every finite bf16 bit pattern at several scales and over random fp32, and
  torch's clamp-then-cast.
* int4: pack/unpack round trip, sign extension, and the 16-entry table checked by decode.
"""

import os

import numpy as np
import pytest
import torch

from oracle.codec import (bf16_to_f32, e4m3_decode, e4m3_encode, int4_e4m3_table,
                          pack_int4, unpack_int4)


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_all_codes():
    ours = e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_fixed_points():
    d = e4m3_decode(np.array([0x7E, 0x01, 0x08, 0x38, 0x7F, 0xFF, 0xFE, 0x07], np.uint8))
    assert d[0] == 448.0 and d[1] == 2.0 ** -9 and d[2] == 2.0 ** -6 and d[3] == 1.0
    assert np.isnan(d[4]) and np.isnan(d[5]) and d[6] == -448.0 and d[7] == 7 * 2.0 ** -9
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)  # codes 0..126 are strictly increasing


def test_encode_decode_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def _brute_encode(v):
    """Nearest finite code by exhaustive distance; ties to the code with LSB 0."""
    v = np.asarray(v, np.float64)
    mags = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    out = np.empty(v.shape, np.uint8)
    flat = v.reshape(-1)
    res = out.reshape(-1)
    for s in range(0, flat.size, 1 << 16):
        a = np.abs(flat[s:s + (1 << 16)])
        d = np.abs(a[:, None] - mags[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among equal-distance codes take the even one
        even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        # saturation: anything past 448 is 448 (the nearest finite code is 448 anyway)
        pick = np.where(a > 448.0, 0x7E, pick)
        res[s:s + (1 << 16)] = pick | (np.signbit(flat[s:s + (1 << 16)]) << 7)
    return out


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 3.0 / 7.0, 2.0 ** 5, 1e-3])
def test_encode_vs_brute_force_all_bf16(scale):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f32(bits).astype(np.float64)
    v = v[np.isfinite(v)] * scale
    assert np.array_equal(e4m3_encode(v), _brute_encode(v))


def test_encode_vs_brute_force_random_fp32():
    rng = np.random.default_rng(123)
    v = (rng.standard_normal(400_000) * np.exp(rng.uniform(-12, 7, 400_000))).astype(np.float32)
    assert np.array_equal(e4m3_encode(v), _brute_encode(v.astype(np.float64)))


def test_encode_vs_torch_clamp_cast():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-14, 8, 1_000_000))).astype(np.float32)
    v[:4] = [0.0, -0.0, 500.0, -1e-9]
    ref = torch.clamp(torch.from_numpy(v), -448.0, 448.0).to(torch.float8_e4m3fn)
    assert np.array_equal(e4m3_encode(v), ref.view(torch.uint8).numpy())


def test_encode_special_values():
    v = np.array([np.nan, -0.0, 0.0, 1e30, -1e30, 464.0, 2.0 ** -10, -2.0 ** -10,
                  3 * 2.0 ** -11, 3 * 2.0 ** -10, 2.0 ** -10 + 2.0 ** -30, 17.0, 18.0])
    # 2^-10 is half the smallest subnormal: a tie, to the even code 0 (sign kept);
    # 1.5 * 2^-9 is a tie between codes 1 and 2 -> 2; 17 is a tie between 16 (0x58,
    # e=11 m=0) and 18 (0x59) -> 0x58
    assert list(e4m3_encode(v)) == [0x7F, 0x80, 0x00, 0x7E, 0xFE, 0x7E, 0x00, 0x80, 0x01,
                                    0x02, 0x01, 0x58, 0x59]


def test_int4_unpack_sign_extension_and_order():
    # byte 0x8F: low nibble 0xF = -1 (even k), high nibble 0x8 = -8 (odd k)
    assert list(unpack_int4(np.array([0x8F, 0x70, 0x12], np.uint8))) == [-1, -8, 0, 7, 2, 1]
    # bit-level: every value at every position of a 4-byte row, one at a time
    for pos in range(8):
        for v in range(-8, 8):
            q = np.zeros(8, np.int8)
            q[pos] = v
            b = np.zeros(4, np.uint8)
            b[pos // 2] = (v & 0xF) << (4 * (pos % 2))
            assert list(unpack_int4(b)) == list(q)


def test_int4_pack_unpack_round_trip():
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, size=(5, 7, 256)).astype(np.int8)
    assert np.array_equal(unpack_int4(pack_int4(q)), q)
    b = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    assert np.array_equal(pack_int4(unpack_int4(b)), b)


def test_nibble_table_is_exact():
    t = int4_e4m3_table()
    nib = np.arange(16)
    assert np.array_equal(_torch_decode_all()[t], np.where(nib >= 8, nib - 16, nib))
    path = os.path.join(os.path.dirname(__file__), "golden", "int4_e4m3_table.txt")
    lines = [ln for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert [int(g, 16) for g in lines[0].split()] == list(t)
