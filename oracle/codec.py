"""Number formats: OCP e4m3fn, packed int4, bf16 -- oracle side (test infrastructure).

e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 15 with mantissa 7 is
NaN, there is no infinity, the largest finite magnitude is 448. The format follows from
the activation scale amax/448 in the memra-engine ``fp8_ffi`` module docs (module text:
one dynamic scale per tensor, amax/448) and from the OCP e4m3 format the FP8
grouped-expert prefill note uses (section 1).

Readings where the pages are silent (all plain IEEE-style choices):
* rounding is to nearest, ties to the even code (mantissa LSB 0);
* magnitudes above 448 saturate to 448 (no NaN from overflow);
* the sign is kept on zero: -0.0 and negatives that round to zero give 0x80;
* NaN encodes to 0x7F.

int4: two's-complement values -8..7, two per byte, the LOW nibble holding the even
index along K (the prefill note, section 1, keeps the bank packed; it is silent on the
nibble order, and low-first is the plain reading).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32 value; bf16 is the top half of an fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn byte -> float64 value, from the field definition.

    exponent field 0: subnormal m * 2^-9; otherwise (1 + m/8) * 2^(e - 7);
    e = 15, m = 7 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Value -> e4m3fn byte: round to nearest even on the e4m3 grid, saturate, keep sign.

    The grid spacing for magnitude a is 2^(floor(log2 a) - 3) in the normal range
    (a >= 2^-6) and 2^-9 in the subnormal range. ``np.rint`` rounds ties to even,
    and an even multiple of the spacing is a code with mantissa LSB 0.
    """
    x = np.asarray(v, dtype=np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    _, e = np.frexp(a)  # a = f * 2^e with f in [0.5, 1) -> floor(log2 a) = e - 1
    binade = np.maximum(e - 1, -6)
    step = np.ldexp(1.0, binade - 3)
    r = np.rint(a / step) * step  # exact: division by a power of two
    # bits of the rounded magnitude r (r <= 448, a representable e4m3 value)
    _, er = np.frexp(r)
    er = er - 1
    sub = r < 2.0 ** -6
    code_sub = np.rint(r / 2.0 ** -9)
    code_norm = ((er + 7) << 3) + np.rint((r / np.ldexp(1.0, er) - 1.0) * 8.0)
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> int4 values [..., K] (int8, -8..7), low nibble first."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    q = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    q = np.where(q >= 8, q - 16, q)  # two's-complement sign extension
    return q.astype(np.int8)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int4 values [..., K] (even K) -> packed bytes [..., K/2], low nibble = even k."""
    q = np.asarray(q, dtype=np.int16)
    assert q.shape[-1] % 2 == 0
    n = (q & 0xF).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def int4_e4m3_table() -> np.ndarray:
    """The 16-entry nibble -> e4m3 table: entry n is the e4m3 code of the int4 value
    whose two's-complement nibble is n. Every value -8..7 is exact in e4m3, which is
    what lets the prefill note (section 1) dequantise the int4 bank to e4m3 on-chip
    with no rounding."""
    nib = np.arange(16)
    return e4m3_encode(np.where(nib >= 8, nib - 16, nib).astype(np.float64))
