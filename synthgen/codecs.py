"""Encoders from float32 to the storage formats used by the inputs.

Written from the format definitions:

* bfloat16 keeps the upper 16 bits of an IEEE-754 binary32; rounding to the kept bits
  is round-to-nearest, ties-to-even.
* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
  when the exponent field is 0, no infinities, and S.1111.111 is the only NaN pattern.
  The largest finite magnitude is 1.75 * 2^8 = 448.  Encoding rounds to nearest-even
  and saturates anything at or beyond 448 to +-448.

Decoding lives in the oracle, written separately from these encoders, so that a
round-trip test checks the two against each other.
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (RNE); return the 16-bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def f32_to_e4m3fn_bits(x):
    """Round float32 values to OCP FP8 E4M3FN (RNE, saturating); return uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value cannot be encoded as E4M3FN input")
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)

    sat = a >= 448.0
    # exponent of the leading bit: a = f * 2^E with f in [0.5, 1)  ->  floor(log2 a) = E - 1
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E - 1
    sub = (a < 2.0 ** -6) & ~sat
    norm = ~sub & ~sat & (a > 0)

    # subnormals: value = q * 2^-9, q in 0..7 (q == 8 rolls into the smallest normal 0x08)
    q_sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(sub, q_sub, code)

    # normals: value = (1 + q/8) * 2^e, e in -6..8
    mant = a / np.exp2(e.astype(np.float64)) - 1.0
    q = np.rint(mant * 8.0).astype(np.int64)
    carry = q == 8
    q = np.where(carry, 0, q)
    e2 = e + carry
    ncode = ((e2 + 7) << 3) | q
    # 0x7F is NaN in this format; anything that rounds past 448 saturates
    ncode = np.where(ncode > 0x7E, 0x7E, ncode)
    code = np.where(norm, ncode, code)
    code = np.where(sat, 0x7E, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)
