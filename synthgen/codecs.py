"""Encoders from float32 to the storage formats used by the inputs.

Written from the format definitions:

* bfloat16 keeps the upper 16 bits of an IEEE-754 binary32; rounding to the kept bits
  is round-to-nearest, ties-to-even.
* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
  when the exponent field is 0, no infinities, and S.1111.111 is the only NaN pattern.
  The largest finite magnitude is 1.75 * 2^8 = 448.  Encoding rounds to nearest-even
  and saturates anything at or beyond 448 to +-448.

* OCP MX FP4 (E2M1 elements with one E8M0 scale per 32 consecutive elements): an
  element is 1 sign bit, 2 exponent bits with bias 1 and 1 mantissa bit, magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6; a scale byte s stands for 2^(s - 127) (255 is NaN).  The
  block's shared exponent is floor(log2(max |x|)) - 2 (2 being the element format's
  largest exponent), elements are x / 2^exponent rounded to nearest-even and saturated
  to +-6, and two elements share a byte, the first in the low nibble.

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


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def f32_to_mxfp4(x):
    """x [..., K] (K % 32 == 0) -> (packed uint8 [..., K/2], scales uint8 [..., K/32])."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value cannot be encoded as MX FP4 input")
    K = x.shape[-1]
    if K % 32:
        raise ValueError("MX FP4 needs a multiple of 32 elements along the last axis")
    blk = x.reshape(x.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, E = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f * 2^E, f in [0.5, 1)
    X = np.where(amax > 0, E - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    scale = (X + 127).astype(np.uint8)
    v = blk / np.exp2(X.astype(np.float64))[..., None]
    a = np.minimum(np.abs(v), 6.0)
    # nearest magnitude, ties to the even code
    d = np.abs(a[..., None] - E2M1_MAGNITUDES) + (np.arange(8) & 1) * 1e-9
    code = np.argmin(d, axis=-1).astype(np.uint8)
    nib = code | (np.signbit(v).astype(np.uint8) << 3)
    nib = nib.reshape(x.shape[:-1] + (K // 2, 2))
    packed = (nib[..., 0] | (nib[..., 1] << 4)).astype(np.uint8)
    return packed, scale
