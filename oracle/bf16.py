"""Exact bfloat16 <-> float64 conversion.

bfloat16 is the top half of an IEEE-754 binary32: sign, 8 exponent bits, 7
stored mantissa bits.  Widening is exact.  Narrowing rounds to nearest, ties to
even, directly from float64 (no intermediate float32, which could round twice).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
import numpy as np

BF16_MAX = float.fromhex("0x1.fe00000000000p+127")


def bf16_bits_to_f64(bits):
    """uint16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> uint16 bfloat16 bit patterns, round to nearest even.

    The spacing of bfloat16 values around |x| = m * 2**e (0.5 <= m < 1) is
    2**(e - 8) in the normal range and 2**-133 for subnormals (e < -125).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    spacing = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(xf / spacing) * spacing          # np.rint rounds half to even
    # values at or beyond BF16_MAX + half a spacing overflow to infinity
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, xf), r)
    out[...] = np.where(finite, r, x)
    f32 = out.astype(np.float32)                  # exact: r has <= 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    return bits


def round_to_bf16(x):
    """float64 -> nearest bfloat16 value, returned as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))
