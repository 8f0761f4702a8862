"""E4M3FN byte decoding and exact BF16 encoding -- oracle (test infrastructure).

The pages store the latent KV pool as ``Float8_e4m3fn`` and cast it to
BFloat16 with ``.to()`` ("The KV Cache Cast Bottleneck", *The Context*;
"When a Faster Kernel Doesn't Speed Up Serving", *Step 3*, CastFromFP8).
They name the format but do not define it.  The definition used here is the
OCP OFP8 E4M3 encoding: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, subnormals when the exponent field is 0, no infinities, and NaN only for
the all-ones exponent-and-mantissa pattern (0x7F / 0xFF).  Largest finite
magnitude 448.

The BF16 side of the cast: every finite E4M3 value has at most 4 significant
bits and an exponent inside BF16's normal range, so its BF16 encoding is exact
(no rounding).  NaN becomes the canonical BF16 quiet NaN 0x7FC0 whatever its
sign; that is what a ``.to(torch.bfloat16)`` produces, and ``.to()`` is the
cast the pages profile.
"""
import math

import numpy as np

BF16_CANONICAL_NAN = 0x7FC0


def e4m3fn_value(code: int) -> float:
    """Real value of one E4M3FN byte, straight from the bit fields."""
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range: %r" % (code,))
    sign = code >> 7
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1-7)  ==  mant * 2^-9
        magnitude = mant * 2.0 ** -9
    else:
        magnitude = (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return -magnitude if sign else magnitude


def decode_table() -> np.ndarray:
    """float64[256]: value of every byte code (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_bits_of(x: float) -> int:
    """BF16 bit pattern of a value that BF16 represents exactly.

    Raises ValueError when ``x`` would need rounding (it never does for an
    E4M3 value) or lies outside BF16's normal range.  Zero keeps its sign.
    """
    if math.isnan(x):
        return BF16_CANONICAL_NAN
    sign = 1 if math.copysign(1.0, x) < 0 else 0
    mag = abs(x)
    if mag == 0.0:
        return sign << 15
    frac, exp = math.frexp(mag)  # mag = frac * 2**exp, frac in [0.5, 1)
    biased = exp - 1 + 127
    if not 1 <= biased <= 254:
        raise ValueError("value outside BF16 normal range: %r" % (x,))
    mant_scaled = (frac * 2.0 - 1.0) * 128.0
    if mant_scaled != math.floor(mant_scaled):
        raise ValueError("value not exactly representable in BF16: %r" % (x,))
    return (sign << 15) | (biased << 7) | int(mant_scaled)


def cast_table_bf16() -> np.ndarray:
    """uint16[256]: BF16 bits of every E4M3FN code (the cast's lookup table)."""
    return np.array([bf16_bits_of(e4m3fn_value(c)) for c in range(256)], dtype=np.uint16)
