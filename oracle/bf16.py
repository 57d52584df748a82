"""bf16 helpers, written from the IEEE-754 binary32 definition (oracle).

bfloat16 is the upper half of an IEEE binary32 word: 1 sign bit, 8 exponent
bits, 7 fraction bits.  All data on the paged path is bf16 (the Pico-vLLM
write-up runs Qwen2.5-1.5B in bfloat16, "project background" section); the
pages do not say how results are rounded to bf16, and this oracle rounds to
nearest, ties to even, everywhere.

bf16 values are carried as numpy ``uint16`` arrays holding the bit patterns.
"""

import numpy as np

_QNAN_BF16 = np.uint16(0x7FC0)


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exactly (bits shifted left 16)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exactly."""
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns stay NaN
        return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16_rne(x):
    """float32 -> bf16 bits, round to nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit word and dropping the
    low 16 bits rounds the magnitude to the nearest bf16 and breaks ties toward
    an even last fraction bit; carries propagate into the exponent, so values
    that round past the largest finite bf16 become infinity.  Any NaN maps to
    the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), _QNAN_BF16, r).astype(np.uint16)


def bf16_ulp(x):
    """Spacing of bf16 numbers at the magnitude of x (float64 in, float64 out).

    bf16 keeps 8 significant bits, so for |x| in [2^(e-1), 2^e) the spacing is
    2^(e-8); below the smallest normal (2^-126) the spacing is fixed at 2^-133.
    """
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)  # x = m * 2^e with m in [0.5, 1)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - 8)


def f64_to_bf16_rne(x):
    """float64 -> bf16 bits with a single rounding (no detour through fp32).

    x / ulp is an exact power-of-two scaling, np.rint rounds half to even, and
    the rounded value is exactly representable in fp32, so the final cast to
    fp32 and the truncation to the high 16 bits are exact.
    """
    x = np.asarray(x, dtype=np.float64)
    q = bf16_ulp(x)
    y = np.rint(x / q) * q
    big = np.abs(y) > 3.3895313892515355e38  # largest finite bf16 (0x7F7F)
    y = np.where(big, np.copysign(np.inf, x), y)
    with np.errstate(invalid="ignore", over="ignore"):
        bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), _QNAN_BF16, bits).astype(np.uint16)
