"""bfloat16 storage emulation (round to nearest, ties to even).

The decoder stores activations, KV entries and logits as bfloat16; every such
storage point in the oracle passes through :func:`round_bf16`.
"""
import numpy as np


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits; the result is returned as float64.
    Values past the largest finite bfloat16 become +-inf, NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(x)  # x = m * 2**e with 0.5 <= |m| < 1
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        # below the smallest normal bfloat16 the spacing is fixed at 2**-133
        tiny = np.abs(x) < 2.0 ** -126
        r = np.where(tiny, np.ldexp(np.rint(np.ldexp(x, 133)), -133), r)
        r = np.where(np.isfinite(x) & (np.abs(r) >= 2.0 ** 128), np.copysign(np.inf, x), r)
    return r


def bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bits(x):
    """float64 -> bfloat16 bit patterns (uint16), rounding to nearest even."""
    r = round_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)
