"""O1: 4-bit substitute weights (uniform, asymmetric, group-wise).

Follows [SSN] Method details, "substitute layer generation": a substitute is
the target layer itself with its weights held at low precision, built with a
plain uniform quantiser that needs no calibration data; [SSR] section 2.2 step
four fixes 4 bits.  The pages leave the group axis, group size, zero-point
form and rounding open; the reading used here:

  * groups of 64 consecutive weights along the input (K) axis of each row;
  * lo = min, hi = max of the group (float32 values of the bf16 weights);
  * scale s: the float32 span fl32(hi - lo) over 15, rounded to the nearest
    fp16 value, then raised to the next fp16 value when 15 s falls below the
    span (15 s is exact in float32), so that the 16 levels always reach hi;
    s := 1 when it is 0 (a constant group); it saturates at the fp16
    maximum instead of overflowing;
  * offset m = fp16(lo) (saturating);
  * code q = clamp(rint_even(fl32(fl32(x - m) / s)), 0, 15) with s, m the
    *stored* fp16 values read back as float32 (no fused multiply-add);
  * dequantised weight  w_hat = q * s + m.

Storage: ``codes`` uint8 [N][K/2], byte j = q[2j] | q[2j+1] << 4;
``meta`` float16 [N][K/64][2] = (s, m).

The round-trip bound |x - w_hat| <= s/2 that the substitutes must meet
holds for every group of bf16 values inside the fp16 range: 15 s covers the
span, and fp16(lo) is lo itself (a bf16 value in the fp16 normal range is an
fp16 value) or lies within half of the smallest fp16 step, 2**-25 <= s/2,
below it.  Rounding the scale to nearest alone breaks it when s is an fp16
subnormal (spans below about 1e-3): there 15 s can fall short of the span by
a large fraction of a step, and the top codes clamp.

Pinned by: the hand-built group whose values sit exactly on the 16 levels,
the brute-force nearest level on small inputs, the round-trip bound
|x - w_hat| <= s/2 at every scale (including subnormal scales), the
degenerate constant group and the byte packing.
"""
import numpy as np

GROUP = 64
LEVELS = 15
FP16_MAX = np.float32(65504.0)


def _to_fp16_saturating(v):
    v = np.asarray(v, dtype=np.float32)
    return np.clip(v, -FP16_MAX, FP16_MAX).astype(np.float16)


def quantize(w, group=GROUP):
    """Quantise a [N][K] matrix of bf16 values (given as float32/float64)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    g = w.reshape(n, k // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    span = (hi - lo).astype(np.float32)                       # fl32 subtraction
    s32 = (span / np.float32(LEVELS)).astype(np.float32)       # fl32 division
    s16 = _to_fp16_saturating(s32)
    short = (s16.astype(np.float32) * np.float32(LEVELS)) < span  # exact product
    up = np.nextafter(s16, np.float16(np.inf))
    s16 = np.where(short & np.isfinite(up), up, s16).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    m16 = _to_fp16_saturating(lo)
    s = s16.astype(np.float32)[:, :, None]
    m = m16.astype(np.float32)[:, :, None]
    t = ((g - m).astype(np.float32) / s).astype(np.float32)   # two fl32 ops, no FMA
    q = np.clip(np.rint(t), 0, LEVELS).astype(np.uint8)       # rint rounds half to even
    q = q.reshape(n, k)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    meta = np.stack([s16, m16], axis=2).astype(np.float16)
    return codes, meta


def unpack_codes(codes):
    """uint8 [N][K/2] -> integer codes [N][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, kh = codes.shape
    q = np.empty((n, 2 * kh), dtype=np.uint8)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return q


def dequantize(codes, meta, group=GROUP):
    """w_hat = q * s + m, in float64."""
    q = unpack_codes(codes).astype(np.float64)
    n, k = q.shape
    meta = np.asarray(meta, dtype=np.float16).astype(np.float64)
    s = np.repeat(meta[:, :, 0], group, axis=1)
    m = np.repeat(meta[:, :, 1], group, axis=1)
    return q * s + m
