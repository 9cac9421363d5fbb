"""O1: low-bit substitute weights (uniform, asymmetric, group-wise).

Follows [SSN] Method details, "substitute layer generation": a substitute is
the target layer itself with its weights held at low precision, built with a
plain uniform quantiser that needs no calibration data, at 2 or 3 bits;
[SSR] section 2.2 step four uses 4 bits.  The pages leave the group axis,
group size, zero-point form and rounding open; the reading used here, for
b in {2, 3, 4} bits and L = 2**b - 1 levels above the lowest:

  * groups of 64 consecutive weights along the input (K) axis of each row;
  * lo = min, hi = max of the group (float32 values of the bf16 weights);
  * scale s: the float32 span fl32(hi - lo) over L, rounded to the nearest
    fp16 value, then raised to the next fp16 value when L s falls below the
    span (L s is exact in float32), so that the 2**b levels always reach hi;
    s := 1 when it is 0 (a constant group); it saturates at the fp16
    maximum instead of overflowing;
  * offset m = fp16(lo) (saturating);
  * code q = clamp(rint_even(fl32(fl32(x - m) / s)), 0, L) with s, m the
    *stored* fp16 values read back as float32 (no fused multiply-add);
  * dequantised weight  w_hat = q * s + m.

Storage (``codes`` uint8, one row of bytes per output row; ``meta`` float16
[N][K/64][2] = (s, m) for every width):
  * 4 bits: [N][K/2], byte j = q[2j] | q[2j+1] << 4;
  * 2 bits: [N][K/4], byte j = q[4j] | q[4j+1] << 2 | q[4j+2] << 4 | q[4j+3] << 6;
  * 3 bits: [N][3K/8], two planes per row: the low two bits of every code in
    the 2-bit layout (K/4 bytes), then the third bit of every code (K/8
    bytes) in 4-byte words of 32 weights whose bytes hold weights 0-7, 16-23,
    8-15 and 24-31 of the word (bit t of a byte: its t-th weight).  With that
    byte order, bits e and e + 16 of a word belong to the same pair of
    weights as the 2-bit fields e and e + 8 of a 16-weight word, so a decoder
    pairs both planes with the same activations.

The round-trip bound |x - w_hat| <= s/2 that the substitutes must meet
holds for every group of bf16 values inside the fp16 range: L s covers the
span, and fp16(lo) is lo itself (a bf16 value in the fp16 normal range is an
fp16 value) or lies within half of the smallest fp16 step, 2**-25 <= s/2,
below it.  Rounding the scale to nearest alone breaks it when s is an fp16
subnormal (spans below about 1e-3 at 4 bits): there L s can fall short of the
span by a large fraction of a step, and the top codes clamp.

Pinned by: the hand-built groups whose values sit exactly on the levels (at
each width, with their byte layouts), the brute-force nearest level on small
inputs, the round-trip bound |x - w_hat| <= s/2 at every scale (including
subnormal scales), the scale as the smallest fp16 value covering the span
(brute force over all fp16 values), the degenerate constant group.
"""
import numpy as np

GROUP = 64
FP16_MAX = np.float32(65504.0)
BITS = (2, 3, 4)
HI_BYTE_BLOCK = (0, 16, 8, 24)  # 3-bit third-bit plane: first weight of each byte of a 32-weight word


def _to_fp16_saturating(v):
    v = np.asarray(v, dtype=np.float32)
    return np.clip(v, -FP16_MAX, FP16_MAX).astype(np.float16)


def levels(bits):
    return (1 << bits) - 1


def row_bytes(k, bits):
    """Bytes of one row of codes."""
    return {4: k // 2, 2: k // 4, 3: 3 * k // 8}[bits]


def quantize(w, group=GROUP, bits=4):
    """Quantise a [N][K] matrix of bf16 values (given as float32/float64)."""
    if bits not in BITS:
        raise ValueError("bits must be 2, 3 or 4")
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    L = levels(bits)
    g = w.reshape(n, k // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    span = (hi - lo).astype(np.float32)                       # fl32 subtraction
    s32 = (span / np.float32(L)).astype(np.float32)            # fl32 division
    s16 = _to_fp16_saturating(s32)
    short = (s16.astype(np.float32) * np.float32(L)) < span    # exact product
    up = np.nextafter(s16, np.float16(np.inf))
    s16 = np.where(short & np.isfinite(up), up, s16).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    m16 = _to_fp16_saturating(lo)
    s = s16.astype(np.float32)[:, :, None]
    m = m16.astype(np.float32)[:, :, None]
    t = ((g - m).astype(np.float32) / s).astype(np.float32)   # two fl32 ops, no FMA
    q = np.clip(np.rint(t), 0, L).astype(np.uint8)            # rint rounds half to even
    q = q.reshape(n, k)
    meta = np.stack([s16, m16], axis=2).astype(np.float16)
    return pack_codes(q, bits), meta


def _pack2(q):
    return (q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6)).astype(np.uint8)


def pack_codes(q, bits):
    """Integer codes [N][K] (each < 2**bits) -> the byte layout of ``bits``."""
    q = np.asarray(q, dtype=np.uint8)
    if bits == 4:
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    if bits == 2:
        return _pack2(q)
    lo2 = _pack2(q & 3)
    b = (q >> 2) & 1
    hi = np.zeros((q.shape[0], q.shape[1] // 8), dtype=np.uint8)
    for j in range(q.shape[1] // 8):
        w, byte = divmod(j, 4)
        first = 32 * w + HI_BYTE_BLOCK[byte]
        for t in range(8):
            hi[:, j] |= (b[:, first + t] << t).astype(np.uint8)
    return np.concatenate([lo2, hi], axis=1)


def unpack_codes(codes, bits=4, k=None):
    """Byte layout of ``bits`` -> integer codes [N][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, nb = codes.shape
    if bits == 4:
        q = np.empty((n, 2 * nb), dtype=np.uint8)
        q[:, 0::2] = codes & 0x0F
        q[:, 1::2] = codes >> 4
        return q
    if k is None:
        k = 4 * nb if bits == 2 else 8 * nb // 3
    q = np.empty((n, k), dtype=np.uint8)
    lo2 = codes[:, :k // 4]
    for t in range(4):
        q[:, t::4] = (lo2 >> (2 * t)) & 3
    if bits == 3:
        hi = codes[:, k // 4:k // 4 + k // 8]
        for j in range(k // 8):
            w, byte = divmod(j, 4)
            first = 32 * w + HI_BYTE_BLOCK[byte]
            for t in range(8):
                q[:, first + t] |= ((hi[:, j] >> t) & 1) << 2
    return q


def dequantize(codes, meta, group=GROUP, bits=4):
    """w_hat = q * s + m, in float64."""
    meta = np.asarray(meta, dtype=np.float16).astype(np.float64)
    k = meta.shape[1] * group
    q = unpack_codes(codes, bits, k).astype(np.float64)
    s = np.repeat(meta[:, :, 0], group, axis=1)
    m = np.repeat(meta[:, :, 1], group, axis=1)
    return q * s + m
