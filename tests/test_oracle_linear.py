"""Pins of the oracle's matrix-vector products (O2)."""
import numpy as np

from oracle.bf16 import round_bf16, bits_to_f64, f64_to_bits
from oracle.model import linear
from oracle.quant import dequantize
from synth import normal_tensor


def test_round_bf16_known_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert round_bf16(-3.0) == -3.0
    assert np.isinf(round_bf16(3.5e38))
    b = f64_to_bits(np.array([1.0, -2.0, 0.15625]))
    np.testing.assert_array_equal(b, np.array([0x3F80, 0xC000, 0x3E20], dtype=np.uint16))
    np.testing.assert_array_equal(bits_to_f64(b), [1.0, -2.0, 0.15625])


def test_all_equal_codes_closed_form():
    rng = np.random.default_rng(7)
    n, k, c = 6, 256, 9
    codes = np.full((n, k // 2), c | (c << 4), dtype=np.uint8)
    meta = np.stack([rng.uniform(0.001, 0.01, (n, k // 64)),
                     rng.uniform(-0.05, 0.0, (n, k // 64))], axis=2).astype(np.float16)
    x = normal_tensor((k,), 1.0, 3).float().numpy().astype(np.float64)
    y = linear(x[None, :], dequantize(codes, meta))[0]
    xs = x.reshape(k // 64, 64).sum(axis=1)
    m64 = meta.astype(np.float64)
    closed = round_bf16(((c * m64[:, :, 0] + m64[:, :, 1]) * xs[None, :]).sum(axis=1))
    ulp = np.abs(closed) * 2.0 ** -7
    assert (np.abs(y - closed) <= ulp).all()


def test_linear_matches_loop_sum():
    w = normal_tensor((5, 64), 0.02, 1).float().numpy()
    x = normal_tensor((3, 64), 1.0, 2).float().numpy()
    y = linear(x, w)
    for i in range(3):
        for n in range(5):
            acc = 0.0
            for k in range(64):
                acc += float(x[i, k]) * float(w[n, k])
            assert abs(y[i, n] - round_bf16(acc)) <= abs(round_bf16(acc)) * 2.0 ** -7
