"""Pins of oracle/sampling.py (O4)."""
import numpy as np
from scipy import stats

from oracle.sampling import (argmax_lowest, fixed_weights, inverse_cdf, sample,
                             softmax_f64, tempered_weights_f32)
from synth import uniform_codes

TWO24 = 1 << 24


def _interval_lengths(fn, V):
    """Measure of U in [0, 2^24) mapped to each token by a nondecreasing fn(U)."""
    starts = []
    for j in range(V):
        lo, hi = 0, TWO24           # first U with fn(U) >= j
        while lo < hi:
            mid = (lo + hi) // 2
            if fn(mid) >= j:
                hi = mid
            else:
                lo = mid + 1
        starts.append(lo)
    starts.append(TWO24)
    return np.diff(np.array(starts, dtype=np.int64))


def test_argmax_lowest_index_on_ties():
    assert argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert argmax_lowest(np.array([5.0])) == 0
    assert argmax_lowest(np.array([-1.0, -1.0])) == 0


def test_inverse_cdf_interval_lengths_are_weights():
    W = np.array([1, 2, 3, 4, 0, 6], dtype=np.int64) << 30
    lens = _interval_lengths(lambda U: inverse_cdf(W, U), len(W))
    np.testing.assert_allclose(lens / TWO24, W / W.sum(), atol=2.0 / TWO24)
    assert lens[4] == 0


def test_sample_probabilities_match_softmax():
    z = np.array([0.5, -1.25, 2.0, 0.0, 1.0], dtype=np.float32)
    for T in (1.0, 0.6, 0.2):
        lens = _interval_lengths(lambda U: sample(z, T, U), len(z))
        np.testing.assert_allclose(lens / TWO24, softmax_f64(z, T), atol=1e-6)


def test_greedy_is_argmax():
    z = np.array([0.1, 0.7, 0.7, -3.0], dtype=np.float32)
    for U in (0, 12345, TWO24 - 1):
        assert sample(z, 0.0, U) == 1


def test_tempered_weights_max_is_one_and_float32():
    z = np.array([3.0, 1.0, -2.0], dtype=np.float32)
    w = tempered_weights_f32(z, 0.2)
    assert w.dtype == np.float32 and w[0] == 1.0
    W, S = fixed_weights(z, 0.2)
    assert W[0] == 1 << 40 and S == int(W.sum())


def test_chi_square_sampling():
    V = 8
    z = np.linspace(-1.0, 1.5, V).astype(np.float32)
    p = softmax_f64(z, 1.0)
    U, _ = uniform_codes(40000, 123)
    counts = np.bincount([sample(z, 1.0, int(u)) for u in U], minlength=V)
    chi2, pval = stats.chisquare(counts, p * len(U))
    assert pval > 1e-3


def test_non_finite_logits_carry_no_probability():
    # a row with NaN / +-Inf entries draws exactly like the row without them
    rng = np.random.default_rng(8)
    V = 11
    bad = {0: np.nan, 3: np.inf, 7: -np.inf, 10: np.nan}
    keep = [j for j in range(V) if j not in bad]
    U, _ = uniform_codes(300, 9)
    for trial in range(30):
        z = np.round(rng.normal(0, 2.0, V) * 8).astype(np.float32) / 8
        zf = z[keep].copy()
        for j, v in bad.items():
            z[j] = v
        for T in (0.0, 0.3, 1.0):
            for u in U[10 * trial:10 * trial + 10]:
                assert sample(z, T, u) == keep[sample(zf, T, u)]
            p = softmax_f64(z, T)
            np.testing.assert_array_equal(p[list(bad)], 0.0)
            np.testing.assert_allclose(p[keep], softmax_f64(zf, T), rtol=1e-15, atol=0)


def test_row_without_finite_logit_gives_token_zero():
    for z in (np.full(6, np.nan, np.float32), np.array([np.inf, -np.inf, np.nan], np.float32)):
        assert argmax_lowest(z) == 0
        for T in (0.0, 0.5, 1.0):
            for u in (0, 12345, TWO24 - 1):
                assert sample(z, T, u) == 0
        W, S = fixed_weights(z, 1.0)
        assert S == 0 and (W == 0).all()
