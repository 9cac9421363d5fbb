"""Pins of oracle/reject.py (O5): the rejection round is an exact sampler."""
import numpy as np
from scipy import stats

from oracle.reject import reject, STATUS_NONFINITE, STATUS_Q_ZERO, STATUS_ZERO_RESIDUAL
from oracle.sampling import sample, softmax_f64
from synth import uniform_codes, logits_pair

TWO24 = 1 << 24


def _first_true(pred):
    """Smallest integer t in [0, 2^24] with pred(t) true (pred monotone)."""
    lo, hi = 0, TWO24
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _token_measure(fn, V):
    starts = [_first_true(lambda U: fn(U) >= j) for j in range(V)] + [TWO24]
    return np.diff(np.array(starts, dtype=np.int64)) / TWO24


def _case(V, seed, T, Td):
    rng = np.random.default_rng(seed)
    zt = np.round(rng.normal(0, 1.5, (2, V)) * 8) / 8
    zd = zt[:1] + np.round(rng.normal(0, 0.8, (1, V)) * 8) / 8
    return zt.astype(np.float32), zd.astype(np.float32)


def _first_token_distribution(zt, zd, T, Td):
    """Exact law of the first emitted token, the oracle treated as a black box."""
    V = zt.shape[1]
    q = _token_measure(lambda U: sample(zd[0], Td, U), V)
    out = np.zeros(V)
    p_accept = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        # acceptance is r < threshold: find the measure of accepting r
        acc = _first_true(lambda R: reject(zt, zd, [x], [R], 0, T, Td)[0] == 0) / TWO24
        p_accept[x] = acc
        out[x] += q[x] * acc
        if acc < 1.0:
            rej = _token_measure(lambda U: reject(zt, zd, [x], [TWO24 - 1], U, T, Td)[1][0], V)
            out += q[x] * (1 - acc) * rej
    return out, q, p_accept


def test_first_token_is_distributed_as_p():
    for seed, (T, Td) in enumerate([(1.0, 1.0), (1.0, 0.5), (0.6, 0.6), (1.0, 0.0)]):
        zt, zd = _case(4, seed, T, Td)
        law, q, pacc = _first_token_distribution(zt, zd, T, Td)
        p = softmax_f64(zt[0], T)
        np.testing.assert_allclose(law, p, atol=2e-6)
        # alpha = P(accept) = sum_x min(p, q)
        alpha = float((q * pacc).sum())
        assert abs(alpha - np.minimum(p, softmax_f64(zd[0], Td)).sum()) < 2e-6


def test_acceptance_probability_product_and_tau():
    # identical, independent positions: P(n >= m) = alpha^m, E[n+1] = (1-a^(g+1))/(1-a)
    from oracle.speedup import tau_iid
    zt1, zd1 = _case(3, 5, 1.0, 1.0)
    V = 3
    p = softmax_f64(zt1[0], 1.0)
    q = softmax_f64(zd1[0], 1.0)
    alpha = np.minimum(p, q).sum()
    gamma = 2
    zt = np.stack([zt1[0]] * (gamma + 1))
    zd = np.stack([zd1[0]] * gamma)
    qm = _token_measure(lambda U: sample(zd[0], 1.0, U), V)
    pacc = [_first_true(lambda R: reject(zt[:2], zd[:1], [x], [R], 0, 1.0, 1.0)[0] == 0) / TWO24
            for x in range(V)]
    a1 = float(np.dot(qm, pacc))
    assert abs(a1 - alpha) < 2e-6
    # P(n >= 2): position 2 only seen when position 1 accepted
    p2 = 0.0
    for x1 in range(V):
        for x2 in range(V):
            acc2 = _first_true(lambda R: reject(zt, zd, [x1, x2], [0, R], 0, 1.0, 1.0)[0] < 2) / TWO24
            p2 += qm[x1] * pacc[x1] * qm[x2] * acc2
    assert abs(p2 - alpha ** 2) < 4e-6
    tau = 1 + a1 + p2
    assert abs(tau - tau_iid(alpha, gamma)) < 1e-5


def test_q_equals_p_accepts_everything():
    zt, _ = logits_pair(6, 300, 9)
    zt = zt.float().numpy()
    R, _ = uniform_codes(6, 1)
    for T in (1.0, 0.6):
        toks = [sample(zt[i], T, 1000 * i + 7) for i in range(6)]
        n, out, st = reject(zt, zt[:6], toks, R, 99, T, T)
        assert n == 6 and out[:6] == toks and len(out) == 7 and st == 0


def test_greedy_is_longest_argmax_prefix():
    zt, zd = logits_pair(8, 500, 4)
    zt = zt.float().numpy()
    am = [int(np.argmax(zt[i])) for i in range(9)]
    for cut in range(9):
        toks = am[:8].copy()
        if cut < 8:
            toks[cut] = (toks[cut] + 1) % 500
        n, out, _ = reject(zt, zd.float().numpy(), toks, [0] * 8, 0, 0.0, 0.0)
        assert n == cut
        assert out == toks[:cut] + [am[cut]]


def test_at_least_one_token_and_ranges():
    zt, zd = logits_pair(4, 1000, 2)
    zt, zd = zt.float().numpy(), zd.float().numpy()
    R, _ = uniform_codes(400, 3)
    Uf, _ = uniform_codes(100, 4)
    Ud, _ = uniform_codes(400, 5)
    for c in range(100):
        toks = [sample(zd[i], 1.0, Ud[4 * c + i]) for i in range(4)]
        n, out, st = reject(zt, zd, toks, R[4 * c:4 * c + 4], Uf[c], 1.0, 1.0)
        assert 0 <= n <= 4 and len(out) == n + 1
        assert all(0 <= t < 1000 for t in out) and st == 0


def test_gamma_zero_is_plain_sampling():
    zt, _ = logits_pair(0, 50, 8)
    zt = zt.float().numpy()
    n, out, _ = reject(zt, np.zeros((0, 50), np.float32), [], [], 777, 1.0, 1.0)
    assert n == 0 and out == [sample(zt[0], 1.0, 777)]


def test_rejection_of_greedy_draft_draws_from_p_without_drafted_token():
    # q = onehot(0) (T_d = 0) against a uniform p: the residual max(0, p - q)
    # is p restricted to tokens 1 and 2, each with half of the mass
    z = np.array([0.0, 0.0, 0.0], dtype=np.float32)
    n, out, st = reject(np.stack([z, z]), z[None], [0], [TWO24 - 1], 0, 1.0, 0.0)
    assert n == 0 and out[0] == 1 and st == 0
    lengths = _token_measure(lambda U: reject(np.stack([z, z]), z[None], [0], [TWO24 - 1], U, 1.0, 0.0)[1][0], 3)
    np.testing.assert_allclose(lengths, [0.0, 0.5, 0.5], atol=1e-7)


def _zero_residual_case(V=6, T=1.0):
    # target = draft, so p = q and max(0, p - q) has no mass; the drafted
    # token sits 40/T below the maximum, so exp(-40) * 2^40 < 1 gives it
    # weight 0 on both sides: q(x) = p(x) = 0, it is rejected, and the
    # residual draw has nothing to draw from
    z = np.array([1.0, 0.5, -0.25, 2.0, 0.0, 2.0 - 40.0 * T][:V], dtype=np.float32)
    return np.stack([z, z]), z[None].copy(), [V - 1]


def test_zero_residual_falls_back_to_p():
    zt, zd, toks = _zero_residual_case()
    for U in (0, 1 << 20, 1 << 23, TWO24 - 1):
        n, out, st = reject(zt, zd, toks, [0], U, 1.0, 1.0)
        assert n == 0
        assert st == STATUS_ZERO_RESIDUAL | STATUS_Q_ZERO
        # the fallback draw is the plain draw from p = softmax(z_t) with the same u
        assert out == [sample(zt[0], 1.0, U)]
    law = _token_measure(lambda U: reject(zt, zd, toks, [0], U, 1.0, 1.0)[1][0], 6)
    np.testing.assert_allclose(law, softmax_f64(zt[0], 1.0), atol=2e-6)


def test_out_of_vocabulary_draft_token_is_rejected():
    # the device marks a skipped draft step with token -1: q(x) = p(x) = 0
    zt, zd = logits_pair(3, 40, 12)
    zt, zd = zt.float().numpy(), zd.float().numpy()
    am = [int(np.argmax(zt[i])) for i in range(4)]
    for T, Td in [(0.0, 0.0), (0.0, 1.0), (1.0, 1.0), (1.0, 0.0)]:
        toks = [am[0], -1, am[2]] if T == 0 else [sample(zd[0], Td, 5), -1, 3]
        n, out, st = reject(zt, zd, toks, [0, 0, 0], 1234, T, Td)
        assert n == 1 and out[0] == toks[0] and st & STATUS_Q_ZERO
        if T == 0:
            assert out[1] == am[1]
        assert 0 <= out[1] < 40
    n, out, st = reject(zt, zd, [40, 0, 0], [0, 0, 0], 99, 0.0, 0.0)
    assert n == 0 and out == [am[0]] and st == STATUS_Q_ZERO


def test_non_finite_logits_reduce_to_the_finite_row():
    # a NaN or +-Inf logit carries no probability: the round decides exactly
    # as on the rows with those entries removed, and flags status bit 1.
    # Rows left finite hold -1e4 there (weight 0 at these temperatures, never
    # the argmax), so removing those columns changes nothing for them either.
    rng = np.random.default_rng(3)
    V, gamma = 9, 2
    bad = {1: np.nan, 4: np.inf, 6: -np.inf}
    keep = [j for j in range(V) if j not in bad]
    for trial in range(40):
        zt = np.round(rng.normal(0, 1.0, (gamma + 1, V)) * 8).astype(np.float32) / 8
        zd = (zt[:gamma] + np.round(rng.normal(0, 0.5, (gamma, V)) * 8) / 8).astype(np.float32)
        zt[:, list(bad)] = -1e4
        zd[:, list(bad)] = -1e4
        T, Td = [(1.0, 1.0), (0.7, 0.0), (0.0, 0.0), (1.0, 0.5)][trial % 4]
        zt_f, zd_f = zt[:, keep].copy(), zd[:, keep].copy()
        rows = [(zt, r) for r in range(gamma + 1)] + [(zd, r) for r in range(gamma)]
        for arr, r in rows:
            if (trial + r) % 2 == 0:
                for j, v in bad.items():
                    arr[r, j] = v
        Ud, _ = uniform_codes(gamma, 100 + trial)
        toks_f = [sample(zd_f[i], Td, Ud[i]) for i in range(gamma)]
        toks = [keep[t] for t in toks_f]
        R, _ = uniform_codes(gamma, 200 + trial)
        Uf = int(uniform_codes(1, 300 + trial)[0][0])
        n_f, out_f, st_f = reject(zt_f, zd_f, toks_f, R, Uf, T, Td)
        n, out, st = reject(zt, zd, toks, R, Uf, T, Td)
        assert n == n_f and out == [keep[t] for t in out_f]
        read_rows = [zt[r] for r in range(n + 1)] + [zd[r] for r in range(min(n + 1, gamma))]
        expect_bad = any(not np.isfinite(z).all() for z in read_rows)
        assert (st & STATUS_NONFINITE) == (STATUS_NONFINITE if expect_bad else 0)
        assert (st & ~STATUS_NONFINITE) == st_f


def test_target_row_without_finite_logit():
    # no mass anywhere in p: nothing is accepted, and every draw gives token 0
    V = 5
    zt = np.full((2, V), np.nan, dtype=np.float32)
    zd = np.array([[0.0, 1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    for T, Td in [(1.0, 1.0), (0.0, 0.0), (1.0, 0.0)]:
        n, out, st = reject(zt, zd, [4], [0], 77, T, Td)
        assert n == 0 and out == [0] and st & STATUS_NONFINITE


def test_chi_square_emitted_tokens():
    V, gamma = 8, 4
    zt, zd = logits_pair(gamma, V, 21, target_std=1.0, draft_noise=0.7)
    zt, zd = zt.float().numpy(), zd.float().numpy()
    p1 = softmax_f64(zt[0], 1.0)
    cycles = 30000
    R, _ = uniform_codes(cycles * gamma, 31)
    Uf, _ = uniform_codes(cycles, 32)
    Ud, _ = uniform_codes(cycles * gamma, 33)
    first = np.zeros(V)
    for c in range(cycles):
        toks = [sample(zd[i], 1.0, Ud[gamma * c + i]) for i in range(gamma)]
        n, out, _ = reject(zt, zd, toks, R[gamma * c:gamma * (c + 1)], Uf[c], 1.0, 1.0)
        first[out[0]] += 1
    _, pval = stats.chisquare(first, p1 * cycles)
    assert pval > 1e-3
