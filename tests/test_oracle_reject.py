"""Pins of oracle/reject.py (O5): the rejection round is an exact sampler."""
import numpy as np
from scipy import stats

from oracle.reject import reject
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


def test_zero_residual_falls_back_to_p():
    # p one-hot-like equal to q except on the drafted token -> D may vanish only when p <= q
    z = np.array([0.0, 0.0, 0.0], dtype=np.float32)
    # draft with T_d = 0 puts q = onehot(0); target uniform: residual = p without token 0
    n, out, st = reject(np.stack([z, z]), z[None], [0], [TWO24 - 1], 0, 1.0, 0.0)
    assert n == 0 and out[0] in (1, 2) and st == 0


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
