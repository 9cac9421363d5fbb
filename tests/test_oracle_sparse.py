"""Pins of the sparse-KV oracle (O7): importance scores, index selection and
the gathered draft attention ("The second ledger of speculative decoding",
sections 3.1-3.2)."""
import itertools

import numpy as np
import pytest

from oracle.cycle import draft_tokens, sparse_speculative_cycle
from oracle.model import attend, forward
from oracle.sparse import attention_probs, build_index, index_bounds, select_index
from synth import kv_history, model_weights, token_ids
from synth.configs import LLAMA8B
from tests.helpers import host, oracle_model

TINY = LLAMA8B.with_(n_layers=2, hidden=64, ffn=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                     vocab=97, n_shared=0)


# ------------------------------------------------------------------ probabilities
def test_probabilities_sum_to_one_and_zero_query_is_uniform():
    rng = np.random.default_rng(0)
    K = rng.normal(size=(50, 16))
    p = attention_probs(rng.normal(size=16), K, 37)
    assert p.shape == (37,) and abs(p.sum() - 1.0) < 1e-12 and (p > 0).all()
    np.testing.assert_allclose(attention_probs(np.zeros(16), K, 20), np.full(20, 1 / 20), rtol=1e-14)


def test_one_hot_values_reproduce_the_probabilities():
    # attend() with V = identity returns the probability vector itself: the
    # two independently written softmaxes must agree.
    rng = np.random.default_rng(1)
    K = rng.normal(size=(16, 16)) * 2
    q = rng.normal(size=16)
    for n in (1, 7, 16):
        np.testing.assert_allclose(attend(q, K, np.eye(16), n)[:n], attention_probs(q, K, n), rtol=1e-12)


# ------------------------------------------------------------------ index selection
def _brute_top_k(score, s, r, K):
    """Among all K-subsets of [s, r), the one whose (score desc, pos asc)
    sorted key list is lexicographically smallest."""
    best = None
    for sub in itertools.combinations(range(s, r), K):
        key = sorted((-score[j], j) for j in sub)
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1])


@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(8, 15))
    score = rng.integers(0, 4, size=L).astype(np.float64)  # many exact ties
    n_sink, n_recent = 2, 3
    for permille in (0, 350, 500, 700, 1000):
        idx = select_index(score, L, n_sink, n_recent, permille)
        s, r, K = index_bounds(L, n_sink, n_recent, permille)
        expect = list(range(s)) + _brute_top_k(score, s, r, K) + list(range(r, L))
        assert idx.tolist() == expect


def test_selection_characterisation_large():
    rng = np.random.default_rng(7)
    L = 5000
    score = np.round(rng.exponential(size=L), 2)  # ties at 2 decimals
    idx = select_index(score, L, 4, 64, 100)
    s, r, K = index_bounds(L, 4, 64, 100)
    assert (s, r, K) == (4, L - 64, 500 - 68)
    assert len(idx) == 500 and (np.diff(idx) > 0).all()
    assert idx[:4].tolist() == [0, 1, 2, 3] and idx[-64:].tolist() == list(range(L - 64, L))
    chosen = set(idx[4:-64].tolist())
    rest = [j for j in range(s, r) if j not in chosen]
    worst_chosen = max((-score[j], j) for j in chosen)
    best_rest = min((-score[j], j) for j in rest)
    assert worst_chosen < best_rest


def test_selection_edge_cases():
    score = np.arange(100, dtype=np.float64)
    assert select_index(score, 100, 4, 64, 1000).tolist() == list(range(100))  # full budget
    assert select_index(score, 50, 4, 64, 100).tolist() == list(range(50))     # L < sink + recent
    assert select_index(score, 3, 4, 64, 100).tolist() == [0, 1, 2]
    assert select_index(score, 0, 4, 64, 100).tolist() == []
    # ceil(0.1 * L) exact in integers: 60000 -> 6000, 60001 -> 6001
    assert index_bounds(60000, 4, 64, 100) == (4, 59936, 6000 - 68)
    assert index_bounds(60001, 4, 64, 100)[2] == 6001 - 68
    # budget below sink + recent: no middle positions
    assert select_index(score, 100, 4, 64, 10).tolist() == list(range(4)) + list(range(36, 100))


# ------------------------------------------------------------------ scores and gather
def _tiny_model_and_kv(ctx, seed=3):
    w = model_weights(TINY, seed, "cpu")
    m = oracle_model(TINY, w, substitute_layers=[1])
    cap = ctx + 32
    K, V = kv_history(TINY.n_layers, TINY.n_kv_heads, ctx, TINY.head_dim, cap, seed + 10, "cpu")
    return m, (host(K).astype(np.float64), host(V).astype(np.float64))


def test_window_scores_sum_to_rows_times_group():
    m, kv = _tiny_model_and_kv(40)
    toks = [int(t) for t in token_ids(6, TINY.vocab, 1)]
    G = TINY.n_q_heads // TINY.n_kv_heads
    for window in (16, 4, 1):
        scores = []
        forward(m, (kv[0].copy(), kv[1].copy()), 40, toks, scores=scores, score_window=window)
        assert len(scores) == TINY.n_layers
        for sc in scores:
            assert sc.shape == (TINY.n_kv_heads, 46)
            np.testing.assert_allclose(sc.sum(axis=1), min(window, 6) * G, rtol=1e-12)
            if window == 1:  # only the last row (position 45) contributes, and it sees every key
                assert (sc > 0).all()


def test_full_budget_index_is_the_dense_draft():
    m, kv = _tiny_model_and_kv(60)
    toks = [int(t) for t in token_ids(4, TINY.vocab, 2)]
    full = [[np.arange(60) for _ in range(TINY.n_kv_heads)] for _ in range(TINY.n_layers)]
    kv_a = (kv[0].copy(), kv[1].copy())
    kv_b = (kv[0].copy(), kv[1].copy())
    ta, za = draft_tokens(m, kv_a, 60, toks[0], 4, 0.0, [0] * 4)
    tb, zb = draft_tokens(m, kv_b, 60, toks[0], 4, 0.0, [0] * 4, index=full)
    assert ta == tb
    np.testing.assert_array_equal(za, zb)


def test_excluded_positions_do_not_matter():
    m, kv = _tiny_model_and_kv(60)
    idx = [[np.r_[0:4, 30:40, 50:60] for _ in range(TINY.n_kv_heads)] for _ in range(TINY.n_layers)]
    base = lambda: (kv[0].copy(), kv[1].copy())
    z0 = forward(m, base(), 60, [5], draft=True, sparse=(idx, 60))[0]
    kv1 = base()
    kv1[1][:, :, 10] = 1e3  # position 10 is outside every index
    z1 = forward(m, kv1, 60, [5], draft=True, sparse=(idx, 60))[0]
    np.testing.assert_array_equal(z0, z1)
    kv2 = base()
    kv2[1][:, :, 35] = 1e3  # position 35 is inside
    z2 = forward(m, kv2, 60, [5], draft=True, sparse=(idx, 60))[0]
    assert not np.array_equal(z0, z2)


def test_sparse_cycle_rebuilds_the_index_over_committed_positions():
    m, kv = _tiny_model_and_kv(80)
    gamma = 3
    n, out, status, toks, dl, tl, scores, index = sparse_speculative_cycle(
        m, kv, 80, 7, gamma, 0.0, 0.0, [0] * gamma, [0] * gamma, 0, None, 2, 8, 16, 300)
    L = 80 + n + 1
    assert len(index) == TINY.n_layers and len(index[0]) == TINY.n_kv_heads
    for l, sc in enumerate(scores):
        assert sc.shape == (TINY.n_kv_heads, 80 + gamma + 1)
        for hk in range(TINY.n_kv_heads):
            assert index[l][hk].tolist() == select_index(sc[hk], L, 2, 8, 300).tolist()
            assert len(index[l][hk]) == -(-300 * L // 1000)
    assert build_index(scores, L, 2, 8, 300)[1][0].tolist() == index[1][0].tolist()
