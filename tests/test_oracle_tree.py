"""Pins of oracle/tree.py (O9): the static tree of k chains of depth D."""
import itertools

import numpy as np

from oracle.cycle import prefill, speculative_cycle, autoregressive_generate
from oracle.model import forward, new_kv
from oracle.reject import STATUS_Q_ZERO, STATUS_ZERO_RESIDUAL
from oracle.sampling import sample, softmax_f64, argmax_lowest
from oracle.tree import (node, depth, chain_of, n_nodes, visible_slots, tree_forward, draft_tree, tree_reject,
                         tree_commit, tree_cycle, tree_generate, top_k_lowest)
from synth import model_weights, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.helpers import oracle_model

TWO24 = 1 << 24
TINY = QWEN7B.with_(n_layers=2, hidden=64, ffn=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                    vocab=97, n_shared=1)


def _tiny(seed=0, subs=(1,)):
    return oracle_model(TINY, model_weights(TINY, seed, "cpu"), subs)


def _uniforms(k, D, seed):
    Ud, _ = uniform_codes(k * D, seed)
    R, _ = uniform_codes(k + D - 1, seed + 1)
    U, _ = uniform_codes(1, seed + 2)
    return [int(u) for u in Ud], [int(r) for r in R], int(U[0])


def test_numbering_and_visibility():
    k, D, kv_len = 3, 4, 10
    seen = set()
    for c in range(k):
        for d in range(1, D + 1):
            t = node(c, d, D)
            assert depth(t, D) == d and chain_of(t, D) == c
            seen.add(t)
            vis = visible_slots(t, kv_len, D)
            # the prefix and the root, then this chain's depth-1..d slots
            assert vis == list(range(kv_len + 1)) + [kv_len + node(c, e, D) for e in range(1, d + 1)]
    assert seen == set(range(1, n_nodes(k, D)))
    assert depth(0, D) == 0 and visible_slots(0, kv_len, D) == list(range(kv_len + 1))


def test_top_k_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(200):
        V = int(rng.integers(1, 9))
        z = rng.integers(-3, 3, V).astype(np.float32)
        if trial % 3 == 0:
            z[rng.integers(0, V)] = np.nan
        if trial % 5 == 0:
            z[rng.integers(0, V)] = np.inf
        k = int(rng.integers(1, 6))
        # brute force: repeated lowest-index argmax over what is left
        left = z.astype(np.float64).copy()
        ref = []
        for _ in range(k):
            if not np.isfinite(left).any():
                ref.append(0)
                continue
            j = argmax_lowest(left)
            ref.append(j)
            left[j] = np.nan
        assert top_k_lowest(z, k) == ref


def _same_start(m, prompt, cap):
    kv = new_kv(m, cap)
    kl = prefill(m, kv, prompt)
    return kv, kl


def test_one_chain_is_the_plain_cycle():
    # k = 1: the tree is the chain of the plain cycle with gamma = D, with the
    # same uniforms in the same places
    m = _tiny(seed=3)
    prompt = [int(t) for t in token_ids(6, TINY.vocab, 11)]
    D = 4
    for i, (T, Td) in enumerate([(0.0, 0.0), (0.0, 1.0), (1.0, 1.0), (0.7, 0.0), (0.8, 0.5)]):
        Ud, R, U = _uniforms(1, D, 40 + 3 * i)
        kv1, kl = _same_start(m, prompt, 32)
        kv2, _ = _same_start(m, prompt, 32)
        n1, out1, st1, toks1, dl1, tl1 = speculative_cycle(m, kv1, kl, prompt[-1], D, T, Td, Ud, R, U)
        n2, out2, st2, c2, toks2, dl2, tl2, new_len = tree_cycle(m, kv2, kl, prompt[-1], 1, D, T, Td, Ud, R, U)
        assert (n1, out1, st1) == (n2, out2, st2)
        assert c2 == (0 if n1 > 0 else -1)
        assert list(toks1) == [int(t) for t in toks2]
        np.testing.assert_array_equal(dl1, dl2)
        np.testing.assert_array_equal(tl1, tl2)
        assert new_len == kl + n1 + 1
        for a, b in zip(kv1, kv2):
            np.testing.assert_array_equal(a[:, :, :new_len], b[:, :, :new_len])


def test_node_logits_equal_a_plain_forward_of_the_path():
    m = _tiny(seed=5)
    prompt = [int(t) for t in token_ids(5, TINY.vocab, 2)]
    k, D = 3, 3
    kv, kl = _same_start(m, prompt, 40)
    Ud, _, _ = _uniforms(k, D, 9)
    toks, dl = draft_tree(m, kv, kl, prompt[-1], k, D, 1.0, Ud)
    tl = tree_forward(m, kv, kl, list(range(n_nodes(k, D))), list(toks), D)
    for c in range(k):
        path = [0] + [node(c, d, D) for d in range(1, D + 1)]
        for draft in (False, True):
            kv2, _ = _same_start(m, prompt, 40)
            ref = forward(m, kv2, kl, [int(toks[t]) for t in path], draft=draft)
            if draft:  # draft rows: the root and depths 1..D-1
                got = np.stack([dl[0]] + [dl[1 + c * (D - 1) + d - 1] for d in range(1, D)])
                np.testing.assert_allclose(got, ref[:D], rtol=1e-9, atol=1e-12)
            else:
                np.testing.assert_allclose(tl[path], ref, rtol=1e-9, atol=1e-12)
    # sampled children come from the root's draft distribution, chains from their own
    assert all(0 <= int(t) < TINY.vocab for t in toks)


def test_greedy_tree_equals_greedy_autoregressive():
    m = _tiny(seed=2)
    prompt = [int(t) for t in token_ids(5, TINY.vocab, 7)]
    G = 16
    ar = autoregressive_generate(m, prompt, G, 0.0, np.zeros(G, np.int64), 96)
    for k, D, Td in [(3, 4, 0.0), (2, 1, 0.0), (4, 2, 1.0), (1, 5, 0.0)]:
        cycles = G
        Ud, _ = uniform_codes(cycles * k * D, 3)
        U = (Ud.reshape(cycles, k * D), np.zeros((cycles, k + D - 1), np.int64), np.zeros(cycles, np.int64))
        out, ns = tree_generate(m, prompt, G, k, D, 0.0, Td, U, 96)
        assert out == ar, (k, D, Td)
        assert all(0 <= n <= D for n in ns)


def _first_true(pred):
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


def _root_case(V, k, seed):
    rng = np.random.default_rng(seed)
    zt = (np.round(rng.normal(0, 1.5, (1 + k, V)) * 8) / 8).astype(np.float32)
    zd = (zt[:1] + np.round(rng.normal(0, 0.9, (1, V)) * 8) / 8).astype(np.float32)
    return zt, zd


def _first_token_law(zt, zd, k, T, Td):
    """Exact law of the first emitted token over the children, the accept
    uniforms and the final draw - the oracle treated as a black box."""
    V = zt.shape[1]
    if Td == 0:
        tuples = [(tuple(top_k_lowest(zd[0], k)), 1.0)]
    else:
        q = _token_measure(lambda U: sample(zd[0], Td, U), V)
        tuples = [(xs, float(np.prod([q[x] for x in xs]))) for xs in itertools.product(range(V), repeat=k)]
    law = np.zeros(V)
    for xs, w in tuples:
        if w == 0:
            continue
        toks = np.zeros(1 + k, np.int64)
        toks[1:] = xs
        reach = 1.0  # probability that children 0..c-1 were all rejected
        for c in range(k):
            R = [TWO24 - 1] * (k + 0)

            def first(Rc, U=0):
                R[c] = Rc
                return tree_reject(zt, zd, toks, k, 1, R, U, T, Td)[3]
            a = _first_true(lambda Rc: first(Rc) != c) / TWO24
            R[c] = TWO24 - 1
            law[xs[c]] += w * reach * a
            reach *= 1.0 - a
            if reach == 0.0:
                break
        if reach > 0.0:
            R = [TWO24 - 1] * k
            law += w * reach * _token_measure(lambda U: tree_reject(zt, zd, toks, k, 1, R, U, T, Td)[1][0], V)
    return law


def test_first_token_is_distributed_as_p():
    for seed, (V, k, T, Td) in enumerate([(4, 2, 1.0, 1.0), (3, 3, 1.0, 0.7), (4, 2, 0.6, 0.6),
                                          (5, 3, 1.0, 0.0), (4, 4, 0.8, 0.0)]):
        zt, zd = _root_case(V, k, seed)
        law = _first_token_law(zt, zd, k, T, Td)
        np.testing.assert_allclose(law, softmax_f64(zt[0], T), atol=4e-6 * k)


def test_more_children_accept_more_often():
    # P(some child accepted) rises with k (same q, same p): the point of width
    V = 5
    zt, zd = _root_case(V, 3, 17)
    q = _token_measure(lambda U: sample(zd[0], 1.0, U), V)
    prev = 0.0
    for k in (1, 2, 3):
        acc = 0.0
        for xs in itertools.product(range(V), repeat=k):
            w = float(np.prod([q[x] for x in xs]))
            toks = np.zeros(1 + k, np.int64)
            toks[1:] = xs
            reach = 1.0
            for c in range(k):
                R = [TWO24 - 1] * k

                def first(Rc):
                    R[c] = Rc
                    return tree_reject(zt[:1 + k], zd, toks, k, 1, R, 0, 1.0, 1.0)[3]
                a = _first_true(lambda Rc: first(Rc) != c) / TWO24
                acc += w * reach * a
                reach *= 1.0 - a
        assert acc > prev
        prev = acc
    p, qf = softmax_f64(zt[0], 1.0), softmax_f64(zd[0], 1.0)
    assert abs(_one_child(p, qf) - np.minimum(p, qf).sum()) < 1e-12


def _one_child(p, q):
    return float(np.minimum(p, q).sum())


def test_greedy_root_takes_the_first_matching_child():
    zt, zd = _root_case(6, 4, 3)
    y = argmax_lowest(zt[0])
    others = [x for x in range(6) if x != y]
    for pos in range(4):
        xs = others[:4]
        xs[pos] = y
        toks = np.array([0] + xs)
        n, out, st, c = tree_reject(zt, zd, toks, 4, 1, [0] * 4, 0, 0.0, 0.0)
        assert c == pos and n == 1 and out[0] == y and st == 0
        assert out[1] == argmax_lowest(zt[1 + pos])  # the bonus from the chain's own row
    toks = np.array([0] + others[:4])
    n, out, st, c = tree_reject(zt, zd, toks, 4, 1, [0] * 4, 0, 0.0, 0.0)
    assert (n, out, c) == (0, [y], -1)


def test_zero_residual_and_skipped_children():
    # p = q and child 0 has weight 0 on both sides: rejected (q(x) = 0), the
    # residual max(0, p - q) has no mass and is replaced by p, after which
    # child 1 (q = p) is accepted for sure
    z = np.array([1.0, 0.5, -0.25, 2.0, 0.0, 2.0 - 40.0], dtype=np.float32)
    zt = np.stack([z, z, z])
    zd = z[None].copy()
    toks = np.array([0, 5, 3])
    n, out, st, c = tree_reject(zt, zd, toks, 2, 1, [0, TWO24 - 1], 0, 1.0, 1.0)
    assert c == 1 and out[0] == 3
    assert st == STATUS_Q_ZERO | STATUS_ZERO_RESIDUAL
    # a child outside the vocabulary is skipped, the next one judged
    y = argmax_lowest(z)
    n, out, st, c = tree_reject(zt, zd, np.array([0, -1, y]), 2, 1, [0, 0], 0, 0.0, 0.0)
    assert c == 1 and out[0] == y and st == STATUS_Q_ZERO
    n, out, st, c = tree_reject(zt, zd, np.array([0, -1, 6]), 2, 1, [0, 0], 77, 1.0, 1.0)
    assert c == -1 and n == 0 and st == STATUS_Q_ZERO
    assert out == [sample(z, 1.0, 77)]  # nothing tested: the draw is from p


def test_commit_moves_the_accepted_chain():
    k, D, kl = 3, 4, 5
    L, H, cap, d = 2, 2, kl + 1 + k * D + 3, 4
    K = np.arange(L * H * cap * d, dtype=np.float64).reshape(L, H, cap, d)
    V = -K
    for c in range(k):
        for n in range(0, D + 1):
            K2, V2 = K.copy(), V.copy()
            new = tree_commit((K2, V2), kl, n, c, D)
            assert new == kl + n + 1
            np.testing.assert_array_equal(K2[:, :, :kl + 1], K[:, :, :kl + 1])
            for i in range(1, n + 1):
                np.testing.assert_array_equal(K2[:, :, kl + i], K[:, :, kl + node(c, i, D)])
                np.testing.assert_array_equal(V2[:, :, kl + i], V[:, :, kl + node(c, i, D)])


def test_committed_kv_equals_autoregressive_kv():
    m = _tiny(seed=6)
    prompt = [int(t) for t in token_ids(4, TINY.vocab, 5)]
    k, D = 3, 3
    kv, kl = _same_start(m, prompt, 80)
    committed = list(prompt)
    for cyc in range(4):
        Ud, R, U = _uniforms(k, D, 100 + cyc)
        n, out, st, c, *_rest, kl = tree_cycle(m, kv, kl, committed[-1], k, D, 0.0, 0.0, Ud, R, U)
        committed += out
    ref = new_kv(m, 80)
    prefill(m, ref, committed)
    assert kl == len(committed) - 1
    for a, b in zip(kv, ref):
        a, b = a[:, :, :kl], b[:, :, :kl]
        np.testing.assert_allclose(a, b, rtol=2.0 ** -7, atol=1e-30)
        assert (a == b).mean() > 0.99


def test_self_draft_tree_accepts_every_chain_token():
    # draft == target (no substitutes) and T = T_d: p = q at every node, so the
    # first child in range is accepted and so is every token of its chain
    m = _tiny(seed=4, subs=())
    prompt = [int(t) for t in token_ids(4, TINY.vocab, 9)]
    k, D = 3, 3
    for skip in range(k):
        kv, kl = _same_start(m, prompt, 64)
        Ud, R, U = _uniforms(k, D, 60 + skip)
        toks, dl = draft_tree(m, kv, kl, prompt[-1], k, D, 0.7, Ud)
        tl = tree_forward(m, kv, kl, list(range(n_nodes(k, D))), list(toks), D)
        for c in range(skip):  # children before `skip` are not vocabulary ids: skipped
            toks[node(c, 1, D)] = -1
        n, out, st, c = tree_reject(tl, dl, toks, k, D, R, U, 0.7, 0.7)
        assert c == skip and n == D
        assert out[:D] == [int(toks[node(skip, d, D)]) for d in range(1, D + 1)]
        assert st == (STATUS_Q_ZERO if skip else 0)


def test_accepted_chain_is_judged_like_its_path():
    # children before c are skipped and R[c] = 0 accepts child c; the rest of
    # the round must be the plain rejection round over chain c's path, with
    # the path's rows taken from plain forwards of the path
    from oracle.reject import reject
    m = _tiny(seed=8)
    prompt = [int(t) for t in token_ids(5, TINY.vocab, 4)]
    k, D = 3, 4
    for i, (T, Td) in enumerate([(1.0, 1.0), (0.5, 0.5), (0.8, 0.0), (0.0, 1.0)]):
        kv, kl = _same_start(m, prompt, 64)
        Ud, R, U = _uniforms(k, D, 80 + i)
        toks, dl = draft_tree(m, kv, kl, prompt[-1], k, D, Td, Ud)
        tl = tree_forward(m, kv, kl, list(range(n_nodes(k, D))), list(toks), D)
        for c in range(k):
            tk = toks.copy()
            for c2 in range(c):
                tk[node(c2, 1, D)] = -1
            Rc = list(R)
            Rc[c] = 0
            tlc = tl
            if T == 0:  # greedy root: make child c the target's argmax (and verify again)
                tk[node(c, 1, D)] = argmax_lowest(tl[0].astype(np.float32))
                kv_v, _ = _same_start(m, prompt, 64)
                tlc = tree_forward(m, kv_v, kl, list(range(n_nodes(k, D))), list(tk), D)
            n, out, st, cc = tree_reject(tlc, dl, tk, k, D, Rc, U, T, Td)
            assert cc == c
            path = [int(tk[0])] + [int(tk[node(c, d, D)]) for d in range(1, D + 1)]
            kv_t, _ = _same_start(m, prompt, 64)
            kv_d, _ = _same_start(m, prompt, 64)
            zt = forward(m, kv_t, kl, path, draft=False)
            zd = np.stack([forward(m, kv_d, kl + d, [path[d]], draft=True)[0] for d in range(D)])
            n2, out2, st2 = reject(zt[1:], zd[1:], path[2:], Rc[k:], U, T, Td)
            assert (n, out) == (1 + n2, [path[1]] + out2), (T, Td, c)
            assert st == st2 | (STATUS_Q_ZERO if c else 0)


def test_residual_weights_stay_below_2_41():
    # children rejected one after another on a flat row: every residual's
    # weights stay below 2^41 (their sums below 2^59), and the law stays p
    from oracle.tree import _residual
    from oracle.sampling import fixed_weights
    rng = np.random.default_rng(1)
    V = 64
    for trial in range(20):
        zt = (rng.normal(0, 0.3, V)).astype(np.float32)
        zd = (zt + rng.normal(0, 0.3, V)).astype(np.float32)
        W, S = fixed_weights(zt, 1.0)
        Wp = W
        Wd, Sd = fixed_weights(zd, 0.5 + trial % 3)
        for c in range(8):
            W = _residual(W, S, Wd, Sd, W is Wp)
            S = int(W.sum())
            assert W.max() < 1 << 41 and S < 1 << 59
            if S == 0:
                break
