"""Pins of oracle/adaptive.py (the entropy-adaptive draft length of "The
second ledger of speculative decoding", section 3.3)."""
import math

import numpy as np
import pytest

from oracle.adaptive import BETA, Controller, entropy


def test_entropy_closed_forms():
    for V in (1, 2, 7, 1000):
        assert abs(entropy(np.zeros(V)) - math.log(V)) < 1e-12
    assert entropy(np.array([0.0, -np.inf, -np.inf])) == 0.0
    assert entropy(np.array([5.0, -1e4, -1e4])) < 1e-12
    for a, b in ((0.0, 1.0), (2.5, -0.5), (3.0, 3.0)):
        p = 1.0 / (1.0 + math.exp(b - a))
        h = -p * math.log(p) - (1 - p) * math.log(1 - p)
        assert abs(entropy(np.array([a, b])) - h) < 1e-12
    # non-finite logits carry no probability
    assert abs(entropy(np.array([1.0, np.nan, 1.0, np.inf])) - math.log(2)) < 1e-12
    # shifting every logit changes nothing; sharper rows have less entropy
    z = np.random.default_rng(0).normal(0, 2, 50)
    assert abs(entropy(z + 7.0) - entropy(z)) < 1e-12
    assert entropy(3 * z) < entropy(z)


def _ctl_with_centres(acc, rej, gamma_max=16, c=0.3):
    ctl = Controller(gamma_max, c)
    ctl.h_acc, ctl.h_rej, ctl.seen_acc, ctl.seen_rej = acc, rej, True, True
    return ctl


def test_soft_class():
    ctl = _ctl_with_centres(1.0, 3.0)
    assert ctl.p_of(1.0) == 1.0 and ctl.p_of(3.0) == 0.0 and ctl.p_of(2.0) == 0.5
    assert ctl.p_of(1.5) == 0.75 and ctl.p_of(0.0) == 0.75  # d_rej / (d_acc + d_rej)
    assert _ctl_with_centres(2.0, 2.0).p_of(2.0) == 0.5
    assert Controller(8, 0.3).p_of(5.0) == 1.0  # centres not seen yet


def _brute_best(p, c, gmax):
    E = [(1 + sum(p ** m for m in range(1, k + 1))) / (k * c + 1) for k in range(1, gmax + 1)]
    return 1 + int(np.argmax(E))  # lowest k on ties


@pytest.mark.parametrize("c", [0.05, 0.2, 0.5, 0.9])
@pytest.mark.parametrize("p", [0.3, 0.6, 0.8, 0.95, 0.99])
def test_stop_rule_matches_brute_force_at_constant_p(p, c):
    # centres 0 and 1, every token at entropy 1 - p: p_i = p for all i; the
    # efficiency is then unimodal in k and the online rule stops at its argmax
    gmax = 48
    ctl = _ctl_with_centres(0.0, 1.0, gmax, c)
    assert abs(ctl.p_of(1.0 - p) - p) < 1e-12
    i = 0
    while ctl.after_token(1.0 - p):
        i += 1
    assert ctl.gamma_eff == _brute_best(ctl.p_of(1.0 - p), c, gmax)


def test_sure_draft_drafts_to_the_end_iff_cheaper_than_verify():
    # p = 1: E(k) = (k + 1)/(k c + 1), whose slope has the sign of 1 - c
    # (S(k) = (alpha k + 1)/(k c + 1) of the blog's section 1 with alpha = 1)
    for c, want in ((0.25, 16), (0.99, 16), (1.5, 1), (3.0, 1)):
        ctl = Controller(16, c)  # centres unseen: p = 1
        while ctl.after_token(0.7):
            pass
        assert ctl.gamma_eff == want


def test_spike_stops_the_draft_at_once():
    ctl = _ctl_with_centres(0.5, 4.0, 32, 0.2)
    for _ in range(5):
        assert ctl.after_token(0.5)  # confident tokens: go on
    assert not ctl.after_token(4.0)  # p = 0: nothing more can be gained
    assert ctl.gamma_eff == 6


def test_ema_updates_and_closed_form():
    ctl = Controller(8, 0.3)
    for h in (1.0, 2.0, 0.5):
        ctl.after_token(h)
    ctl.gamma_eff = 3
    ctl.after_round(1)  # token 1 accepted, token 2 rejected, token 3 unjudged
    assert ctl.h_acc == 1.0 and ctl.h_rej == 2.0 and ctl.seen_acc and ctl.seen_rej
    hs = [0.2, 0.4, 0.9, 0.1]
    for h in hs:
        ctl.after_token(h)
    ctl.gamma_eff = 4
    ctl.after_round(4)  # all accepted: no rejected token
    want = 1.0
    for h in hs:
        want = want + BETA * (h - want)
    assert abs(ctl.h_acc - want) < 1e-15 and ctl.h_rej == 2.0
    # closed form of the EMA: (1-b)^4 h0 + sum_j b (1-b)^(3-j) h_j
    cf = (1 - BETA) ** 4 * 1.0 + sum(BETA * (1 - BETA) ** (3 - j) * hs[j] for j in range(4))
    assert abs(ctl.h_acc - cf) < 1e-12
    assert ctl.gamma_eff == 8 and ctl.H == []  # the next round starts fresh


def test_greedy_adaptive_decoding_is_lossless():
    from oracle.cycle import adaptive_generate, autoregressive_generate
    from synth import model_weights, token_ids
    from synth.configs import QWEN7B
    from tests.helpers import oracle_model
    shape = QWEN7B.with_(n_layers=2, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, vocab=300, n_shared=1)
    w = model_weights(shape, 4, "cpu")
    om = oracle_model(shape, w, [1])
    prompt = [int(t) for t in token_ids(6, shape.vocab, 5)]
    G, gmax = 30, 6
    z = np.zeros((64, gmax), np.int64)
    out, ns, gs = adaptive_generate(om, prompt, G, gmax, 0.3, 0.0, 0.0, (z, z, np.zeros(64, np.int64)), 128)
    ref = autoregressive_generate(om, prompt, G, 0.0, np.zeros(G, np.int64), 128)
    assert out == ref
    assert all(1 <= g <= gmax for g in gs) and all(0 <= n <= g for n, g in zip(ns, gs))
    assert len(set(gs)) > 1  # the length adapts
