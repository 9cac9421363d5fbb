"""Pins of oracle/multilevel.py (O10): a 2-bit draft for the 4-bit draft."""
import numpy as np
from scipy import stats

from oracle.cycle import autoregressive_generate, prefill, speculative_cycle
from oracle.model import OracleModel, forward, new_kv
from oracle.multilevel import middle_tokens, multilevel_cycle, multilevel_generate
from oracle.sampling import softmax_f64
from synth import model_weights, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.helpers import oracle_model

TINY = QWEN7B.with_(n_layers=2, hidden=64, ffn=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                    vocab=97, n_shared=1)


def _models(seed, shape=TINY, bits2=2):
    w = model_weights(shape, seed, "cpu")
    om4 = oracle_model(shape, w, [1])
    om2 = oracle_model(shape, w, [])
    om2.make_substitutes([1], bits=bits2)
    return w, om4, om2


def _uniforms(cycles, gamma, gamma2, seed):
    U2, _ = uniform_codes(cycles * gamma * gamma2, seed)
    R2, _ = uniform_codes(cycles * gamma * gamma2, seed + 1)
    F2, _ = uniform_codes(cycles * gamma, seed + 2)
    R, _ = uniform_codes(cycles * gamma, seed + 3)
    U, _ = uniform_codes(cycles, seed + 4)
    return (U2.reshape(cycles, gamma, gamma2), R2.reshape(cycles, gamma, gamma2), F2.reshape(cycles, gamma),
            R.reshape(cycles, gamma), U)


def test_greedy_multilevel_equals_greedy_autoregressive():
    _, om4, om2 = _models(2)
    prompt = [int(t) for t in token_ids(5, TINY.vocab, 7)]
    G = 16
    ar = autoregressive_generate(om4, prompt, G, 0.0, np.zeros(G, np.int64), 96)
    for gamma, gamma2 in [(4, 2), (3, 5), (6, 1)]:
        out, ns = multilevel_generate(om4, om2, prompt, G, gamma, gamma2, 0.0, 0.0, 0.0,
                                      _uniforms(G, gamma, gamma2, 3), 96)
        assert out == ar, (gamma, gamma2)
        assert all(0 <= n <= gamma for n in ns)


def test_equal_inner_models_accept_every_inner_draft():
    # the "2-bit" model equal to the 4-bit one and T2 = T_mid: p = q in every
    # inner round, so every inner draft is kept
    _, om4, _ = _models(4)
    prompt = [int(t) for t in token_ids(4, TINY.vocab, 9)]
    kv = new_kv(om4, 64)
    kl = prefill(om4, kv, prompt)
    U2, R2, F2, R, U = _uniforms(1, 6, 3, 11)
    toks, mlog, rounds = middle_tokens(om4, om4, kv, kl, prompt[-1], 6, 3, 0.7, 0.7, U2[0], R2[0], F2[0])
    assert all(n == g for g, n, st in rounds)
    assert len(toks) == 7 and mlog.shape == (6, TINY.vocab)


def _mid_model(om4, om2):
    """A model whose target is the 4-bit model and whose draft is the 2-bit
    model: the plain cycle on it is one inner round."""
    layers = []
    for l in range(om4.n_layers):
        lw = dict(om4.layers[l])
        for name in ("qkv", "o", "gate_up", "down"):
            lw[name] = om4.weight(l, name, True)
        layers.append(lw)
    m = OracleModel(om4.n_layers, om4.hidden, om4.ffn, om4.n_q_heads, om4.n_kv_heads, om4.head_dim, om4.vocab,
                    om4.rope_theta, om4.rms_eps, om4.embed, om4.final_norm, om4.lm_head, layers)
    m.substitute = om2.substitute
    return m


def test_middle_tokens_are_plain_rounds_of_the_4bit_model():
    _, om4, om2 = _models(6)
    mid = _mid_model(om4, om2)
    prompt = [int(t) for t in token_ids(6, TINY.vocab, 2)]
    for i, (T_mid, T2, gamma, gamma2) in enumerate([(1.0, 1.0, 7, 3), (0.6, 0.0, 5, 2), (0.0, 0.8, 6, 4)]):
        U2, R2, F2, _, _ = _uniforms(1, gamma, gamma2, 20 + i)
        kv1, kv2 = new_kv(om4, 64), new_kv(om4, 64)
        kl = prefill(om4, kv1, prompt)
        prefill(om4, kv2, prompt)
        toks, mlog, rounds = middle_tokens(om4, om2, kv1, kl, prompt[-1], gamma, gamma2, T_mid, T2,
                                           U2[0], R2[0], F2[0])
        # the same rounds as plain cycles of the mid model, one after another
        ref = [prompt[-1]]
        ref_log = []
        for r, (g, n_r, st_r) in enumerate(rounds):
            base = len(ref) - 1
            n, out, st, _, _, tl = speculative_cycle(mid, kv2, kl + base, ref[-1], g, T_mid, T2,
                                                     list(U2[0][r]), list(R2[0][r]), F2[0][r])
            assert (n, st) == (n_r, st_r)
            take = min(n + 1, gamma - base)
            ref += out[:take]
            ref_log += [tl[j] for j in range(take)]
        assert toks == ref
        np.testing.assert_array_equal(mlog, np.array(ref_log))


def _peaky(seed):
    """A 1-layer model with 6 tokens and a larger lm_head (distributions far
    from uniform), and as the 2-bit level a different random model."""
    shape = QWEN7B.with_(n_layers=1, hidden=64, ffn=128, n_q_heads=4, n_kv_heads=2, head_dim=16, vocab=6,
                         n_shared=0)
    w = model_weights(shape, seed, "cpu")
    w["lm_head"] = w["lm_head"] * 6
    om4 = oracle_model(shape, w, [0])
    w2 = model_weights(shape, seed + 100, "cpu")
    w2["lm_head"] = w["lm_head"]
    w2["embed"] = w["embed"]
    om2 = oracle_model(shape, w2, [])
    om2.make_substitutes([0], bits=2)
    return shape, om4, om2


def test_first_emitted_token_is_distributed_as_the_target():
    shape, om4, om2 = _peaky(31)
    prompt = [1, 4, 2]
    gamma, gamma2, T, T_mid, T2 = 2, 2, 1.0, 0.7, 1.3
    kv0 = new_kv(om4, 16)
    kl = prefill(om4, kv0, prompt)
    p = softmax_f64(forward(om4, (kv0[0].copy(), kv0[1].copy()), kl, [prompt[-1]])[0], T)
    N = 2000
    counts = np.zeros(shape.vocab)
    U2, R2, F2, R, U = _uniforms(N, gamma, gamma2, 500)
    for s in range(N):
        kv = (kv0[0].copy(), kv0[1].copy())
        n, out, *_ = multilevel_cycle(om4, om2, kv, kl, prompt[-1], gamma, gamma2, T, T_mid, T2,
                                      U2[s], R2[s], F2[s], R[s], U[s])
        counts[out[0]] += 1
    keep = p * N >= 5
    assert keep.sum() >= 4
    chi = stats.chisquare(counts[keep], p[keep] / p[keep].sum() * counts[keep].sum())
    assert chi.pvalue > 1e-3, (counts, p * N)
