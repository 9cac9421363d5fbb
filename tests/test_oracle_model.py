"""Pins of the oracle forward (O3) and the speculative cycle (O6)."""
import numpy as np
from scipy.special import softmax

from oracle.bf16 import round_bf16
from oracle.cycle import autoregressive_generate, speculative_generate, prefill
from oracle.model import attend, forward, new_kv, rmsnorm, rope
from synth import model_weights, uniform_codes, token_ids
from synth.configs import QWEN7B
from tests.helpers import oracle_model

TINY = QWEN7B.with_(n_layers=2, hidden=64, ffn=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                    vocab=97, n_shared=1)


def test_rmsnorm_constant_vector():
    for c in (0.5, -3.0, 1e-3):
        out = rmsnorm(np.full(64, c), np.ones(64), 1e-6)
        np.testing.assert_array_equal(out, round_bf16(np.full(64, c / np.sqrt(c * c + 1e-6))))


def test_rope_hand_computed(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "rope_rmsnorm.json")))
    for case in g["rope"]:
        out = rope(np.array(case["x"], dtype=np.float64), case["pos"], case["theta"])
        np.testing.assert_allclose(out, case["out"], rtol=0, atol=1e-12)


def test_rmsnorm_hand_computed_with_weight(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "rope_rmsnorm.json")))
    for case in g["rmsnorm"]:
        out = rmsnorm(np.array([case["h"]]), np.array(case["g"]), case["eps"])[0]
        np.testing.assert_array_equal(out, case["out"])


def test_rope_properties():
    rng = np.random.default_rng(0)
    q, k = rng.normal(size=128), rng.normal(size=128)
    np.testing.assert_allclose(rope(q, 0, 1e6), q, atol=0)
    for pos in (1, 17, 5000):
        r = rope(q, pos, 1e6)
        pairs = q[:64] ** 2 + q[64:] ** 2
        np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, pairs, rtol=1e-12)
    # relative position: <R_m q, R_n k> depends on m - n only
    a = rope(q, 40, 1e4) @ rope(k, 33, 1e4)
    b = rope(q, 107, 1e4) @ rope(k, 100, 1e4)
    assert abs(a - b) < 1e-9


def test_attention_matches_masked_softmax():
    rng = np.random.default_rng(1)
    K, V = rng.normal(size=(20, 16)), rng.normal(size=(20, 16))
    Q = rng.normal(size=(5, 16))
    scores = Q @ K.T / 4.0
    mask = np.arange(20)[None, :] > (14 + np.arange(5))[:, None]
    scores[mask] = -np.inf
    ref = softmax(scores, axis=1) @ V
    for j in range(5):
        np.testing.assert_allclose(attend(Q[j], K, V, 15 + j), ref[j], rtol=1e-12, atol=1e-12)


def _tiny(seed=0, subs=(1,)):
    w = model_weights(TINY, seed, "cpu")
    return oracle_model(TINY, w, subs)


def test_verify_rows_equal_single_token_decode():
    m = _tiny()
    ctx = token_ids(9, TINY.vocab, 3)
    for draft in (False, True):
        kv1 = new_kv(m, 32)
        kv2 = new_kv(m, 32)
        kl = prefill(m, kv1, list(ctx[:6]))
        prefill(m, kv2, list(ctx[:6]))
        toks = list(ctx[5:9])
        batch = forward(m, kv1, kl, toks, draft=draft)
        for j, t in enumerate(toks):
            one = forward(m, kv2, kl + j, [t], draft=draft)[0]
            diff = np.abs(batch[j] - one)
            assert (diff <= np.abs(one) * 2.0 ** -7 + 1e-30).all()
            assert (diff == 0).mean() > 0.99


def test_shared_layers_and_no_substitutes():
    m = _tiny(subs=())
    kv1, kv2 = new_kv(m, 16), new_kv(m, 16)
    a = forward(m, kv1, 0, [3, 5, 7], draft=True)
    b = forward(m, kv2, 0, [3, 5, 7], draft=False)
    np.testing.assert_array_equal(a, b)
    m2 = _tiny(subs=(1,))
    kv3 = new_kv(m2, 16)
    c = forward(m2, kv3, 0, [3, 5, 7], draft=True)
    assert np.abs(c - b).max() > 0  # the substitute changes the draft


def test_greedy_speculative_equals_greedy_autoregressive():
    m = _tiny(seed=2)
    prompt = list(token_ids(5, TINY.vocab, 7))
    G, gamma = 14, 4
    cycles = G
    U = (np.zeros((cycles, gamma), np.int64), np.zeros((cycles, gamma), np.int64), np.zeros(cycles, np.int64))
    sd, ns = speculative_generate(m, prompt, G, gamma, 0.0, 0.0, U, 64)
    ar = autoregressive_generate(m, prompt, G, 0.0, np.zeros(G, np.int64), 64)
    assert sd == ar
    assert all(0 <= n <= gamma for n in ns)


def test_self_draft_accepts_everything():
    # draft == target (no substitutes) and T = T_d: p = q, so every draft is kept
    m = _tiny(seed=4, subs=())
    prompt = list(token_ids(4, TINY.vocab, 9))
    gamma, cycles = 3, 3
    Ud, _ = uniform_codes(cycles * gamma, 1)
    R, _ = uniform_codes(cycles * gamma, 2)
    Uf, _ = uniform_codes(cycles, 3)
    U = (Ud.reshape(cycles, gamma), R.reshape(cycles, gamma), Uf)
    out, ns = speculative_generate(m, prompt, (gamma + 1) * cycles, gamma, 0.7, 0.7, U, 64)
    assert ns == [gamma] * cycles


def test_float32_sums_agree_over_one_layer():
    # the definition fixes the bf16 storage points, not the precision of the
    # sums: float32 sums of one layer stay well inside the logits tolerance
    from synth import model_weights, kv_history, token_ids
    from synth.configs import QWEN7B
    from tests.helpers import host, oracle_model
    shape = QWEN7B.with_(n_layers=1, hidden=512, ffn=1024, n_q_heads=4, n_kv_heads=2, vocab=500,
                         n_shared=0)
    w = model_weights(shape, 3, "cpu")
    om = oracle_model(shape, w, [0])
    K, V = kv_history(1, 2, 20, 128, 24, 4, "cpu")
    kv = lambda: (host(K).astype(np.float64), host(V).astype(np.float64))
    toks = [int(t) for t in token_ids(3, 500, 5)]
    for draft in (False, True):
        a = forward(om, kv(), 20, toks, draft=draft)
        b = forward(om, kv(), 20, toks, draft=draft, acc=np.float32)
        rel = np.abs(a - b).max() / np.abs(a).max()
        assert 0 < rel < 1e-2
