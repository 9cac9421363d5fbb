"""Sparse-KV drafting on the GPU ("The second ledger of speculative
decoding", sections 3.1-3.2) against the oracle (oracle/sparse.py):
importance scores written by verify, the index rebuild, the gathered draft
attention, whole sparse cycles, and the long-context shape's properties."""
import numpy as np
import pytest
import torch

from oracle.model import forward
from oracle.sparse import index_bounds, select_index
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import CONFIGS, kv_history, model_weights, token_ids
from synth.configs import LLAMA8B
from tests.gpu_util import log, rel_err
from tests.helpers import host, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2

TINY = LLAMA8B.with_(n_layers=2, hidden=256, ffn=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                     vocab=1000, n_shared=0)
SP = dict(n_sink=4, n_recent=16, window=16, budget_permille=100)


def _setup(shape, seed, cap, gamma, ctx, sparse, device="cuda"):
    w = model_weights(shape, seed, device)
    dm = DeviceModel(shape, w)
    dec = SpecDecoder(dm, cap, gamma, 0.0, 0.0, sparse=sparse)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, ctx, shape.head_dim, cap, seed + 7, device)
    dec.load_kv(K, V, ctx, 0)
    om = oracle_model(shape, w, dm.substitute_layers)
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    return dm, dec, om, kv


def _gpu_index(dec):
    n = int(dec.kv_index_len.item())
    return host(dec.kv_index[:, :, :n]).astype(np.int64)


def test_scores_select_and_gathered_draft_match_oracle(cuda):
    ctx, cap, gamma = 700, 800, 4
    log("sparse tiny: scores, select, gathered draft")
    dm, dec, om, kv = _setup(TINY, 5, cap, gamma, ctx, SP)
    G = TINY.n_q_heads // TINY.n_kv_heads
    toks = [int(t) for t in token_ids(gamma + 1, TINY.vocab, 6)]
    dec.tokens.copy_(torch.tensor(toks, dtype=torch.int32))
    dec.verify()
    torch.cuda.synchronize()
    # importance scores of the verify pass vs the oracle's (float64)
    scores = []
    kv2 = (kv[0].copy(), kv[1].copy())
    forward(om, kv2, ctx, toks, scores=scores, score_window=SP["window"])
    got = host(dec.kv_score[:, :, :ctx + gamma + 1]).astype(np.float64)
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(got[l].sum(axis=1), (gamma + 1) * G, rtol=1e-4)
        assert np.abs(got[l] - scores[l]).max() <= TOL * scores[l].max(), l
    # index rebuild after a rollback of n = 2: L = ctx + 3
    L = ctx + 3
    dec.kv_len.fill_(L)
    _lib.kv_select(dm.c, dec.c)
    torch.cuda.synchronize()
    idx = _gpu_index(dec)
    assert idx.shape[2] == _lib.index_count(L, SP["n_sink"], SP["n_recent"], SP["budget_permille"])
    s, r, K = index_bounds(L, SP["n_sink"], SP["n_recent"], SP["budget_permille"])
    assert K > 0 and r - s > K  # the radix-select path runs
    for l in range(TINY.n_layers):
        for hk in range(TINY.n_kv_heads):
            # bit-exact: the oracle's rule applied to the GPU's float32 scores
            ref = select_index(got[l, hk], L, SP["n_sink"], SP["n_recent"], SP["budget_permille"])
            np.testing.assert_array_equal(idx[l, hk], ref)
            # against the oracle's own scores: differences only at near-ties
            ref_o = select_index(scores[l][hk], L, SP["n_sink"], SP["n_recent"], SP["budget_permille"])
            diff = set(ref.tolist()) ^ set(ref_o.tolist())
            kth = np.sort(scores[l][hk][s:r])[::-1][K - 1]
            for j in diff:
                assert abs(scores[l][hk][j] - kth) <= TOL * kth, (l, hk, j)
    # gathered draft, teacher-forced on the GPU's tokens and index
    dec.tokens[0] = toks[1]
    dec.c.use_index = 1
    dec.draft()
    torch.cuda.synchronize()
    gtoks = [toks[1]] + host(dec.tokens[1:]).astype(np.int64).tolist()
    index = [[idx[l, hk] for hk in range(TINY.n_kv_heads)] for l in range(TINY.n_layers)]
    for i in range(gamma):
        ref_z = forward(om, kv2, L + i, [gtoks[i]], draft=True, sparse=(index, L))[0]
        assert rel_err(host(dec.draft_logits[i]), ref_z) < TOL, i


def test_full_budget_draft_is_the_dense_draft(cuda):
    ctx, cap, gamma = 650, 700, 3
    log("sparse tiny: full budget == dense")
    sp = dict(SP, budget_permille=1000)
    dm, dec, om, kv = _setup(TINY, 8, cap, gamma, ctx, sp)
    toks = [int(t) for t in token_ids(gamma + 1, TINY.vocab, 9)]
    dec.tokens.copy_(torch.tensor(toks, dtype=torch.int32))
    dec.verify()
    _lib.kv_select(dm.c, dec.c)
    torch.cuda.synchronize()
    assert int(dec.kv_index_len.item()) == ctx
    np.testing.assert_array_equal(_gpu_index(dec)[1, 0], np.arange(ctx))
    dec.c.use_index = 0
    dec.draft()
    dense = dec.draft_logits.clone()
    dense_t = dec.tokens.clone()
    dec.c.use_index = 1
    dec.draft()
    torch.cuda.synchronize()
    assert torch.equal(dense, dec.draft_logits) and torch.equal(dense_t, dec.tokens)


def _teacher_forced_cycles(dec, dm, om, kv_o, sp, gamma, cycles, T=0.0, Td=0.0, uni=None):
    """Run GPU cycles and, for each, the oracle teacher-forced on the GPU's own
    draft tokens and sparse index: draft logits (gathered when the cycle drafts
    over the index) and verify logits within TOL, importance scores within TOL,
    the rejection round recomputed by the oracle from the GPU's own logits
    bit-exact (n, tokens, status), and the rebuilt index bit-exact to the
    oracle's rule on the GPU's scores.  Returns the number of cycles that
    drafted over the index."""
    from oracle.reject import reject as oreject
    from oracle.sampling import sample as osample
    L_layers, Hkv = om.n_layers, om.n_kv_heads
    G = om.n_q_heads // Hkv
    sparse_cycles = 0
    for c in range(cycles):
        used_index = int(dec.c.use_index)
        index = None
        if used_index:
            gi = _gpu_index(dec)
            index = [[gi[l, hk] for hk in range(Hkv)] for l in range(L_layers)]
        kv_len = int(dec.kv_len.item())
        last = int(dec.tokens[0].item())
        if uni is not None:
            ud, rr, uf = uni[0][c], uni[1][c], uni[2][c:c + 1]
            dec.cycle(ud, rr, uf)
        else:
            dec.cycle()
        torch.cuda.synchronize()
        toks = [last] + host(dec.tokens[1:gamma + 1]).astype(np.int64).tolist()
        dz = host(dec.draft_logits[:gamma]).astype(np.float32)
        tz = host(dec.target_logits[:gamma + 1]).astype(np.float32)
        sparse = None if index is None else (index, kv_len)
        for i in range(gamma):
            ref = forward(om, kv_o, kv_len + i, [toks[i]], draft=True, sparse=sparse)[0]
            assert rel_err(dz[i], ref) < TOL, (c, i)
            u = 0 if uni is None else int(host(uni[0][c])[i])
            assert osample(dz[i], Td, u) == toks[i + 1], (c, i)  # the GPU drew from its own logits
        scores = []
        ref_t = forward(om, kv_o, kv_len, toks, scores=scores, score_window=sp["window"])
        for j in range(gamma + 1):
            assert rel_err(tz[j], ref_t[j]) < TOL, (c, j)
        got_sc = host(dec.kv_score[:, :, :kv_len + gamma + 1]).astype(np.float64)
        for l in range(L_layers):
            assert np.abs(got_sc[l] - scores[l]).max() <= TOL * scores[l].max(), (c, l)
            np.testing.assert_allclose(got_sc[l].sum(axis=1), min(sp["window"], gamma + 1) * G, rtol=1e-4)
        n = int(dec.n_accepted.item())
        out = host(dec.out_tokens[:n + 1]).astype(np.int64).tolist()
        R = [0] * gamma if uni is None else host(uni[1][c]).astype(np.int64).tolist()
        U = 0 if uni is None else int(host(uni[2][c]))
        assert (n, out, int(dec.status.item())) == oreject(tz, dz, toks[1:], R, U, T, Td), c
        L = kv_len + n + 1
        assert int(dec.kv_len.item()) == L
        gi = _gpu_index(dec)
        for l in range(L_layers):
            for hk in range(Hkv):
                ref = select_index(got_sc[l, hk], L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
                np.testing.assert_array_equal(gi[l, hk], ref)
        sparse_cycles += used_index
    return sparse_cycles


def test_sparse_greedy_cycles_match_oracle(cuda):
    ctx, cap, gamma, cycles = 600, 700, 4, 5
    log("sparse tiny: greedy cycles, teacher-forced")
    sp = dict(n_sink=4, n_recent=16, window=16, budget_permille=150)
    dm, dec, om, kv = _setup(TINY, 11, cap, gamma, ctx, sp)
    dec.reset(ctx, int(token_ids(1, TINY.vocab, 12)[0]))
    n_sparse = _teacher_forced_cycles(dec, dm, om, (kv[0].copy(), kv[1].copy()), sp, gamma, cycles)
    assert n_sparse == cycles - 1  # the first cycle drafts densely, every later one over the index


def test_sparse_stochastic_cycles_match_oracle(cuda):
    ctx, cap, gamma, cycles = 520, 640, 4, 4
    log("sparse tiny: stochastic cycles, teacher-forced")
    sp = dict(n_sink=4, n_recent=16, window=16, budget_permille=200)
    w = model_weights(TINY, 14, cuda)
    dm = DeviceModel(TINY, w)
    dec = SpecDecoder(dm, cap, gamma, 1.0, 0.6, sparse=sp)
    K, V = kv_history(TINY.n_layers, TINY.n_kv_heads, ctx, TINY.head_dim, cap, 21, cuda)
    dec.load_kv(K, V, ctx, int(token_ids(1, TINY.vocab, 15)[0]))
    om = oracle_model(TINY, w, dm.substitute_layers)
    from synth import uniform_codes
    from tests.gpu_util import codes_i32
    Ud, _ = uniform_codes(cycles * gamma, 31)
    R, _ = uniform_codes(cycles * gamma, 32)
    Uf, _ = uniform_codes(cycles, 33)
    uni = (codes_i32(Ud.reshape(cycles, gamma), cuda), codes_i32(R.reshape(cycles, gamma), cuda),
           codes_i32(Uf, cuda))
    kv_o = (host(K).astype(np.float64), host(V).astype(np.float64))
    n_sparse = _teacher_forced_cycles(dec, dm, om, kv_o, sp, gamma, cycles, 1.0, 0.6, uni)
    assert n_sparse == cycles - 1


def test_long_context_layer_matches_oracle(cuda):
    """One Llama-3.1-8B-shaped layer over 60,000 positions of synthetic KV,
    gamma 11, budget 10 %: the verify pass (logits and importance scores, the
    multi-tile verify attention), the index rebuild, and draft steps over the
    ~6000-entry index, which run the gathered per-head draft attention with 8
    key splits and 3 chunks in flight per wave (the long-context workload's
    own launch configuration), all against the oracle."""
    wl = CONFIGS["longctx8b"]
    shape = wl.shape.with_(n_layers=1)
    gamma, ctx = wl.gamma, wl.prompt
    cap = ctx + 64
    sp = dict(n_sink=wl.extra["n_sink"], n_recent=wl.extra["n_recent"], window=wl.extra["window"],
              budget_permille=wl.extra["budget_permille"])
    log("sparse 60K layer: setup")
    dm, dec, om, kv = _setup(shape, 23, cap, gamma, ctx, sp)
    G = shape.n_q_heads // shape.n_kv_heads
    toks = [int(t) for t in token_ids(gamma + 1, shape.vocab, 24)]
    dec.tokens.copy_(torch.tensor(toks, dtype=torch.int32))
    log("sparse 60K layer: verify")
    dec.verify()
    torch.cuda.synchronize()
    kv2 = (kv[0].copy(), kv[1].copy())
    scores = []
    ref_t = forward(om, kv2, ctx, toks, scores=scores, score_window=sp["window"])
    got_t = host(dec.target_logits)
    for j in range(gamma + 1):
        assert rel_err(got_t[j], ref_t[j]) < TOL, j
    got = host(dec.kv_score[:, :, :ctx + gamma + 1]).astype(np.float64)
    np.testing.assert_allclose(got[0].sum(axis=1), (gamma + 1) * G, rtol=1e-3)
    assert np.abs(got[0] - scores[0]).max() <= TOL * scores[0].max()
    # index after a rollback of n = 2
    L = ctx + 3
    dec.kv_len.fill_(L)
    _lib.kv_select(dm.c, dec.c)
    torch.cuda.synchronize()
    idx = _gpu_index(dec)
    s, r, K = index_bounds(L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
    assert idx.shape[2] == s + K + (L - r) > 6000
    for hk in range(shape.n_kv_heads):
        ref = select_index(got[0, hk], L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
        np.testing.assert_array_equal(idx[0, hk], ref)
        ref_o = select_index(scores[0][hk], L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
        kth = np.sort(scores[0][hk][s:r])[::-1][K - 1]
        for j in set(ref.tolist()) ^ set(ref_o.tolist()):
            assert abs(scores[0][hk][j] - kth) <= TOL * kth, (hk, j)
    # draft steps over the index, teacher-forced on the GPU's tokens
    log("sparse 60K layer: gathered draft steps")
    dec.tokens[0] = toks[1]
    dec.c.use_index = 1
    index = [[idx[0, hk] for hk in range(shape.n_kv_heads)]]
    for i in range(3):
        _lib.draft_step(dm.c, dec.c, i, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    gtoks = [toks[1]] + host(dec.tokens[1:4]).astype(np.int64).tolist()
    for i in range(3):
        ref_z = forward(om, kv2, L + i, [gtoks[i]], draft=True, sparse=(index, L))[0]
        assert rel_err(host(dec.draft_logits[i]), ref_z) < TOL, i


def test_long_context_shape_properties(cuda):
    """Llama-3.1-8B shape, 60,000 positions of synthetic KV, gamma 11: the
    properties that hold at any size (score sums, index structure, the select
    rule on the GPU's own scores for sampled lists)."""
    wl = CONFIGS["longctx8b"]
    shape, gamma, ctx = wl.shape, wl.gamma, wl.prompt
    cap = ctx + 64
    log("sparse long context: build")
    sp = dict(n_sink=wl.extra["n_sink"], n_recent=wl.extra["n_recent"], window=wl.extra["window"],
              budget_permille=wl.extra["budget_permille"])
    w = model_weights(shape, 0, cuda)
    dm = DeviceModel(shape, w, substitute_layers=range(shape.n_layers))
    dec = SpecDecoder(dm, cap, gamma, 0.0, 0.0, sparse=sp)
    for l in range(shape.n_layers):  # layer by layer: the full history is 7.9 GB
        K, V = kv_history(1, shape.n_kv_heads, ctx, shape.head_dim, ctx, 60 + l, cuda)
        dec.k_cache[l, :, :ctx].copy_(K[0])
        dec.v_cache[l, :, :ctx].copy_(V[0])
    dec.reset(ctx, int(token_ids(1, shape.vocab, 61)[0]))
    G = shape.n_q_heads // shape.n_kv_heads
    for c in range(2):
        log(f"sparse long context: cycle {c}")
        dec.cycle()
        torch.cuda.synchronize()
        n = int(dec.n_accepted.item())
        assert 0 <= n <= gamma
        L = int(dec.kv_len.item())
        sc = dec.kv_score[:, :, :L - n - 1 + gamma + 1].double()
        sums = sc.sum(dim=2).cpu().numpy()
        np.testing.assert_allclose(sums, min(sp["window"], gamma + 1) * G, rtol=1e-3)
        cnt = int(dec.kv_index_len.item())
        assert cnt == _lib.index_count(L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
        idx = dec.kv_index[:, :, :cnt]
        assert bool((idx[:, :, 1:] > idx[:, :, :-1]).all()) and int(idx.max()) < L
        assert bool((idx[:, :, :sp["n_sink"]] == torch.arange(sp["n_sink"], device=cuda)).all())
        rec = torch.arange(L - sp["n_recent"], L, device=cuda)
        assert bool((idx[:, :, -sp["n_recent"]:] == rec).all())
        host_scores = host(dec.kv_score[:, :, :L]).astype(np.float64)
        for l, hk in ((0, 0), (13, 5), (shape.n_layers - 1, shape.n_kv_heads - 1)):
            ref = select_index(host_scores[l, hk], L, sp["n_sink"], sp["n_recent"], sp["budget_permille"])
            np.testing.assert_array_equal(host(idx[l, hk]).astype(np.int64), ref)
