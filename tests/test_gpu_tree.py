"""The static deep/narrow token tree on the GPU against oracle/tree.py: draft
levels, the tree's verify pass, the tree rejection round and the commit, on
seeded random-init models and synthetic logits."""
import numpy as np
import pytest
import torch

from oracle.cycle import autoregressive_generate
from oracle.sampling import sample as osample
from oracle.tree import (node, n_nodes, tree_forward, tree_reject, tree_commit, tree_generate, root_children)
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import TreeDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import model_weights, kv_history, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.gpu_util import codes_i32, log, rel_err
from tests.helpers import host, memo_weights, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                    vocab=1000, n_shared=1)


def _setup(shape, seed, cap, k, D, kv_len, T=0.0, Td=0.0, device="cuda", graphs=False):
    w = model_weights(shape, seed, device)
    dm = DeviceModel(shape, w)
    dec = TreeDecoder(dm, cap, k, D, T, Td, graphs=graphs)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, seed + 7, device)
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    om = memo_weights(oracle_model(shape, w, dm.substitute_layers))
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    return dm, dec, om, kv


def _uniforms(k, D, cycles, seed, device):
    Ud, _ = uniform_codes(cycles * k * D, seed)
    R, _ = uniform_codes(cycles * (k + D - 1), seed + 1)
    U, _ = uniform_codes(cycles, seed + 2)
    host_u = (Ud.reshape(cycles, k * D), R.reshape(cycles, k + D - 1), U)
    return host_u, tuple(codes_i32(x, device) for x in host_u)


def _check_tree_cycle(dec, om, kv_o, k, D, T, Td, uni_host=None, uni_dev=None, c=0, levels_checked=None,
                      verify_rows=None):
    """One GPU tree cycle, the oracle teacher-forced on the GPU's own tokens:
    draft levels' logits within TOL (levels in ``levels_checked``, default
    all), every drafted token the oracle's choice from the GPU's own draft
    logits, the verify rows within TOL (rows in ``verify_rows``, default
    all), the K/V of every node, the round recomputed by the oracle from the
    GPU's logits bit-exact, and the commit (kv_len, moved K/V) exact.
    Returns (n, chain)."""
    kv_len = int(dec.kv_len.item())
    Ud = [0] * (k * D) if uni_host is None else [int(x) for x in uni_host[0][c]]
    R = [0] * (k + D - 1) if uni_host is None else [int(x) for x in uni_host[1][c]]
    U = 0 if uni_host is None else int(uni_host[2][c])
    if uni_dev is not None:
        dec.ud_buf.copy_(uni_dev[0][c])
        dec.r_buf.copy_(uni_dev[1][c])
        dec.uf_buf.copy_(uni_dev[2][c:c + 1])
    stoch = uni_dev is not None
    dec.draft(dec.ud_buf if stoch else None)
    torch.cuda.synchronize()
    toks = host(dec.tokens).astype(np.int64)
    dz = host(dec.draft_logits).astype(np.float32)
    # the root level
    if levels_checked is None or 0 in levels_checked:
        ref = tree_forward(om, kv_o, kv_len, [0], [int(toks[0])], D, draft=True)[0]
        assert rel_err(dz[0], ref) < TOL, "root"
    else:
        tree_forward(om, kv_o, kv_len, [0], [int(toks[0])], D, draft=True, logit_rows=[])
    assert [int(toks[node(c2, 1, D)]) for c2 in range(k)] == root_children(dz[0], k, Td, Ud[:k])
    for d in range(1, D):
        nodes = [node(c2, d, D) for c2 in range(k)]
        rows = None if levels_checked is None or d in levels_checked else []
        ref = tree_forward(om, kv_o, kv_len, nodes, [int(toks[t]) for t in nodes], D, draft=True, logit_rows=rows)
        for c2 in range(k):
            got = dz[1 + c2 * (D - 1) + d - 1]
            if rows is None:
                assert rel_err(got, ref[c2]) < TOL, (d, c2)
            u = Ud[k + c2 * (D - 1) + d - 1]
            assert osample(got, Td, u) == int(toks[node(c2, d + 1, D)]), (d, c2)
    # the verify pass over every node
    dec.verify()
    torch.cuda.synchronize()
    tz = host(dec.target_logits).astype(np.float32)
    rows = list(range(n_nodes(k, D))) if verify_rows is None else verify_rows
    ref_t = tree_forward(om, kv_o, kv_len, list(range(n_nodes(k, D))), [int(t) for t in toks], D, logit_rows=rows)
    for i, r in enumerate(rows):
        assert rel_err(tz[r], ref_t[i]) < TOL, ("verify row", r)
    sl = slice(kv_len, kv_len + n_nodes(k, D))
    assert rel_err(host(dec.k_cache[:, :, sl]), kv_o[0][:, :, sl]) < TOL
    assert rel_err(host(dec.v_cache[:, :, sl]), kv_o[1][:, :, sl]) < TOL
    # the round, recomputed from the GPU's own logits
    dec.reject(dec.r_buf if stoch else None, dec.uf_buf if stoch else None)
    torch.cuda.synchronize()
    n, chain = int(dec.n_accepted.item()), int(dec.chain.item())
    out = host(dec.out_tokens[:n + 1]).astype(np.int64).tolist()
    assert (n, out, int(dec.status.item()), chain) == tree_reject(tz, dz, toks, k, D, R, U, T, Td), c
    # the commit moves the accepted chain's K/V exactly
    before_k, before_v = dec.k_cache.clone(), dec.v_cache.clone()
    dec.commit()
    torch.cuda.synchronize()
    assert int(dec.kv_len.item()) == kv_len + n + 1
    assert int(dec.tokens[0].item()) == out[-1]
    for i in range(1, n + 1):
        src = kv_len + node(chain, i, D)
        assert torch.equal(dec.k_cache[:, :, kv_len + i], before_k[:, :, src])
        assert torch.equal(dec.v_cache[:, :, kv_len + i], before_v[:, :, src])
    assert torch.equal(dec.k_cache[:, :, :kv_len + 1], before_k[:, :, :kv_len + 1])
    tree_commit(kv_o, kv_len, n, max(chain, 0), D)
    return n, chain


@pytest.mark.parametrize("k,D,T,Td", [(3, 4, 0.0, 0.0), (3, 4, 1.0, 1.0), (2, 5, 0.6, 0.0), (4, 3, 0.0, 0.7),
                                      (1, 6, 1.0, 0.5)])
def test_tree_cycles_tiny_teacher_forced(cuda, k, D, T, Td):
    log(f"tree cycles tiny k={k} D={D} T={T} Td={Td}")
    cycles, ctx = 6, 40
    dm, dec, om, kv = _setup(TINY, 9, 256, k, D, ctx, T, Td)
    dec.reset(ctx, int(token_ids(1, TINY.vocab, 17)[0]))
    kv_o = (kv[0].copy(), kv[1].copy())
    uh, ud = _uniforms(k, D, cycles, 70, cuda) if (T > 0 or Td > 0) else (None, None)
    ns = []
    for c in range(cycles):
        n, chain = _check_tree_cycle(dec, om, kv_o, k, D, T, Td, uh, ud, c)
        ns.append((n, chain))
    log(f"  (n, chain) per cycle: {ns}")


@pytest.mark.parametrize("k,D,T,Td", [(6, 8, 0.0, 0.0), (6, 48, 0.0, 0.0), (6, 8, 1.0, 1.0)])
def test_tree_cycle_7b_layer(cuda, k, D, T, Td):
    """One Qwen2.5-7B-shaped layer (vocab 152064) at 1000 KV positions: a
    tree of k chains, greedy or drawn; with k = 6, D = 48 the verify pass
    runs 289 positions (the GEMMs in three slices of up to 128)."""
    log(f"tree cycle 7B layer k={k} D={D} T={T} Td={Td}")
    shape = QWEN7B.with_(n_layers=1, n_shared=0)
    ctx = 1000
    cap = ctx + n_nodes(k, D) + 16
    dm, dec, om, kv = _setup(shape, 3, cap, k, D, ctx, T, Td)
    dec.reset(ctx, int(token_ids(1, shape.vocab, 11)[0]))
    kv_o = (kv[0].copy(), kv[1].copy())
    levels = None if D <= 8 else [0, 1, D // 2, D - 1]
    rows = None if D <= 8 else sorted({0, 1, 2, D, D + 1, 2 * D, 3 * D + 7, 5 * D + 1, n_nodes(k, D) - 1})
    uh, ud = _uniforms(k, D, 1, 77, cuda) if (T > 0 or Td > 0) else (None, None)
    n, chain = _check_tree_cycle(dec, om, kv_o, k, D, T, Td, uh, ud, levels_checked=levels, verify_rows=rows)
    log(f"  n={n} chain={chain}")


def test_greedy_tree_generation_matches_oracle(cuda):
    log("greedy tree generation tiny")
    k, D = 3, 4
    dm, dec, om, _ = _setup(TINY, 8, 256, k, D, 0)
    prompt = [int(t) for t in token_ids(9, TINY.vocab, 13)]
    G = 24
    got, ns = dec.generate(prompt, G)
    z = np.zeros((64, k * D), np.int64)
    ref, ref_ns = tree_generate(om, prompt, G, k, D, 0.0, 0.0, (z, np.zeros((64, k + D - 1), np.int64),
                                                                    np.zeros(64, np.int64)), 256)
    assert ref == autoregressive_generate(om, prompt, G, 0.0, np.zeros(G, np.int64), 256)
    assert got == ref
    assert ns == ref_ns[:len(ns)]
    assert int(dec.kv_len.item()) == len(prompt) - 1 + sum(n + 1 for n in ns)


def _exact_weights(shape, seed, device):
    """Every layer the identity (zero weights), embedding rows of +-1 and an
    lm_head of small multiples of 2^-4: every logit is an exact sum, so
    draft and target logits are bit-identical on both sides."""
    w = model_weights(shape, seed, device)
    g = torch.Generator(device="cpu").manual_seed(seed)
    for lw in w["layers"]:
        for name in ("qkv", "o", "gate_up", "down"):
            lw[name].zero_()
    sign = torch.randint(0, 2, (shape.vocab, shape.hidden), generator=g) * 2 - 1
    w["embed"].copy_(sign.to(torch.bfloat16))
    lm = torch.randint(-1, 2, (shape.vocab, shape.hidden), generator=g).float() * 0.0625
    w["lm_head"].copy_(lm.to(torch.bfloat16))
    return w


@pytest.mark.parametrize("T,Td", [(1.0, 1.0), (1.0, 0.5), (0.6, 0.0)])
def test_stochastic_tree_generation_exact_model(cuda, T, Td):
    log(f"stochastic tree generation, exact model, T={T} Td={Td}")
    shape = TINY
    k, D, G = 3, 3, 20
    w = _exact_weights(shape, 21, cuda)
    dm = DeviceModel(shape, w)
    dec = TreeDecoder(dm, 256, k, D, T, Td)
    om = oracle_model(shape, w, dm.substitute_layers)
    prompt = [int(t) for t in token_ids(5, shape.vocab, 23)]
    uh, ud = _uniforms(k, D, G, 95, cuda)
    got, ns = dec.generate(prompt, G, ud)
    ref, ref_ns = tree_generate(om, prompt, G, k, D, T, Td, uh, 256)
    assert got == ref
    assert ns == ref_ns[:len(ns)]


def test_tree_graph_replay_equals_eager(cuda):
    log("tree graph replay")
    k, D = 3, 4
    prompt = [int(t) for t in token_ids(7, TINY.vocab, 3)]
    outs = []
    for graphs in (False, True):
        dm, dec, om, _ = _setup(TINY, 4, 256, k, D, 0, graphs=graphs)
        outs.append(dec.generate(prompt, 30))
    assert outs[0] == outs[1]


def test_tree_that_does_not_fit_emits_one_token(cuda):
    """kv_len + 1 + k D above the capacity: every child is -1 (no node
    written past the cache), the round skips them and emits the target's
    token at the root, and the commit advances kv_len by one."""
    log("tree past capacity")
    k, D = 3, 4
    cap = 128
    dm, dec, om, kv = _setup(TINY, 6, cap, k, D, cap - 6)
    dec.reset(cap - 6, int(token_ids(1, TINY.vocab, 2)[0]))
    before_k = dec.k_cache.clone()
    root = int(token_ids(1, TINY.vocab, 2)[0])
    dec.cycle()
    torch.cuda.synchronize()
    assert (host(dec.tokens[1:]) == -1).all()
    assert int(dec.n_accepted.item()) == 0 and int(dec.chain.item()) == -1
    assert int(dec.status.item()) == _lib.STATUS_Q_ZERO
    assert int(dec.kv_len.item()) == cap - 5
    ref = tree_forward(om, (kv[0].copy(), kv[1].copy()), cap - 6, [0], [root], D)[0]
    got = host(dec.target_logits[0])
    assert rel_err(got, ref) < TOL
    assert int(dec.out_tokens[0].item()) == int(np.argmax(got))
    # slots past the root were written only below the capacity; the history is intact
    assert torch.equal(dec.k_cache[:, :, :cap - 6], before_k[:, :, :cap - 6])


def _tree_logits(k, D, V, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    zt = (np.round(rng.normal(0, 2.0, (n_nodes(k, D), V)) * 8) / 8).astype(np.float32)
    zd = np.concatenate([zt[:1], zt[1:1 + k * (D - 1)]])  # draft rows near the target's
    zd = (zd + np.round(rng.normal(0, spread, zd.shape) * 8) / 8).astype(np.float32)
    return zt, zd


@pytest.mark.parametrize("k,D,V,T,Td", [(6, 48, 1000, 0.0, 0.0), (6, 48, 1000, 1.0, 1.0), (6, 8, 1000, 0.6, 0.0),
                                        (4, 4, 152064, 1.0, 1.0), (6, 48, 152064, 0.6, 0.6),
                                        (3, 1, 500, 1.0, 0.8), (1, 16, 1000, 1.0, 1.0)])
def test_tree_reject_matches_oracle(cuda, k, D, V, T, Td):
    """The round on synthetic bf16 logits, children and chains drawn from the
    draft rows (or greedy), against the oracle bit-exact; the first children
    are pushed towards rejection (their q large where p is small) so that
    the multi-step residuals are exercised."""
    log(f"tree reject k={k} D={D} V={V} T={T} Td={Td}")
    trials = 6 if V > 10000 else 20
    ws = torch.zeros(1 << 26, dtype=torch.uint8, device=cuda)
    _lib.workspace_init(ws)
    seen_chain = set()
    for t in range(trials):
        zt, zd = _tree_logits(k, D, V, 100 + t, spread=1.0 + t % 3)
        Ud, _ = uniform_codes(k * D, 300 + t)
        R, _ = uniform_codes(k + D - 1, 400 + t)
        U = int(uniform_codes(1, 500 + t)[0][0])
        toks = np.zeros(n_nodes(k, D), np.int64)
        toks[0] = 7
        for c, x in enumerate(root_children(zd[0], k, Td, Ud[:k])):
            toks[node(c, 1, D)] = x
        for c in range(k):
            for d in range(1, D):
                toks[node(c, d + 1, D)] = osample(zd[1 + c * (D - 1) + d - 1], Td, int(Ud[k + c * (D - 1) + d - 1]))
        if t % 4 == 1:
            toks[node(0, 1, D)] = -1  # a child outside the vocabulary is skipped
        if t % 4 == 2 and k > 1:
            toks[node(1, 1, D)] = toks[node(0, 1, D)]  # duplicate children
        zt_d = torch.from_numpy(zt).to(torch.bfloat16).to(cuda)
        zd_d = torch.from_numpy(zd).to(torch.bfloat16).to(cuda)
        tk = torch.from_numpy(toks.astype(np.int32)).to(cuda)
        rr = codes_i32(R, cuda)
        uu = codes_i32([U], cuda)
        n_d = torch.zeros(1, dtype=torch.int32, device=cuda)
        ch = torch.zeros(1, dtype=torch.int32, device=cuda)
        out = torch.zeros(D + 1, dtype=torch.int32, device=cuda)
        st = torch.zeros(1, dtype=torch.int32, device=cuda)
        _lib.tree_reject(k, D, V, T, Td, zt_d, zd_d, tk, rr, uu, n_d, ch, out, st, ws)
        torch.cuda.synchronize()
        n = int(n_d.item())
        got = (n, host(out[:n + 1]).astype(np.int64).tolist(), int(st.item()), int(ch.item()))
        ref = tree_reject(host(zt_d).astype(np.float32), host(zd_d).astype(np.float32), toks, k, D,
                          [int(r) for r in R], U, T, Td)
        assert got == ref, (t, got, ref)
        seen_chain.add(ref[3])
    log(f"  accepted chains seen: {sorted(seen_chain)}")
    if k > 1 and V == 1000 and Td > 0:  # the seeded cases reach later chains and all-rejected roots
        assert -1 in seen_chain and max(seen_chain) > 0


def test_tree_reject_zero_residual_and_skipped_children(cuda):
    """Crafted rounds (the oracle's own pins): p = q with a weight-0 first
    child (rejected, q(x) = 0, no residual mass -> back to p, status 2 | 4,
    the next child accepted), and children outside the vocabulary."""
    z = np.array([1.0, 0.5, -0.25, 2.0, 0.0, 2.0 - 40.0], dtype=np.float32)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=cuda)
    _lib.workspace_init(ws)
    cases = [(2, 1, np.stack([z, z, z]), z[None], [0, 5, 3], [0, (1 << 24) - 1], 0, 1.0, 1.0),
             (2, 1, np.stack([z, z, z]), z[None], [0, -1, 3], [0, 0], 0, 0.0, 0.0),
             (2, 1, np.stack([z, z, z]), z[None], [0, -1, 6], [0, 0], 77, 1.0, 1.0),
             (2, 2, np.stack([z] * 5), np.stack([z] * 3), [0, 5, 1, 3, 2], [0, (1 << 24) - 1, 5], 9, 1.0, 1.0)]
    for k, D, zt, zd, toks, R, U, T, Td in cases:
        zt_d = torch.from_numpy(zt).to(torch.bfloat16).to(cuda)
        zd_d = torch.from_numpy(zd.astype(np.float32)).to(torch.bfloat16).to(cuda)
        tk = torch.tensor(toks, dtype=torch.int32, device=cuda)
        n_d, ch, st = (torch.zeros(1, dtype=torch.int32, device=cuda) for _ in range(3))
        out = torch.zeros(D + 1, dtype=torch.int32, device=cuda)
        _lib.tree_reject(k, D, 6, T, Td, zt_d, zd_d, tk, codes_i32(R, cuda), codes_i32([U], cuda), n_d, ch, out,
                         st, ws)
        torch.cuda.synchronize()
        n = int(n_d.item())
        got = (n, host(out[:n + 1]).astype(np.int64).tolist(), int(st.item()), int(ch.item()))
        ref = tree_reject(zt, zd, np.array(toks), k, D, R, U, T, Td)
        assert got == ref, (toks, got, ref)
    assert tree_reject(cases[0][2], cases[0][3], np.array(cases[0][4]), 2, 1, cases[0][5], 0, 1.0, 1.0)[2] == \
        _lib.STATUS_Q_ZERO | _lib.STATUS_ZERO_RESIDUAL
