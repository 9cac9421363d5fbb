"""Recorded cycles (HIP graph replay) against eager cycles: the same kernels
with the same arguments, so every replay must reproduce the eager decoder
bit for bit.  Replays are separated by the host's own work (uniform copies,
reading back the emitted tokens), and every cycle is compared."""
import numpy as np
import pytest
import torch

from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import kv_history, model_weights, token_ids, uniform_codes
from synth.configs import LLAMA8B, QWEN7B
from tests.gpu_util import codes_i32, log

pytestmark = pytest.mark.gpu

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                    vocab=1000, n_shared=1)
TINY_L = LLAMA8B.with_(n_layers=2, hidden=256, ffn=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                       vocab=1000, n_shared=0)


def _pair(shape, seed, cap, gamma, T, Td, sparse=None, ctx=0, cuda="cuda"):
    w = model_weights(shape, seed, cuda)
    dm = DeviceModel(shape, w)
    decs = [SpecDecoder(dm, cap, gamma, T, Td, sparse=sparse, graphs=g) for g in (False, True)]
    if ctx:
        K, V = kv_history(shape.n_layers, shape.n_kv_heads, ctx, shape.head_dim, cap, seed + 3, cuda)
        for d in decs:
            d.load_kv(K, V, ctx, 5)
    return decs


def _run_and_compare(decs, cycles, uni=None):
    for c in range(cycles):
        outs = []
        for d in decs:
            if uni is None:
                d.cycle()
            else:
                d.cycle(uni[0][c], uni[1][c], uni[2][c:c + 1])
            n = int(d.n_accepted.item())
            outs.append((n, d.out_tokens[:n + 1].tolist(), int(d.kv_len.item()), int(d.status.item())))
        assert outs[0] == outs[1], (c, outs)
        a, b = decs
        assert torch.equal(a.draft_logits, b.draft_logits), c
        assert torch.equal(a.target_logits, b.target_logits), c
        if a.sparse:
            assert torch.equal(a.kv_index, b.kv_index) and torch.equal(a.kv_index_len, b.kv_index_len), c
    assert decs[1]._graphs, "no cycle was replayed from a graph"


def test_graph_replay_matches_eager_greedy(cuda):
    log("graphs: greedy")
    decs = _pair(TINY, 31, 256, 4, 0.0, 0.0)
    prompt = [int(t) for t in token_ids(9, TINY.vocab, 32)]
    for d in decs:
        d.prefill(prompt)
    _run_and_compare(decs, 8)


def test_graph_replay_matches_eager_stochastic(cuda):
    log("graphs: stochastic")
    gamma, cycles = 4, 8
    decs = _pair(TINY, 33, 256, gamma, 1.0, 0.5)
    prompt = [int(t) for t in token_ids(7, TINY.vocab, 34)]
    for d in decs:
        d.prefill(prompt)
    Ud, _ = uniform_codes(cycles * gamma, 35)
    R, _ = uniform_codes(cycles * gamma, 36)
    Uf, _ = uniform_codes(cycles, 37)
    uni = (codes_i32(Ud.reshape(cycles, gamma), cuda), codes_i32(R.reshape(cycles, gamma), cuda),
           codes_i32(Uf, cuda))
    _run_and_compare(decs, cycles, uni)


def test_graph_replay_matches_eager_sparse(cuda):
    log("graphs: sparse draft")
    sp = dict(n_sink=4, n_recent=16, window=16, budget_permille=150)
    decs = _pair(TINY_L, 38, 700, 4, 0.0, 0.0, sparse=sp, ctx=600)
    _run_and_compare(decs, 6)
    # after a reset the first cycle is dense again, then the recorded sparse cycle
    for d in decs:
        d.reset(600, 9)
    _run_and_compare(decs, 3)
