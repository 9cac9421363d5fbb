"""The draft attention inside the QKV projection's launch (tiled low-bit QKV
substitutes, dense keys): bit for bit what the two launches give, for every
key-split count and ring depth it takes, both code widths, the embedding
prologue on a substitute layer, skipped positions and graph replays; the
workspace counts it uses are left at zero and no bounded wait gives up.
Against the oracle the fused path is covered by the draft-step parity tests
(tiled substitutes are the default layout)."""
import numpy as np
import pytest
import torch

from oracle.model import forward
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import kv_history, model_weights, token_ids
from synth.configs import QWEN7B
from tests.gpu_util import log, rel_err
from tests.helpers import host, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2
READY_OFF, READY_END = 48 * 1024, 64 * 1024  # the counts and the give-up word
FAULT_OFF = 65408

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128, vocab=1000,
                    n_shared=1)
TINY_W4 = TINY.with_(n_shared=0)  # layer 0 a substitute: the embedding prologue in the fused launch
LAYER7B = QWEN7B.with_(n_layers=1, n_shared=0)


def _ready_clear(dec):
    torch.cuda.synchronize()
    region = dec.ws[READY_OFF:READY_END].cpu().numpy()
    assert not region[FAULT_OFF - READY_OFF:].any(), "a bounded wait gave up"
    assert not region.any(), np.flatnonzero(region)[:8]


def _steps(dm, dec, K, V, kv_len, tok, steps, own):
    dec.c.attn_own_launch = own
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    dec.reset(kv_len, tok)
    for s in range(steps):
        _lib.draft_step(dm.c, dec.c, s, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    return (dec.draft_logits[:steps].clone(), dec.tokens[:steps + 1].clone(), dec.k_cache.clone(),
            dec.v_cache.clone())


# (shape, kv_len, capacity, bits, steps): key splits 3 (ring 1), 1 (no
# partials), 8 with rings 1 and 2, 2-bit codes, a substitute layer 0
CASES = {
    "tiny_s3": (TINY, 100, 256, 4, 4),
    "tiny_s1": (TINY, 3, 64, 4, 4),
    "tiny_2bit": (TINY, 100, 256, 2, 3),
    "tiny_embed": (TINY_W4, 150, 256, 4, 3),
    "layer7b_ring1": (LAYER7B, 700, 768, 4, 2),
    "layer7b_ring2": (LAYER7B, 1400, 1536, 4, 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_own_launch(cuda, name):
    shape, kv_len, cap, bits, steps = CASES[name]
    log(f"qkv+attn vs own launch: {name}")
    w = model_weights(shape, 21, cuda)
    dm = DeviceModel(shape, w, bits=bits)
    dec = SpecDecoder(dm, cap, 16)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, 22, cuda)
    tok = int(token_ids(1, shape.vocab, 23)[0])
    fused = _steps(dm, dec, K, V, kv_len, tok, steps, 0)
    _ready_clear(dec)
    own = _steps(dm, dec, K, V, kv_len, tok, steps, 1)
    for a, b in zip(fused, own):
        assert torch.equal(a, b)
    # and again fused: the counts left by the first calls were all zero
    again = _steps(dm, dec, K, V, kv_len, tok, steps, 0)
    for a, b in zip(fused, again):
        assert torch.equal(a, b)
    _ready_clear(dec)


def test_fused_layer7b_ring2_matches_oracle(cuda):
    """One 7B substitute layer at 1400 keys (8 key splits, two chunks a wave
    in flight): the fused draft step's logits within 1e-2 of the oracle."""
    shape, kv_len, cap = LAYER7B, 1400, 1536
    log("qkv+attn ring 2 vs oracle")
    w = model_weights(shape, 31, cuda)
    dm = DeviceModel(shape, w)
    dec = SpecDecoder(dm, cap, 4)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, 32, cuda)
    tok = int(token_ids(1, shape.vocab, 33)[0])
    logits, _, _, _ = _steps(dm, dec, K, V, kv_len, tok, 1, 0)
    om = oracle_model(shape, w, dm.substitute_layers)
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    ref = forward(om, kv, kv_len, [tok], draft=True)[0]
    assert rel_err(host(logits[0]), ref) < TOL
    _ready_clear(dec)


def test_fused_skipped_position_leaves_counts_clear(cuda):
    """A draft step past the capacity is skipped by both kinds of block (no
    counts, no waits); the next valid steps still match the own-launch path."""
    shape, cap = TINY, 256
    w = model_weights(shape, 41, cuda)
    dm = DeviceModel(shape, w)
    dec = SpecDecoder(dm, cap, 4)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, cap - 1, shape.head_dim, cap, 42, cuda)
    tok = int(token_ids(1, shape.vocab, 43)[0])
    dec.c.attn_own_launch = 0
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    dec.reset(cap - 1, tok)
    for s in range(3):  # positions cap - 1 (valid), cap, cap + 1 (skipped)
        _lib.draft_step(dm.c, dec.c, s, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    assert int(dec.tokens[2]) == -1 and int(dec.tokens[3]) == -1
    _ready_clear(dec)
    fused = _steps(dm, dec, K, V, 120, tok, 3, 0)
    own = _steps(dm, dec, K, V, 120, tok, 3, 1)
    for a, b in zip(fused, own):
        assert torch.equal(a, b)
    _ready_clear(dec)


def test_fused_graph_replays_match_eager(cuda):
    """Draft steps recorded in a HIP graph and replayed five times, with eager
    work between the replays: every replay equals the eager steps."""
    shape, kv_len, cap, steps = TINY, 90, 256, 3
    w = model_weights(shape, 51, cuda)
    dm = DeviceModel(shape, w)
    dec = SpecDecoder(dm, cap, 4)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, 52, cuda)
    tok = int(token_ids(1, shape.vocab, 53)[0])
    eager = _steps(dm, dec, K, V, kv_len, tok, steps, 0)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    dec.reset(kv_len, tok)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(steps):
                _lib.draft_step(dm.c, dec.c, t, 0.0, None, dec.ws, stream=s.cuda_stream)
    for _ in range(5):
        dec.k_cache.copy_(K)
        dec.v_cache.copy_(V)
        dec.reset(kv_len, tok)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (dec.draft_logits[:steps], dec.tokens[:steps + 1], dec.k_cache, dec.v_cache)
        for a, b in zip(eager, got):
            assert torch.equal(a, b)
        _ready_clear(dec)
    del g
