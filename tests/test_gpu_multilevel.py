"""Multi-level substitutes on the GPU (a 2-bit draft for the 4-bit draft)
against oracle/multilevel.py: every inner round's drafts, 4-bit pass and
decision, and the outer verify and decision, teacher-forced on the GPU's
tokens; greedy generation against autoregressive decoding; stochastic
generation on an exactly-representable model."""
import numpy as np
import pytest
import torch

from oracle.cycle import autoregressive_generate
from oracle.model import forward
from oracle.multilevel import multilevel_generate
from oracle.reject import reject as oreject
from oracle.sampling import sample as osample
from self_speculative_decoding_w4a16_amd.engine import MultiLevelDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import model_weights, kv_history, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.gpu_util import log, rel_err
from tests.helpers import host, memo_weights, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                    vocab=1000, n_shared=1)


def _models(shape, w):
    dm4 = DeviceModel(shape, w)
    dm2 = DeviceModel(shape, w, bits=2)
    om4 = oracle_model(shape, w, dm4.substitute_layers)
    om2 = oracle_model(shape, w, [])
    om2.make_substitutes(dm4.substitute_layers, bits=2)
    return dm4, dm2, om4, om2


def _uniforms(cycles, gamma, gamma2, seed):
    U2, _ = uniform_codes(cycles * gamma * gamma2, seed)
    R2, _ = uniform_codes(cycles * gamma * gamma2, seed + 1)
    F2, _ = uniform_codes(cycles * gamma, seed + 2)
    R, _ = uniform_codes(cycles * gamma, seed + 3)
    U, _ = uniform_codes(cycles, seed + 4)
    return (U2.reshape(cycles, gamma, gamma2), R2.reshape(cycles, gamma, gamma2), F2.reshape(cycles, gamma),
            R.reshape(cycles, gamma), U)


@pytest.mark.parametrize("T,T_mid,T2", [(0.0, 0.0, 0.0), (1.0, 1.0, 1.0), (0.0, 0.6, 0.0), (0.8, 0.0, 1.0)])
def test_multilevel_cycles_teacher_forced(cuda, T, T_mid, T2):
    log(f"multi-level cycles T={T} T_mid={T_mid} T2={T2}")
    _check_cycles(TINY, 9, 40, 256, 6, 3, T, T_mid, T2, 3, cuda)


@pytest.mark.parametrize("T,T_mid,T2", [(0.0, 0.0, 0.0), (1.0, 1.0, 1.0)])
def test_multilevel_cycle_7b_layer(cuda, T, T_mid, T2):
    """One Qwen2.5-7B-shaped layer (4-bit and 2-bit substitutes, vocab
    152064) at 1000 KV positions, the bench's gamma = 16 and gamma2 = 4."""
    log(f"multi-level cycle 7B layer T={T} T_mid={T_mid} T2={T2}")
    _check_cycles(QWEN7B.with_(n_layers=1, n_shared=0), 5, 1000, 1040, 16, 4, T, T_mid, T2, 1, cuda)


def _check_cycles(shape, seed, ctx, cap, gamma, gamma2, T, T_mid, T2, cycles, cuda):
    w = model_weights(shape, seed, cuda)
    dm4, dm2, om4, om2 = _models(shape, w)
    memo_weights(om4)
    memo_weights(om2)
    dec = MultiLevelDecoder(dm4, dm2, cap, gamma, gamma2, T, T_mid, T2)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, ctx, shape.head_dim, cap, 16, cuda)
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    kv_o = (host(K).astype(np.float64), host(V).astype(np.float64))
    dec.reset(ctx, int(token_ids(1, shape.vocab, 17)[0]))
    uni = _uniforms(cycles, gamma, gamma2, 70)
    for c in range(cycles):
        kv_len = int(dec.kv_len.item())
        U2, R2, F2, R, U = (u[c] for u in uni)
        base, r = 0, 0
        while base < gamma:  # the inner rounds, one at a time
            g = min(gamma2, gamma - base)
            dec.u2_buf[base:base + g] = torch.as_tensor(U2[r][:g], dtype=torch.int32)
            dec.r2_buf[:g] = torch.as_tensor(R2[r][:g], dtype=torch.int32)
            dec.f2_buf[0] = int(F2[r])
            n = dec.inner_round(base, g)
            torch.cuda.synchronize()
            toks = host(dec.tokens).astype(np.int64).tolist()
            zi = host(dec.inner_logits[base:base + g]).astype(np.float32)
            zm = host(dec.mid_logits[base:base + g + 1]).astype(np.float32)
            # the 2-bit drafts, re-drawn from the GPU's 2-bit logits; the append
            # replaced drafted token n by the round's last token
            seq = [toks[base]]
            for i in range(g):
                ref = forward(om2, kv_o, kv_len + base + i, [seq[-1]], draft=True)[0]
                assert rel_err(zi[i], ref) < TOL, (c, r, i)
                seq.append(osample(zi[i], T2, int(U2[r][i])))
                if i != n:
                    assert toks[base + 1 + i] == seq[-1], (c, r, i)
            ref_m = forward(om4, kv_o, kv_len + base, seq, draft=True)
            for j in range(g + 1):
                assert rel_err(zm[j], ref_m[j]) < TOL, (c, r, j)
            n_ref, out_ref, st_ref = oreject(zm, zi, seq[1:], list(R2[r][:g]), int(F2[r]), T_mid, T2)
            assert (n, int(dec.in_status.item())) == (n_ref, st_ref), (c, r)
            assert host(dec.in_out[:n + 1]).astype(np.int64).tolist() == out_ref
            assert toks[base + 1 + n] == out_ref[-1]  # the round's last token appended
            base += min(n + 1, gamma - base)
            r += 1
        log(f"  cycle {c}: {r} inner rounds")
        # the outer round over the gamma middle tokens
        dec.verify()
        if T > 0:
            dec.r_buf[:gamma] = torch.as_tensor(R[:gamma], dtype=torch.int32)
            dec.uf_buf[0] = int(U)
            dec.reject(dec.r_buf, dec.uf_buf)
        else:
            dec.reject()
        torch.cuda.synchronize()
        toks = host(dec.tokens[:gamma + 1]).astype(np.int64).tolist()
        tz = host(dec.target_logits).astype(np.float32)
        mz = host(dec.mid_logits[:gamma]).astype(np.float32)
        ref_t = forward(om4, kv_o, kv_len, toks)
        for j in range(gamma + 1):
            assert rel_err(tz[j], ref_t[j]) < TOL, (c, j)
        n = int(dec.n_accepted.item())
        got = (n, host(dec.out_tokens[:n + 1]).astype(np.int64).tolist(), int(dec.status.item()))
        assert got == oreject(tz, mz, toks[1:], list(R[:gamma]), int(U), T, T_mid), c
        dec.commit()
        torch.cuda.synchronize()
        assert int(dec.kv_len.item()) == kv_len + n + 1


def test_greedy_multilevel_generation_matches_oracle(cuda):
    log("multi-level greedy generation")
    w = model_weights(TINY, 8, cuda)
    dm4, dm2, om4, om2 = _models(TINY, w)
    dec = MultiLevelDecoder(dm4, dm2, 256, 5, 2)
    prompt = [int(t) for t in token_ids(9, TINY.vocab, 13)]
    G = 20
    got, ns = dec.generate(prompt, G)
    assert got == autoregressive_generate(om4, prompt, G, 0.0, np.zeros(G, np.int64), 256)
    assert int(dec.kv_len.item()) == len(prompt) - 1 + sum(n + 1 for n in ns)


def _exact_weights(shape, seed, device):
    """Every layer the identity (zero weights), embedding rows of +-1 and an
    lm_head of small multiples of 2^-4: exact logits on both sides (the
    2-bit and 4-bit substitutes of zero weights are zero)."""
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


@pytest.mark.parametrize("T,T_mid,T2", [(1.0, 1.0, 1.0), (1.0, 0.5, 0.8)])
def test_stochastic_multilevel_generation_exact_model(cuda, T, T_mid, T2):
    log(f"multi-level stochastic generation, exact model, T={T} T_mid={T_mid} T2={T2}")
    gamma, gamma2, G = 4, 2, 16
    w = _exact_weights(TINY, 21, cuda)
    dm4, dm2, om4, om2 = _models(TINY, w)
    dec = MultiLevelDecoder(dm4, dm2, 256, gamma, gamma2, T, T_mid, T2)
    prompt = [int(t) for t in token_ids(5, TINY.vocab, 23)]
    uni = _uniforms(G, gamma, gamma2, 95)
    got, ns = dec.generate(prompt, G, uni)
    ref, ref_ns = multilevel_generate(om4, om2, prompt, G, gamma, gamma2, T, T_mid, T2, uni, 256)
    assert got == ref
    assert ns == ref_ns[:len(ns)]
