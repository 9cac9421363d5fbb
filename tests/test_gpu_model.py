"""Model-level parity: draft step, verify pass and whole cycles on the GPU
against the oracle forward, on seeded random-init models."""
import numpy as np
import pytest
import torch

from oracle.cycle import speculative_generate, autoregressive_generate
from oracle.model import forward, new_kv
from oracle.sampling import argmax_lowest
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import model_weights, kv_history, token_ids, uniform_codes
from synth.configs import QWEN7B, QWEN32B
from tests.gpu_util import codes_i32, log, rel_err
from tests.helpers import host, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                    vocab=1000, n_shared=1)


def _argmax_ok(gpu_tok, gpu_logits, ref_logits):
    """GPU token is the argmax of its own logits, and the oracle's argmax unless
    the oracle's top logits are tied within the logits tolerance."""
    g = np.asarray(gpu_logits, np.float64)
    r = np.asarray(ref_logits, np.float64)
    assert gpu_tok == argmax_lowest(g)
    ro = argmax_lowest(r)
    if gpu_tok != ro:
        assert r[ro] - r[gpu_tok] <= TOL * np.abs(r).max(), (gpu_tok, ro)
    return gpu_tok == ro


def _setup(shape, seed, cap, gamma, kv_len, subs=None, T=0.0, Td=0.0, device="cuda"):
    w = model_weights(shape, seed, device)
    dm = DeviceModel(shape, w, subs)
    dec = SpecDecoder(dm, cap, gamma, T, Td)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, seed + 7, device)
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    om = oracle_model(shape, w, dm.substitute_layers)
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    return dm, dec, om, kv


@pytest.mark.parametrize("shape_name", ["tiny", "tiny_short", "layer7b", "layer7b_cap1024", "layer7b_ctx40k",
                                        "layer32b"])
def test_draft_step_and_verify_match_oracle(cuda, shape_name):
    gamma = 16
    if shape_name == "tiny":
        shape, kv_len, cap = TINY, 100, 256
    elif shape_name == "tiny_short":
        shape, kv_len, cap = TINY, 3, 64
    elif shape_name == "layer7b":
        shape, kv_len, cap = QWEN7B.with_(n_layers=1, n_shared=0), 1024, 1088
    elif shape_name == "layer7b_cap1024":
        shape, kv_len, cap = QWEN7B.with_(n_layers=1, n_shared=0), 1000, 1024
    elif shape_name == "layer7b_ctx40k":
        # long context: the verify attention walks several 128-key tiles per block
        shape, kv_len, cap = QWEN7B.with_(n_layers=1, n_shared=0), 40000, 40064
    else:  # one 32B-shaped layer at the 32B workload's context and draft length
        shape, kv_len, cap, gamma = QWEN32B.with_(n_layers=1, n_shared=0), 2048, 2112, 48
    log(f"draft/verify parity {shape_name}")
    dm, dec, om, kv = _setup(shape, 3, cap, gamma, kv_len)
    toks = token_ids(gamma + 1, shape.vocab, 11)
    dec.reset(kv_len, toks[0])
    # draft step 0
    _lib.draft_step(dm.c, dec.c, 0, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    ref = forward(om, (kv[0].copy(), kv[1].copy()), kv_len, [int(toks[0])], draft=True)[0]
    got = host(dec.draft_logits[0])
    assert rel_err(got, ref) < TOL
    _argmax_ok(int(dec.tokens[1].item()), got, ref)
    # verify gamma+1 positions (synthetic draft tokens)
    dec.tokens.copy_(torch.tensor(toks, dtype=torch.int32))
    dec.verify()
    torch.cuda.synchronize()
    kv2 = (kv[0].copy(), kv[1].copy())
    ref_v = forward(om, kv2, kv_len, [int(t) for t in toks], draft=False)
    got_v = host(dec.target_logits)
    for j in range(gamma + 1):
        assert rel_err(got_v[j], ref_v[j]) < TOL, j
    # committed target K/V of the verified positions
    kc = host(dec.k_cache[:, :, kv_len:kv_len + gamma + 1])
    vc = host(dec.v_cache[:, :, kv_len:kv_len + gamma + 1])
    assert rel_err(kc, kv2[0][:, :, kv_len:kv_len + gamma + 1]) < TOL
    assert rel_err(vc, kv2[1][:, :, kv_len:kv_len + gamma + 1]) < TOL
    # history untouched
    assert torch.equal(dec.k_cache[:, :, :kv_len].cpu(), torch.from_numpy(kv[0][:, :, :kv_len]).to(torch.bfloat16))


def test_verify_row_equals_draft_decode_when_shared(cuda):
    # with no substitutes, draft step i and verify row i run the same weights
    shape = TINY.with_(n_shared=TINY.n_layers)
    dm, dec, om, kv = _setup(shape, 5, 256, 4, 40, subs=[])
    toks = token_ids(1, shape.vocab, 2)
    dec.reset(40, toks[0])
    dec.draft()
    dec.verify()
    torch.cuda.synchronize()
    d = host(dec.draft_logits)
    v = host(dec.target_logits)
    for i in range(4):
        assert rel_err(d[i], v[i]) < TOL
    # the draft tokens were drawn greedily from the same model: verify accepts them all
    dec.reject()
    torch.cuda.synchronize()
    assert int(dec.n_accepted.item()) == 4


@pytest.mark.parametrize("cap", [256, 1024])
def test_draft_steps_past_capacity_are_skipped(cuda, cap):
    """Positions at or past the KV capacity are skipped on the device (token -1,
    no K/V written, the draft attention's split blocks all leave before they
    count in); the next in-range draft step still matches the oracle, so the
    per-head arrival counters were left at zero."""
    gamma = 4
    log(f"draft steps past capacity, cap {cap}")
    dm, dec, om, kv = _setup(TINY, 13, cap, gamma, cap - 2)
    toks = token_ids(2, TINY.vocab, 5)
    dec.reset(cap - 2, toks[0])
    for step in range(gamma):
        _lib.draft_step(dm.c, dec.c, step, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    t = dec.tokens.cpu().numpy()
    assert t[1] >= 0 and t[2] >= 0  # positions cap-2, cap-1
    assert t[3] == -1 and t[4] == -1  # positions cap, cap+1: skipped
    # an in-range step afterwards
    kv_len = cap // 2
    dec.k_cache.copy_(torch.from_numpy(kv[0]).to(torch.bfloat16))
    dec.v_cache.copy_(torch.from_numpy(kv[1]).to(torch.bfloat16))
    dec.reset(kv_len, toks[1])
    _lib.draft_step(dm.c, dec.c, 0, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    ref = forward(om, (kv[0].copy(), kv[1].copy()), kv_len, [int(toks[1])], draft=True)[0]
    got = host(dec.draft_logits[0])
    assert rel_err(got, ref) < TOL
    _argmax_ok(int(dec.tokens[1].item()), got, ref)


def test_greedy_generation_matches_oracle(cuda):
    log("greedy generation tiny")
    dm, dec, om, _ = _setup(TINY, 8, 256, 4, 0)
    prompt = [int(t) for t in token_ids(9, TINY.vocab, 13)]
    G = 24
    got, ns = dec.generate(prompt, G)
    ref_sd, ref_ns = speculative_generate(om, prompt, G, 4, 0.0, 0.0, None_uniforms(64, 4), 256)
    ref_ar = autoregressive_generate(om, prompt, G, 0.0, np.zeros(G, np.int64), 256)
    assert ref_sd == ref_ar
    assert got == ref_sd
    assert ns == ref_ns[:len(ns)]
    assert int(dec.kv_len.item()) == len(prompt) - 1 + sum(n + 1 for n in ns)


def None_uniforms(cycles, gamma):
    z = np.zeros((cycles, gamma), np.int64)
    return z, z, np.zeros(cycles, np.int64)


def _exact_weights(shape, seed, device):
    """A model whose forward is exact in float32 and float64 alike: zero layer
    weights (every layer is the identity on the residual stream), embedding
    rows of +-1 (RMSNorm maps them to +-1 exactly in bf16) and an lm_head of
    small multiples of 2^-4, so every logit is an exact sum.  Draft and
    target then see bit-identical logits and every stochastic decision must
    agree exactly."""
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


@pytest.mark.parametrize("T,Td", [(1.0, 1.0), (1.0, 0.5), (0.6, 0.0), (0.0, 0.2)])
def test_stochastic_generation_exact_model(cuda, T, Td):
    log(f"stochastic exact-model generation T={T} Td={Td}")
    shape = TINY
    gamma, G = 4, 24
    w = _exact_weights(shape, 21, cuda)
    dm = DeviceModel(shape, w)
    dec = SpecDecoder(dm, 256, gamma, T, Td)
    om = oracle_model(shape, w, dm.substitute_layers)
    prompt = [int(t) for t in token_ids(5, shape.vocab, 23)]
    cycles = G
    Ud, _ = uniform_codes(cycles * gamma, 91)
    R, _ = uniform_codes(cycles * gamma, 92)
    Uf, _ = uniform_codes(cycles, 93)
    Ud, R = Ud.reshape(cycles, gamma), R.reshape(cycles, gamma)
    uni = (codes_i32(Ud, cuda), codes_i32(R, cuda), codes_i32(Uf, cuda))
    got, ns = dec.generate(prompt, G, uni)
    ref, ref_ns = speculative_generate(om, prompt, G, gamma, T, Td, (Ud, R, Uf), 256)
    assert got == ref
    assert ns == ref_ns[:len(ns)]
    if T > 0 and Td != T:
        assert min(ns) < gamma  # the residual path was taken


def _teacher_forced_cycles(dec, om, kv_o, gamma, cycles, T, Td, uni=None, draft_checked=None,
                           kv_o32=None):
    """GPU cycles with the oracle teacher-forced on the GPU's own draft tokens:
    draft and verify logits within TOL of the oracle forward (the first
    ``draft_checked`` draft steps, default all), every draft token the
    oracle's draw from the GPU's own draft logits, and the rejection round
    recomputed by the oracle from the GPU's own logits, tokens and uniforms,
    bit-exact (n, emitted tokens, status).  Verify overwrites the draft's K/V
    of every speculative position, so unchecked draft steps do not change the
    oracle's cache for the verify pass.
    ``kv_o32`` (deep models): a second oracle cache, on which the oracle runs
    the same cycle with float32 sums; logits must then lie within
    max(TOL, 2 x the distance between the float64- and float32-summed
    evaluations), the spread that bf16 roundings compound to over many
    random-init layers.  Returns the per-cycle n."""

    def check(got, ref, ref32, where):
        tol = TOL if ref32 is None else max(TOL, 2.0 * rel_err(ref32, ref))
        e = rel_err(got, ref)
        if ref32 is not None:
            log(f"  {where}: rel_err {e:.4f}, f32/f64 oracle spread {rel_err(ref32, ref):.4f}, tol {tol:.4f}")
        assert e < tol, (where, e, tol)

    from oracle.reject import reject as oreject
    from oracle.sampling import sample as osample
    ns = []
    for c in range(cycles):
        kv_len = int(dec.kv_len.item())
        last = int(dec.tokens[0].item())
        if uni is not None:
            dec.cycle(uni[0][c], uni[1][c], uni[2][c:c + 1])
        else:
            dec.cycle()
        torch.cuda.synchronize()
        toks = [last] + host(dec.tokens[1:gamma + 1]).astype(np.int64).tolist()
        dz = host(dec.draft_logits[:gamma]).astype(np.float32)
        tz = host(dec.target_logits[:gamma + 1]).astype(np.float32)
        Ud = [0] * gamma if uni is None else host(uni[0][c]).astype(np.int64).tolist()
        R = [0] * gamma if uni is None else host(uni[1][c]).astype(np.int64).tolist()
        U = 0 if uni is None else int(host(uni[2][c]))
        for i in range(gamma):
            if draft_checked is None or i < draft_checked:
                ref = forward(om, kv_o, kv_len + i, [toks[i]], draft=True)[0]
                ref32 = None
                if kv_o32 is not None:
                    ref32 = forward(om, kv_o32, kv_len + i, [toks[i]], draft=True, acc=np.float32)[0]
                check(dz[i], ref, ref32, f"cycle {c} draft {i}")
            assert osample(dz[i], Td, Ud[i]) == toks[i + 1], (c, i)
        ref_t = forward(om, kv_o, kv_len, toks)
        ref_t32 = None if kv_o32 is None else forward(om, kv_o32, kv_len, toks, acc=np.float32)
        for j in range(gamma + 1):
            check(tz[j], ref_t[j], None if ref_t32 is None else ref_t32[j], f"cycle {c} verify row {j}")
        n = int(dec.n_accepted.item())
        out = host(dec.out_tokens[:n + 1]).astype(np.int64).tolist()
        assert (n, out, int(dec.status.item())) == oreject(tz, dz, toks[1:], R, U, T, Td), c
        assert int(dec.kv_len.item()) == kv_len + n + 1
        ns.append(n)
    return ns


@pytest.mark.parametrize("T,Td", [(1.0, 1.0), (0.0, 0.2), (0.6, 0.6), (1.0, 0.0)])
def test_stochastic_cycles_random_model_teacher_forced(cuda, T, Td):
    """Random-init model at T > 0 (or a sharpened draft): logits agree with the
    oracle to the bf16 tolerance only, so whole generations may part at CDF
    boundaries; teacher-forced on the GPU's tokens, every cycle's logits are
    compared and every decision is recomputed exactly from the GPU's logits."""
    log(f"stochastic cycles T={T} Td={Td}")
    gamma, cycles, ctx = 4, 10, 40
    dm, dec, om, kv = _setup(TINY, 9, 256, gamma, ctx, T=T, Td=Td)
    dec.reset(ctx, int(token_ids(1, TINY.vocab, 17)[0]))
    Ud, _ = uniform_codes(cycles * gamma, 81)
    R, _ = uniform_codes(cycles * gamma, 82)
    Uf, _ = uniform_codes(cycles, 83)
    uni = (codes_i32(Ud.reshape(cycles, gamma), cuda), codes_i32(R.reshape(cycles, gamma), cuda),
           codes_i32(Uf, cuda))
    ns = _teacher_forced_cycles(dec, om, (kv[0].copy(), kv[1].copy()), gamma, cycles, T, Td, uni)
    if T > 0:
        assert min(ns) < gamma  # rejections (and residual draws) happened


@pytest.mark.timeout(1200)
def test_full_7b_model_teacher_forced_cycle(cuda):
    """The full 28-layer Qwen2.5-7B-shaped model of the 7B workload (layers
    0-10 shared bf16, 11-27 W4 substitutes, vocab 152064, gamma 16), from 512
    positions of synthetic KV: one greedy cycle and one sharpened-draft cycle
    (T_d = 0.2), each with draft step logits, all 17 verify rows and the
    decision compared against the oracle run from host copies of the same
    weights (the oracle quantises its own substitutes).  Draft step 0 is
    compared with the oracle forward; every draft token with the oracle's draw
    from the GPU's logits.  Over 28 random-init layers the float64- and
    float32-summed oracle evaluations themselves part by a few percent, so the
    logits bound is twice that spread (at least TOL); decisions stay exact."""
    from synth.configs import CONFIGS
    wl = CONFIGS["full7b"]
    shape, gamma, ctx = wl.shape, wl.gamma, 512
    cap = 640
    log("full 7B teacher-forced: setup")
    dm, dec, om, kv = _setup(shape, 0, cap, gamma, ctx)
    kv_o = (kv[0].copy(), kv[1].copy())
    kv_o32 = (kv[0].copy(), kv[1].copy())
    dec.reset(ctx, int(token_ids(1, shape.vocab, 5)[0]))
    log("full 7B teacher-forced: greedy cycle")
    _teacher_forced_cycles(dec, om, kv_o, gamma, 1, 0.0, 0.0, draft_checked=1, kv_o32=kv_o32)
    log("full 7B teacher-forced: sharpened-draft cycle")
    dec.draft_temp = 0.2
    Ud, _ = uniform_codes(gamma, 41)
    uni = (codes_i32(Ud.reshape(1, gamma), cuda), codes_i32(np.zeros((1, gamma), np.int64), cuda),
           codes_i32([0], cuda))
    _teacher_forced_cycles(dec, om, kv_o, gamma, 1, 0.0, 0.2, uni, draft_checked=1, kv_o32=kv_o32)
