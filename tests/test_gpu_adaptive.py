"""The entropy-adaptive draft length ("The second ledger of speculative
decoding", section 3.3) on the GPU against oracle/adaptive.py: the entropy of
each draft token's logits, the controller's stop decisions and its EMA
centres (bit-exact when the oracle controller is fed the GPU's float32
entropies), the rejection round over a draft stopped early, teacher-forced
cycles, and greedy decoding that stays lossless while the length adapts."""
import numpy as np
import pytest
import torch

from oracle.adaptive import Controller, entropy
from oracle.model import forward
from oracle.reject import reject as oreject
from oracle.sampling import sample as osample
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import kv_history, logits_pair, model_weights, normal_tensor, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.gpu_util import codes_i32, log, rel_err, ws
from tests.helpers import host, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2
TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, vocab=1000, n_shared=1)


def _state(ctl):
    """The GPU controller state as the oracle's fields."""
    st = ctl.cpu().numpy()
    return float(st[0]), float(st[1]), bool(st[2]), bool(st[3]), float(st[4]), float(st[5])


@pytest.mark.parametrize("V", [1000, 152064])
def test_entropy_and_stop_decisions(cuda, V):
    """Crafted draft rows of rising temperature; the controller starts from
    given centres; every step's entropy is compared with the oracle's, and
    the stop step and the running state with the oracle controller fed the
    GPU's entropies."""
    log(f"adaptive controller V={V}")
    gmax = 12
    shape = TINY.with_(vocab=V)
    w = model_weights(shape, 3, cuda)
    dm = DeviceModel(shape, w)
    for trial, (acc, rej, c) in enumerate([(0.5, 4.0, 0.3), (1.0, 1.2, 0.05), (3.0, 0.2, 0.6), (2.0, 2.0, 0.2)]):
        dec = SpecDecoder(dm, 64, gmax, adaptive=dict(c=c, beta=0.125))
        dec.ctl_state[:4] = torch.tensor([acc, rej, 1.0, 1.0], dtype=torch.float64)
        scale = np.linspace(0.2, 4.0, gmax) if trial % 2 == 0 else np.linspace(4.0, 0.2, gmax)
        for i in range(gmax):
            z = normal_tensor((V,), float(scale[i]), 100 * trial + i, cuda)
            if i == 3:
                z[5] = float("nan")  # a non-finite logit carries no probability
            dec.draft_logits[i].copy_(z)
        ref = Controller(gmax, c)
        ref.h_acc, ref.h_rej, ref.seen_acc, ref.seen_rej = acc, rej, True, True
        go = True
        for i in range(gmax):
            _lib.draft_control(dm.c, dec.c, i, dec.ctl, dec.ws)
            torch.cuda.synchronize()
            h_gpu = float(dec.entropy[i].item()) if go else None
            if go:
                h_ref = entropy(host(dec.draft_logits[i]).astype(np.float64))
                assert abs(h_gpu - h_ref) <= 1e-5 * max(1.0, h_ref), (trial, i, h_gpu, h_ref)
                go = ref.after_token(np.float32(h_gpu))
            assert int(dec.draft_len.item()) == ref.gamma_eff, (trial, i)
            st = _state(dec.ctl_state)
            assert st[4] == ref.P and st[5] == ref.A, (trial, i)
        # the rejection round's outcome updates the centres
        for n in (0, min(2, ref.gamma_eff), ref.gamma_eff):
            d2 = dict(zip(("h_acc", "h_rej", "seen_acc", "seen_rej"), _state(dec.ctl_state)[:4]))
            ctl2 = Controller(gmax, c)
            ctl2.__dict__.update(d2)
            ctl2.H = [float(dec.entropy[i].item()) for i in range(ref.gamma_eff)]
            ctl2.gamma_eff = ref.gamma_eff
            saved = dec.ctl_state.clone(), dec.draft_len.clone()
            dec.n_accepted.fill_(n)
            _lib.control_update(dec.ctl, dec.n_accepted)
            torch.cuda.synchronize()
            ctl2.after_round(n)
            st = _state(dec.ctl_state)
            assert st[:4] == (ctl2.h_acc, ctl2.h_rej, ctl2.seen_acc, ctl2.seen_rej), (trial, n)
            assert int(dec.draft_len.item()) == gmax and st[4] == 1.0 and st[5] == 1.0
            assert int(dec.ctl_state[6].item()) == ref.gamma_eff
            dec.ctl_state.copy_(saved[0])
            dec.draft_len.copy_(saved[1])


@pytest.mark.parametrize("T,Td", [(0.0, 0.0), (1.0, 1.0), (0.6, 0.0), (1.0, 0.2)])
def test_reject_over_a_shortened_draft(cuda, T, Td):
    log(f"reject_len T={T} Td={Td}")
    gamma, V = 8, 3000
    zt, zd = logits_pair(gamma, V, 31, target_std=1.0, draft_noise=0.3, device=cuda)
    zth, zdh = host(zt).astype(np.float32), host(zd).astype(np.float32)
    buf = ws(1 << 22, cuda)
    n_out = torch.zeros(1, dtype=torch.int32, device=cuda)
    out = torch.zeros(gamma + 1, dtype=torch.int32, device=cuda)
    st = torch.zeros(1, dtype=torch.int32, device=cuda)
    Ud, _ = uniform_codes(gamma, 32)
    R, _ = uniform_codes(gamma, 33)
    toks = [osample(zdh[i], Td, int(Ud[i])) for i in range(gamma)]
    if T == 0:
        toks = [int(np.argmax(zth[i])) for i in range(gamma)]
    for g in range(0, gamma + 1):
        for uf in (5, 9999999):
            glen = torch.tensor([g], dtype=torch.int32, device=cuda)
            t2 = toks[:g] + [-1] * (gamma - g)  # steps past the draft length carry token -1
            _lib.reject_len(gamma, V, T, Td, zt, zd, codes_i32(t2, cuda), codes_i32(R, cuda), codes_i32([uf], cuda),
                            glen, n_out, out, st, None, buf)
            torch.cuda.synchronize()
            n = int(n_out.item())
            ref = oreject(zth[:g + 1], zdh[:g], toks[:g], R[:g], uf, T, Td)
            assert (n, out[:n + 1].tolist(), int(st.item())) == ref, (g, uf)


def _adaptive_setup(seed, T, Td, c, graphs=False):
    gmax, cap, ctx = 8, 256, 40
    w = model_weights(TINY, seed, "cuda")
    dm = DeviceModel(TINY, w)
    dec = SpecDecoder(dm, cap, gmax, T, Td, adaptive=dict(c=c, beta=0.125), graphs=graphs)
    K, V = kv_history(TINY.n_layers, TINY.n_kv_heads, ctx, TINY.head_dim, cap, seed + 1, "cuda")
    dec.load_kv(K, V, ctx, int(token_ids(1, TINY.vocab, seed + 2)[0]))
    om = oracle_model(TINY, w, dm.substitute_layers)
    kv_o = (host(K).astype(np.float64), host(V).astype(np.float64))
    return dm, dec, om, kv_o, gmax


@pytest.mark.parametrize("T,Td,c,graphs", [(0.0, 0.0, 0.3, False), (1.0, 1.0, 0.2, False), (0.0, 0.2, 0.5, False),
                                            (1.0, 1.0, 0.2, True), (0.0, 0.0, 0.3, True)])
def test_adaptive_cycles_teacher_forced(cuda, T, Td, c, graphs):
    """Cycles with the device controller, the oracle teacher-forced on the
    GPU's tokens and entropies: the same draft length every cycle, drafted
    logits within TOL, the decision bit-exact from the GPU's logits, and the
    centres equal after every round.  With graphs the draft runs as replayed
    segments that stop at the controller's draft length."""
    log(f"adaptive cycles T={T} Td={Td} c={c} graphs={graphs}")
    dm, dec, om, kv_o, gmax = _adaptive_setup(41, T, Td, c, graphs)
    cycles = 10
    Ud, _ = uniform_codes(cycles * gmax, 42)
    R, _ = uniform_codes(cycles * gmax, 43)
    Uf, _ = uniform_codes(cycles, 44)
    Ud, R = Ud.reshape(cycles, gmax), R.reshape(cycles, gmax)
    uni = (codes_i32(Ud, cuda), codes_i32(R, cuda), codes_i32(Uf, cuda))
    ctl = Controller(gmax, c, 0.125)
    lengths = []
    for cy in range(cycles):
        kv_len = int(dec.kv_len.item())
        last = int(dec.tokens[0].item())
        dec.cycle(uni[0][cy], uni[1][cy], uni[2][cy:cy + 1])
        torch.cuda.synchronize()
        g = dec.last_draft_len()
        hs = host(dec.entropy[:g]).astype(np.float32)
        toks = [last] + host(dec.tokens[1:g + 1]).astype(np.int64).tolist()
        dz = host(dec.draft_logits[:g]).astype(np.float32)
        tz = host(dec.target_logits[:g + 1]).astype(np.float32)
        for i in range(g):
            ref = forward(om, kv_o, kv_len + i, [toks[i]], draft=True)[0]
            assert rel_err(dz[i], ref) < TOL, (cy, i)
            h_ref = entropy(dz[i].astype(np.float64))
            assert abs(float(hs[i]) - h_ref) <= 1e-5 * max(1.0, h_ref)
            assert osample(dz[i], Td, int(Ud[cy][i])) == toks[i + 1]
            go = ctl.after_token(hs[i])
            assert go == (i + 1 < g), (cy, i)
        assert ctl.gamma_eff == g
        ref_t = forward(om, kv_o, kv_len, toks)
        for j in range(g + 1):
            assert rel_err(tz[j], ref_t[j]) < TOL
        n = int(dec.n_accepted.item())
        out = host(dec.out_tokens[:n + 1]).astype(np.int64).tolist()
        assert (n, out, int(dec.status.item())) == oreject(tz, dz, toks[1:], R[cy][:g], int(Uf[cy]), T, Td)
        ctl.after_round(n)
        st = _state(dec.ctl_state)
        assert st[:4] == (ctl.h_acc, ctl.h_rej, ctl.seen_acc, ctl.seen_rej), cy
        assert int(dec.kv_len.item()) == kv_len + n + 1
        lengths.append(g)
    assert len(set(lengths)) > 1  # the length adapts


def test_greedy_adaptive_generation_is_lossless(cuda):
    from oracle.cycle import autoregressive_generate
    log("adaptive greedy generation")
    w = model_weights(TINY, 51, cuda)
    dm = DeviceModel(TINY, w)
    dec = SpecDecoder(dm, 256, 8, adaptive=dict(c=0.3, beta=0.125), graphs=True)
    prompt = [int(t) for t in token_ids(7, TINY.vocab, 52)]
    G = 40
    lengths = []
    got, ns = dec.generate(prompt, G, on_cycle=lambda c, n: lengths.append(dec.last_draft_len()))
    om = oracle_model(TINY, w, dm.substitute_layers)
    ref = autoregressive_generate(om, prompt, G, 0.0, np.zeros(G, np.int64), 256)
    assert got == ref
    assert all(1 <= g <= 8 for g in lengths) and all(n <= g for n, g in zip(ns, lengths))
