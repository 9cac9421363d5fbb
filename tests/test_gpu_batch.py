"""Batch > 1 with shared substitutes ("SubSpec" report, section 10.3, item 11):
B independent rejection rounds in one launch set, each bit-exact to the
oracle's round on its own slice, and the 4-bit skinny GEMM on the matrix
cores for up to 16 positions against the oracle's dense product on the
dequantised weights."""
import numpy as np
import pytest
import torch

from oracle.cycle import autoregressive_generate
from oracle.model import forward, linear
from oracle.quant import dequantize, quantize as oq
from oracle.reject import reject as oreject
from oracle.sampling import sample as osample
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import BatchDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import kv_history, logits_pair, model_weights, normal_tensor, token_ids, uniform_codes
from synth.configs import QWEN7B
from tests.gpu_util import codes_i32, log, rel_err, ws
from tests.helpers import host, memo_weights, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.mark.parametrize("B,gamma,V,T,Td", [(1, 4, 1000, 1.0, 1.0), (3, 4, 1000, 0.0, 0.0), (8, 6, 5000, 1.0, 0.2),
                                            (5, 16, 152064, 0.6, 0.6), (4, 0, 1000, 1.0, 1.0)])
def test_reject_batch_matches_oracle_per_round(cuda, B, gamma, V, T, Td):
    log(f"reject batch B={B} gamma={gamma} V={V} T={T} Td={Td}")
    zts, zds, toks, Rs, Us, glen = [], [], [], [], [], []
    for b in range(B):
        zt, zd = logits_pair(gamma, V, 200 + b, target_std=1.0, draft_noise=0.5)
        zth, zdh = host(zt).astype(np.float32), host(zd).astype(np.float32)
        Ud, _ = uniform_codes(max(gamma, 1), 300 + b)
        R, _ = uniform_codes(max(gamma, 1), 400 + b)
        t = [osample(zdh[i], Td, int(Ud[i])) for i in range(gamma)]
        if T == 0 and gamma:
            t = [int(np.argmax(zth[i])) for i in range(gamma)]
            t[b % gamma] = (t[b % gamma] + 1) % V  # a rejection at a different place per round
        zts.append(zth)
        zds.append(zdh if gamma else np.zeros((0, V), np.float32))
        toks.append(t)
        Rs.append(list(R[:gamma]))
        Us.append(int(uniform_codes(1, 500 + b)[0][0]))
        glen.append(gamma - (b % 3) if gamma else 0)  # some drafts stopped early
    dev = lambda a: torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).to(cuda)
    zt_d = dev(np.stack(zts))
    zd_d = dev(np.stack(zds)) if gamma else torch.zeros(1, dtype=torch.bfloat16, device=cuda)
    tk = codes_i32(np.array(toks).reshape(-1) if gamma else [0], cuda)
    rc = codes_i32(np.array(Rs).reshape(-1) if gamma else [0], cuda)
    uc = codes_i32(Us, cuda)
    gl = codes_i32(glen, cuda)
    n_out = torch.full((B,), -7, dtype=torch.int32, device=cuda)
    out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=cuda)
    st = torch.full((B,), -7, dtype=torch.int32, device=cuda)
    probs = torch.zeros((B, max(gamma, 1), 2), dtype=torch.float32, device=cuda)
    buf = ws(_lib.reject_workspace_bytes(B, gamma, V), cuda)
    for use_len in (False, True):
        _lib.reject_batch(B, gamma, V, T, Td, zt_d, zd_d, tk, rc, uc, gl if use_len else None, n_out, out, st,
                          probs, buf)
        torch.cuda.synchronize()
        for b in range(B):
            g = glen[b] if use_len else gamma
            ref = oreject(zts[b][:g + 1], zds[b][:g], toks[b][:g], Rs[b][:g], Us[b], T, Td)
            n = int(n_out[b].item())
            assert (n, out[b, :n + 1].tolist(), int(st[b].item())) == ref, (use_len, b)
    assert int(buf[:65536].sum().item()) == 0  # arrival counters left at zero


def _w4(w):
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=w.device)
    _lib.quantize(w, codes, meta)
    return codes, meta


@pytest.mark.parametrize("n,k", [(512, 512), (1000, 640), (4608, 3584), (3584, 18944), (130, 128)])
@pytest.mark.parametrize("m", [1, 2, 5, 16])
def test_w4_gemm_matches_oracle(cuda, n, k, m):
    log(f"w4 gemm {n}x{k} m={m}")
    w = normal_tensor((n, k), 0.02, 60 + n, cuda)
    x = normal_tensor((m, k), 1.0, 61 + m, cuda)
    codes, meta = _w4(w)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=cuda)
    buf = ws(_lib.w4_gemm_workspace_bytes(n, k, m), cuda)
    _lib.w4_gemm(_lib.linear(codes=codes, meta=meta), x, y, buf)
    torch.cuda.synchronize()
    rows = np.arange(n) if n <= 4608 else np.unique(np.r_[0, n - 1, np.random.default_rng(0).integers(0, n, 512)])
    rc, rm = oq(host(w[rows]))
    ref = linear(host(x), dequantize(rc, rm))
    got = host(y)[:, rows]
    for t in range(m):
        assert rel_err(got[t], ref[t]) < TOL, t


def test_w4_gemm_gate_up_shape_sampled(cuda):
    n, k, m = 37888, 3584, 8
    log("w4 gemm gate/up shape")
    w = normal_tensor((n, k), 0.02, 70, cuda)
    x = normal_tensor((m, k), 1.0, 71, cuda)
    codes, meta = _w4(w)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=cuda)
    _lib.w4_gemm(_lib.linear(codes=codes, meta=meta), x, y, ws(_lib.w4_gemm_workspace_bytes(n, k, m), cuda))
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, n - 1, np.random.default_rng(1).integers(0, n, 512)])
    rc, rm = oq(host(w[rows]))
    ref = linear(host(x), dequantize(rc, rm))
    for t in range(m):
        assert rel_err(host(y)[t, rows], ref[t]) < TOL


# ---------------------------------------------------------------- batched decoding

TINY = QWEN7B.with_(n_layers=3, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                    vocab=1000, n_shared=1)


def _batch_setup(shape, seed, B, cap, gamma, ctxs, T=0.0, Td=0.0, device="cuda"):
    """A batch decoder whose sequence b starts from its own synthetic KV
    history of ctxs[b] positions; the oracle gets one cache per sequence."""
    w = model_weights(shape, seed, device)
    dm = DeviceModel(shape, w)
    dec = BatchDecoder(dm, B, cap, gamma, T, Td)
    om = memo_weights(oracle_model(shape, w, dm.substitute_layers))
    kvs = []
    for b in range(B):
        K, V = kv_history(shape.n_layers, shape.n_kv_heads, ctxs[b], shape.head_dim, cap, seed + 11 + b, device)
        dec.k_cache[:, b].copy_(K)
        dec.v_cache[:, b].copy_(V)
        kvs.append((host(K).astype(np.float64), host(V).astype(np.float64)))
    return dm, dec, om, kvs


@pytest.mark.parametrize("shape_name,B,gamma,T,Td", [("tiny", 1, 4, 1.0, 1.0), ("tiny", 3, 4, 0.0, 0.0), ("tiny", 4, 3, 1.0, 1.0),
                                                     ("tiny", 2, 5, 0.6, 0.0), ("tiny", 5, 4, 0.0, 0.5),
                                                     ("layer7b", 8, 4, 0.0, 0.0), ("layer7b", 16, 16, 1.0, 0.2)])
def test_batch_cycles_teacher_forced(cuda, shape_name, B, gamma, T, Td):
    """Every sequence of a batched cycle against the oracle run on that
    sequence alone, teacher-forced on the GPU's tokens: draft and verify
    logits within 1e-2, every draft token the oracle's draw from the GPU's
    own draft logits, each round recomputed bit-exact, each kv_len moved by
    its own n + 1.  The sequences start at different lengths."""
    log(f"batch cycles {shape_name} B={B} gamma={gamma} T={T} Td={Td}")
    shape = TINY if shape_name == "tiny" else QWEN7B.with_(n_layers=1, n_shared=0)
    base = 40 if shape_name == "tiny" else 600
    ctxs = [base + 3 * b for b in range(B)]
    cap = max(ctxs) + 4 * (gamma + 1) + 16
    cycles = 3 if shape_name == "tiny" else 1
    dm, dec, om, kvs = _batch_setup(shape, 5, B, cap, gamma, ctxs, T, Td)
    last = [int(t) for t in token_ids(B, shape.vocab, 19)]
    dec.reset(torch.tensor(ctxs, dtype=torch.int32), last)
    stoch = T > 0 or Td > 0
    for c in range(cycles):
        lens = dec.kv_len.tolist()
        if stoch:
            Ud, _ = uniform_codes(B * gamma, 600 + c)
            R, _ = uniform_codes(B * gamma, 700 + c)
            U, _ = uniform_codes(B, 800 + c)
            Ud, R = Ud.reshape(B, gamma), R.reshape(B, gamma)
            dec.cycle(codes_i32(Ud, cuda), codes_i32(R, cuda), codes_i32(U, cuda))
        else:
            Ud = np.zeros((B, gamma), np.int64)
            R = np.zeros((B, gamma), np.int64)
            U = np.zeros(B, np.int64)
            dec.cycle()
        torch.cuda.synchronize()
        dz = host(dec.draft_logits).astype(np.float32)
        tz = host(dec.target_logits).astype(np.float32)
        n_all = dec.n_accepted.tolist()
        out_all = dec.out_tokens.tolist()
        st_all = dec.status.tolist()
        drafted = dec.tokens[:, 1:].tolist()  # the rollback rewrites only tokens[b][0]
        for b in range(B):
            kv_len = lens[b]
            toks = [None] * (gamma + 1)
            toks[0] = int(last[b])
            for i in range(gamma):
                ref = forward(om, kvs[b], kv_len + i, [toks[i]], draft=True)[0]
                assert rel_err(dz[b, i], ref) < TOL, (b, i)
                toks[i + 1] = osample(dz[b, i], Td, int(Ud[b, i]))
                assert toks[i + 1] == drafted[b][i], (b, i)
            ref_t = forward(om, kvs[b], kv_len, toks)
            for j in range(gamma + 1):
                assert rel_err(tz[b, j], ref_t[j]) < TOL, (b, j)
            n = n_all[b]
            assert (n, out_all[b][:n + 1], st_all[b]) == oreject(tz[b], dz[b], toks[1:], list(R[b]), int(U[b]), T, Td)
            last[b] = out_all[b][n]
        assert dec.kv_len.tolist() == [lens[b] + n_all[b] + 1 for b in range(B)]
        assert dec.tokens[:, 0].tolist() == last


def test_batch_greedy_generation_matches_oracle(cuda):
    """Four prompts decoded together, greedy: each sequence's tokens equal
    greedy autoregressive decoding of its prompt alone (the oracle)."""
    log("batch greedy generation")
    B, gamma, G = 4, 4, 16
    w = model_weights(TINY, 8, cuda)
    dm = DeviceModel(TINY, w)
    dec = BatchDecoder(dm, B, 128, gamma)
    om = oracle_model(TINY, w, dm.substitute_layers)
    prompts = [[int(t) for t in token_ids(9, TINY.vocab, 30 + b)] for b in range(B)]
    got, ns = dec.generate(prompts, G)
    for b in range(B):
        assert got[b] == autoregressive_generate(om, prompts[b], G, 0.0, np.zeros(G, np.int64), 128), b


def test_batch_ar_step_matches_oracle(cuda):
    """Plain batched autoregressive decoding on the full-precision model (no
    substitutes) equals the oracle's greedy decoding of every prompt."""
    log("batch AR")
    B, G = 3, 6
    w = model_weights(TINY, 12, cuda)
    full = DeviceModel(TINY, w, substitute_layers=[])
    dec = BatchDecoder(full, B, 64, 1)
    om = oracle_model(TINY, w, [])
    prompts = [[int(t) for t in token_ids(7, TINY.vocab, 50 + b)] for b in range(B)]
    dec.prefill(prompts)
    outs = [[] for _ in range(B)]
    for _ in range(G):
        dec.ar_step()
        for b, t in enumerate(dec.tokens[:, 0].tolist()):
            outs[b].append(t)
    for b in range(B):
        assert outs[b] == autoregressive_generate(om, prompts[b], G, 0.0, np.zeros(G, np.int64), 64), b
    assert dec.kv_len.tolist() == [6 + G] * B


def test_batch_step_past_capacity_is_skipped(cuda):
    """A sequence whose draft position is past its capacity gets token -1 and
    writes nothing; the others draft normally."""
    log("batch past capacity")
    B, gamma, cap = 2, 3, 64
    dm, dec, om, kvs = _batch_setup(TINY, 7, B, cap, gamma, [cap - 2, 20])
    dec.reset(torch.tensor([cap - 2, 20], dtype=torch.int32), [5, 9])
    before = dec.k_cache.clone()
    dec.draft()
    torch.cuda.synchronize()
    t = dec.tokens.tolist()
    assert t[0][1] >= 0 and t[0][2] >= 0 and t[0][3] == -1  # positions cap-2, cap-1, then cap
    assert all(x >= 0 for x in t[1][1:])
    assert torch.equal(dec.k_cache[:, 0, :, :cap - 2], before[:, 0, :, :cap - 2])
