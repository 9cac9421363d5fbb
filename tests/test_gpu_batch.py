"""Batch > 1 with shared substitutes ("SubSpec" report, section 10.3, item 11):
B independent rejection rounds in one launch set, each bit-exact to the
oracle's round on its own slice, and the 4-bit skinny GEMM on the matrix
cores for up to 16 positions against the oracle's dense product on the
dequantised weights."""
import numpy as np
import pytest
import torch

from oracle.model import linear
from oracle.quant import dequantize, quantize as oq
from oracle.reject import reject as oreject
from oracle.sampling import sample as osample
from self_speculative_decoding_w4a16_amd import _lib
from synth import logits_pair, normal_tensor, uniform_codes
from tests.gpu_util import codes_i32, log, rel_err, ws
from tests.helpers import host

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
