"""Kernel-level parity: HIP path through the C ABI vs the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle.model import linear, rmsnorm, silu
from oracle.bf16 import round_bf16
from oracle.quant import quantize as oq, dequantize
from oracle.sampling import sample as osample
from oracle.reject import reject as oreject, acceptance_probabilities
from self_speculative_decoding_w4a16_amd import _lib
from synth import normal_tensor, uniform_codes, logits_pair
from tests.gpu_util import codes_i32, log, rel_err, ws
from tests.helpers import host

pytestmark = pytest.mark.gpu
TOL = 1e-2

SHAPES_7B = {"qkv": (4608, 3584), "o": (3584, 3584), "gate_up": (37888, 3584), "down": (3584, 18944)}


def _quant_gpu(w):
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=w.device)
    _lib.quantize(w, codes, meta)
    torch.cuda.synchronize()
    return codes, meta


@pytest.mark.parametrize("n,k,seed", [(512, 512, 0), (37, 192, 1), (1000, 640, 2)])
def test_quantize_bit_exact(cuda, n, k, seed):
    log(f"quantize {n}x{k}")
    w = normal_tensor((n, k), 0.02, seed, cuda)
    codes, meta = _quant_gpu(w)
    rc, rm = oq(host(w))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(meta.cpu().numpy().view(np.uint16), rm.view(np.uint16))


def test_quantize_degenerate_groups(cuda):
    w = torch.zeros((4, 128), dtype=torch.bfloat16, device=cuda)
    w[1] = 0.3
    w[2, :64] = torch.linspace(-1, 1, 64)
    w[3] = torch.tensor([70000.0, -70000.0] * 64)  # beyond fp16: saturating scale and min
    codes, meta = _quant_gpu(w)
    rc, rm = oq(host(w))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(meta.cpu().numpy().view(np.uint16), rm.view(np.uint16))


@pytest.mark.parametrize("name", list(SHAPES_7B))
def test_quantize_full_shapes_sampled_rows(cuda, name):
    n, k = SHAPES_7B[name]
    log(f"quantize full {name} {n}x{k}")
    w = normal_tensor((n, k), 0.02, 10, cuda)
    codes, meta = _quant_gpu(w)
    rows = np.unique(np.r_[0, n - 1, np.random.default_rng(0).integers(0, n, 64)])
    rc, rm = oq(host(w[rows]))
    np.testing.assert_array_equal(codes[rows].cpu().numpy(), rc)
    np.testing.assert_array_equal(meta[rows].cpu().numpy().view(np.uint16), rm.view(np.uint16))


@pytest.mark.parametrize("n,k,seed", [(512, 512, 0), (1000, 640, 1), (3, 64, 2), (4608, 3584, 3),
                                      (20000, 1024, 4), (9001, 2112, 5), (70001, 2112, 6)])
def test_w4_gemv(cuda, n, k, seed):
    log(f"w4 gemv {n}x{k}")
    w = normal_tensor((n, k), 0.02, seed, cuda)
    x = normal_tensor((k,), 1.0, seed + 100, cuda)
    codes, meta = _quant_gpu(w)
    y = torch.empty(n, dtype=torch.bfloat16, device=cuda)
    _lib.w4_gemv(codes, meta, n, k, x, y)
    torch.cuda.synchronize()
    rc, rm = oq(host(w))
    ref = linear(host(x)[None, :], dequantize(rc, rm))[0]
    assert rel_err(host(y), ref) < TOL


@pytest.mark.parametrize("name", list(SHAPES_7B))
def test_w4_gemv_full_shapes_sampled_rows(cuda, name):
    n, k = SHAPES_7B[name]
    log(f"w4 gemv full {name}")
    w = normal_tensor((n, k), 0.02, 20, cuda)
    x = normal_tensor((k,), 1.0, 21, cuda)
    codes, meta = _quant_gpu(w)
    y = torch.empty(n, dtype=torch.bfloat16, device=cuda)
    _lib.w4_gemv(codes, meta, n, k, x, y)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, n - 1, np.random.default_rng(1).integers(0, n, 256)])
    rc, rm = oq(host(w[rows]))
    ref = linear(host(x)[None, :], dequantize(rc, rm))[0]
    assert rel_err(host(y)[rows], ref) < TOL


@pytest.mark.parametrize("n,k,seed", [(512, 512, 0), (1000, 648, 1), (5, 8, 2), (152064, 3584, 3),
                                      (9001, 1032, 4), (70001, 520, 5)])
def test_bf16_gemv(cuda, n, k, seed):
    log(f"bf16 gemv {n}x{k}")
    w = normal_tensor((n, k), 0.02, seed, cuda)
    x = normal_tensor((k,), 1.0, seed + 100, cuda)
    y = torch.empty(n, dtype=torch.bfloat16, device=cuda)
    _lib.bf16_gemv(w, x, y)
    torch.cuda.synchronize()
    rows = np.arange(n) if n <= 4096 else np.unique(np.r_[0, n - 1, np.random.default_rng(2).integers(0, n, 512)])
    ref = linear(host(x)[None, :], host(w[rows]))[0]
    assert rel_err(host(y)[rows], ref) < TOL


def _fused_ref(wd, x, g, eps, epilogue, resid):
    """Oracle of the fused draft GEMV: RMSNorm prologue, then store / residual
    add / SiLU(gate)*up, composed from the oracle's forward-pass steps."""
    xn = rmsnorm(x[None, :], g, eps) if g is not None else x[None, :]
    y = linear(xn, wd)[0]
    if epilogue == 1:
        return round_bf16(resid + y)
    if epilogue == 2:
        F = wd.shape[0] // 2
        return round_bf16(silu(y[:F]) * y[F:])
    return y


@pytest.mark.parametrize("w4", [True, False])
@pytest.mark.parametrize("n,k,norm,epilogue", [(1000, 640, True, 0), (1000, 640, True, 2),
                                               (1000, 640, False, 1), (4608, 3584, True, 0),
                                               (3584, 18944, False, 1), (778, 6144, True, 2),
                                               (130, 64, True, 2)])
def test_fused_gemv(cuda, w4, n, k, norm, epilogue):
    log(f"fused gemv w4={w4} {n}x{k} norm={norm} epilogue={epilogue}")
    w = normal_tensor((n, k), 0.02, 30, cuda)
    x = normal_tensor((k,), 1.0, 31, cuda)
    g = normal_tensor((k,), 1.0, 32, cuda) if norm else None
    resid = normal_tensor((n,), 1.0, 33, cuda) if epilogue == 1 else None
    if w4:
        codes, meta = _quant_gpu(w)
        lin = _lib.linear(codes=codes, meta=meta)
        rc, rm = oq(host(w))
        wd = dequantize(rc, rm)
    else:
        lin = _lib.linear(w=w)
        wd = host(w)
    y = torch.empty(n // 2 if epilogue == 2 else n, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(lin, x, y, norm_w=g, eps=1e-6, epilogue=epilogue, resid=resid)
    torch.cuda.synchronize()
    ref = _fused_ref(wd, host(x), None if g is None else host(g), 1e-6, epilogue,
                     None if resid is None else host(resid))
    assert rel_err(host(y), ref) < TOL


@pytest.mark.parametrize("w4", [True, False])
def test_fused_gemv_gate_up_full_shape_sampled_rows(cuda, w4):
    F, k = 18944, 3584
    log(f"fused gate_up full w4={w4}")
    w = normal_tensor((2 * F, k), 0.02, 40, cuda)
    x = normal_tensor((k,), 1.0, 41, cuda)
    g = normal_tensor((k,), 1.0, 42, cuda)
    if w4:
        codes, meta = _quant_gpu(w)
        lin = _lib.linear(codes=codes, meta=meta)
    else:
        lin = _lib.linear(w=w)
    y = torch.empty(F, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(lin, x, y, norm_w=g, eps=1e-6, epilogue=2)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, F - 1, np.random.default_rng(3).integers(0, F, 256)])
    wr = host(w[np.r_[rows, F + rows]])
    if w4:
        rc, rm = oq(wr)
        wr = dequantize(rc, rm)
    ref = _fused_ref(wr, host(x), host(g), 1e-6, 2, None)
    assert rel_err(host(y)[rows], ref) < TOL


@pytest.mark.parametrize("m", [1, 5, 17, 33, 49, 64, 65, 130, 289, 512])
def test_bf16_gemm_small(cuda, m):
    n, k = 1000, 640
    log(f"gemm m={m} {n}x{k}")
    w = normal_tensor((n, k), 0.02, 7, cuda)
    x = normal_tensor((m, k), 1.0, 8, cuda)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=cuda)
    _lib.bf16_gemm(w, x, y, ws(1 << 26, cuda))
    torch.cuda.synchronize()
    ref = linear(host(x), host(w))
    assert rel_err(host(y), ref) < TOL


@pytest.mark.parametrize("name", list(SHAPES_7B) + ["lm_head"])
def test_bf16_gemm_full_shapes(cuda, name):
    n, k = SHAPES_7B.get(name, (152064, 3584))
    m = 17
    log(f"gemm full {name} m={m}")
    w = normal_tensor((n, k), 0.02, 30, cuda)
    x = normal_tensor((m, k), 1.0, 31, cuda)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=cuda)
    buf = ws(1 << 27, cuda)
    for _ in range(2):  # second call reuses the self-reset split-k counters
        y.zero_()
        _lib.bf16_gemm(w, x, y, buf)
        torch.cuda.synchronize()
        rows = np.unique(np.r_[0, n - 1, np.random.default_rng(3).integers(0, n, 256)])
        ref = linear(host(x), host(w[rows]))
        assert rel_err(host(y)[:, rows], ref) < TOL
    assert int(buf[:16384].sum().item()) == 0


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_bf16_gemm_full_shapes_many_positions(cuda, name):
    """289 positions (a k = 6, D = 48 tree's verify pass): three slices of up
    to 128 positions, sampled rows and positions against the oracle."""
    n, k = SHAPES_7B[name]
    m = 289
    log(f"gemm full {name} m={m}")
    w = normal_tensor((n, k), 0.02, 32, cuda)
    x = normal_tensor((m, k), 1.0, 33, cuda)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=cuda)
    _lib.bf16_gemm(w, x, y, ws(1 << 28, cuda))
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.unique(np.r_[0, n - 1, rng.integers(0, n, 128)])
    pos = np.unique(np.r_[0, 127, 128, 255, 256, m - 1, rng.integers(0, m, 16)])
    ref = linear(host(x)[pos], host(w[rows]))
    assert rel_err(host(y)[np.ix_(pos, rows)], ref) < TOL


@pytest.mark.parametrize("V,T", [(1000, 0.0), (1000, 1.0), (1000, 0.2), (152064, 0.2), (152064, 1.0), (7, 1.0)])
def test_sample_matches_oracle(cuda, V, T):
    log(f"sample V={V} T={T}")
    buf = ws(1 << 20, cuda)
    tok = torch.zeros(1, dtype=torch.int32, device=cuda)
    U, _ = uniform_codes(24, 40 + V)
    for s in range(6):
        z = normal_tensor((V,), 3.0, 50 + s, cuda)
        zh = host(z).astype(np.float32)
        for u in U[4 * s:4 * s + 4]:
            uc = codes_i32([u], cuda)
            _lib.sample(z, T, uc, tok, buf)
            torch.cuda.synchronize()
            assert int(tok.item()) == osample(zh, T, int(u))


REJECT_CASES = [
    (4, 1000, 1.0, 1.0), (4, 1000, 0.0, 0.0), (4, 1000, 0.6, 0.6), (4, 1000, 1.0, 0.0),
    (4, 1000, 0.0, 0.2), (16, 152064, 0.0, 0.0), (16, 152064, 1.0, 0.2), (48, 4096, 0.6, 0.6),
    (48, 152064, 0.6, 0.6), (0, 1000, 1.0, 1.0),
]


@pytest.mark.parametrize("gamma,V,T,Td", REJECT_CASES)
def test_reject_matches_oracle(cuda, gamma, V, T, Td):
    log(f"reject gamma={gamma} V={V} T={T} Td={Td}")
    zt, zd = logits_pair(gamma, V, 60 + gamma, device=cuda)
    zth, zdh = host(zt).astype(np.float32), host(zd).astype(np.float32)
    buf = ws(1 << 22, cuda)
    n_out = torch.zeros(1, dtype=torch.int32, device=cuda)
    out = torch.zeros(gamma + 1, dtype=torch.int32, device=cuda)
    st = torch.zeros(1, dtype=torch.int32, device=cuda)
    probs = torch.zeros((max(gamma, 1), 2), dtype=torch.float32, device=cuda)
    trials = 12
    Ud, _ = uniform_codes(trials * max(gamma, 1), 70)
    R, _ = uniform_codes(trials * max(gamma, 1), 71)
    Uf, _ = uniform_codes(trials, 72)
    seen_n = set()
    for t in range(trials):
        # draft tokens drawn from q with the oracle's sampler (T_d), so they are plausible
        toks = [osample(zdh[i], Td, int(Ud[t * gamma + i])) for i in range(gamma)]
        if T == 0.0 and gamma > 0:
            # greedy target: argmax prefix with a mismatch at position t % (gamma + 1)
            cut = t % (gamma + 1)
            toks = [int(np.argmax(zth[i])) for i in range(gamma)]
            if cut < gamma:
                toks[cut] = (toks[cut] + 1) % V
        elif t % 3 == 2 and gamma > 0:  # force some rejections
            toks[gamma // 2] = (toks[gamma // 2] + 1) % V
        rr = R[t * gamma:(t + 1) * gamma]
        _lib.reject(gamma, V, T, Td, zt, zd if gamma else None, codes_i32(toks, cuda) if gamma else None,
                    codes_i32(rr, cuda) if gamma else None, codes_i32([Uf[t]], cuda), n_out, out, st,
                    probs, buf)
        torch.cuda.synchronize()
        n_ref, out_ref, st_ref = oreject(zth, zdh, toks, rr, int(Uf[t]), T, Td)
        n = int(n_out.item())
        assert n == n_ref
        assert out[:n + 1].tolist() == out_ref
        assert int(st.item()) == st_ref
        seen_n.add(n)
        if gamma:
            p, q = acceptance_probabilities(zth, zdh, toks, T, Td)
            k = min(n + 1, gamma)
            got = probs[:k].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(got[:, 0], p[:k], rtol=1e-5, atol=1e-12)
            np.testing.assert_allclose(got[:, 1], q[:k], rtol=1e-5, atol=1e-12)
    if gamma and V <= 4096:
        assert len(seen_n) > 1
    assert int(buf[:65536].sum().item()) == 0


@pytest.mark.parametrize("nbytes", [16, 16 * 1001, 3 * (1 << 20) + 16 * 37, 64 << 20])
def test_hbm_read_fold(cuda, nbytes):
    """The read-ceiling kernel reads every word once: its XOR fold equals the
    XOR of all 32-bit words (ragged tails and a buffer of one word included),
    and it accumulates into the sink."""
    log(f"hbm read {nbytes} B")
    g = torch.Generator(device=cuda)
    g.manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=cuda, generator=g)
    words = buf.cpu().numpy().view(np.uint32)
    want = int(np.bitwise_xor.reduce(words))
    sink = torch.zeros(1, dtype=torch.int32, device=cuda)
    _lib.hbm_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
    _lib.hbm_read(buf, sink)  # a second fold cancels the first
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == 0
