"""2- and 3-bit substitutes on the GPU against the oracle: codes and scales
bit-exact (every layout), the fused draft GEMV at each epilogue within the
logits tolerance, a draft step of a model whose substitutes mix 4, 3 and 2
bits, and greedy speculative decoding with a 2-bit draft, which must still
emit exactly the target's greedy tokens."""
import numpy as np
import pytest
import torch

from oracle.bf16 import round_bf16
from oracle.cycle import autoregressive_generate, speculative_generate
from oracle.model import forward, linear, rmsnorm, silu
from oracle.quant import dequantize, quantize as oq, row_bytes
from self_speculative_decoding_w4a16_amd import _lib
from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
from self_speculative_decoding_w4a16_amd.model import DeviceModel
from synth import kv_history, model_weights, normal_tensor, token_ids
from synth.configs import QWEN7B
from tests.gpu_util import log, rel_err
from tests.helpers import host, oracle_model

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _quant(w, bits):
    n, k = w.shape
    codes = torch.empty((n, row_bytes(k, bits)), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=w.device)
    _lib.quantize(w, codes, meta, bits=bits)
    torch.cuda.synchronize()
    return codes, meta


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n,k,std", [(512, 512, 0.02), (37, 256, 0.02), (300, 1024, 1e-6),
                                     (1000, 640, 3.0), (4608, 3584, 0.02)])
def test_quantize_low_bits_bit_exact(cuda, bits, n, k, std):
    if bits == 3 and k % 128:
        pytest.skip("3-bit rows need k % 128 == 0")
    log(f"quantize {bits}-bit {n}x{k} std={std}")
    w = normal_tensor((n, k), std, 50 + n, cuda)
    codes, meta = _quant(w, bits)
    rows = np.arange(n) if n <= 1024 else np.unique(np.r_[0, n - 1, np.random.default_rng(0).integers(0, n, 128)])
    rc, rm = oq(host(w[rows]), bits=bits)
    np.testing.assert_array_equal(codes[rows].cpu().numpy(), rc)
    np.testing.assert_array_equal(meta[rows].cpu().numpy().view(np.uint16), rm.view(np.uint16))


def _fused_ref(wd, x, g, eps, epilogue, resid):
    xn = rmsnorm(x[None, :], g, eps) if g is not None else x[None, :]
    y = linear(xn, wd)[0]
    if epilogue == 1:
        return round_bf16(resid + y)
    if epilogue == 2:
        F = wd.shape[0] // 2
        return round_bf16(silu(y[:F]) * y[F:])
    return y


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n,k,norm,epilogue", [(1000, 640, True, 0), (1000, 640, True, 2), (1000, 640, False, 1),
                                               (4608, 3584, True, 0), (3584, 3584, False, 1),
                                               (3584, 18944, False, 1), (778, 6144, True, 2),
                                               (130, 128, True, 2), (3, 128, False, 0), (20000, 1024, False, 0)])
def test_fused_gemv_low_bits(cuda, bits, n, k, norm, epilogue):
    if bits == 3 and k % 128:
        pytest.skip("3-bit rows need k % 128 == 0")
    log(f"fused gemv {bits}-bit {n}x{k} norm={norm} epilogue={epilogue}")
    w = normal_tensor((n, k), 0.02, 60, cuda)
    x = normal_tensor((k,), 1.0, 61, cuda)
    g = normal_tensor((k,), 1.0, 62, cuda) if norm else None
    resid = normal_tensor((n,), 1.0, 63, cuda) if epilogue == 1 else None
    codes, meta = _quant(w, bits)
    lin = _lib.linear(codes=codes, meta=meta, bits=bits)
    y = torch.empty(n // 2 if epilogue == 2 else n, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(lin, x, y, norm_w=g, eps=1e-6, epilogue=epilogue, resid=resid)
    torch.cuda.synchronize()
    rc, rm = oq(host(w), bits=bits)
    ref = _fused_ref(dequantize(rc, rm, bits=bits), host(x), None if g is None else host(g), 1e-6, epilogue,
                     None if resid is None else host(resid))
    assert rel_err(host(y), ref) < TOL


@pytest.mark.parametrize("bits", [2, 3])
def test_fused_gemv_low_bits_gate_up_full_shape(cuda, bits):
    F, k = 18944, 3584
    log(f"fused gate_up full {bits}-bit")
    w = normal_tensor((2 * F, k), 0.02, 70, cuda)
    x = normal_tensor((k,), 1.0, 71, cuda)
    g = normal_tensor((k,), 1.0, 72, cuda)
    codes, meta = _quant(w, bits)
    y = torch.empty(F, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(_lib.linear(codes=codes, meta=meta, bits=bits), x, y, norm_w=g, eps=1e-6, epilogue=2)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, F - 1, np.random.default_rng(4).integers(0, F, 256)])
    rc, rm = oq(host(w[np.r_[rows, F + rows]]), bits=bits)
    ref = _fused_ref(dequantize(rc, rm, bits=bits), host(x), host(g), 1e-6, 2, None)
    assert rel_err(host(y)[rows], ref) < TOL


TINY = QWEN7B.with_(n_layers=4, hidden=256, ffn=512, n_q_heads=4, n_kv_heads=2, head_dim=128, vocab=1000,
                    n_shared=1)


def test_draft_step_mixed_widths_matches_oracle(cuda):
    """Layers 1, 2, 3 substituted at 4, 3 and 2 bits (layer 0 shared): one
    draft step against the oracle forward of the same substitutes."""
    log("draft step with 4/3/2-bit substitutes")
    widths = {1: 4, 2: 3, 3: 2}
    w = model_weights(TINY, 17, cuda)
    dm = DeviceModel(TINY, w, bits=widths)
    cap, kv_len = 256, 100
    dec = SpecDecoder(dm, cap, 4)
    K, V = kv_history(TINY.n_layers, TINY.n_kv_heads, kv_len, TINY.head_dim, cap, 18, cuda)
    dec.load_kv(K, V, kv_len, int(token_ids(1, TINY.vocab, 19)[0]))
    om = oracle_model(TINY, w, [])
    om.make_substitutes([1, 2, 3], bits=[4, 3, 2])
    _lib.draft_step(dm.c, dec.c, 0, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    ref = forward(om, kv, kv_len, [int(dec.tokens[0].item())], draft=True)[0]
    assert rel_err(host(dec.draft_logits[0]), ref) < TOL


@pytest.mark.parametrize("bits", [2, 3])
def test_greedy_generation_low_bit_draft_is_lossless(cuda, bits):
    """A 2- or 3-bit draft drafts worse, but greedy verification still emits
    exactly the target's greedy tokens (and the oracle's cycle by cycle)."""
    log(f"greedy generation, {bits}-bit draft")
    w = model_weights(TINY, 23, cuda)
    dm = DeviceModel(TINY, w, bits=bits)
    dec = SpecDecoder(dm, 256, 4)
    prompt = [int(t) for t in token_ids(9, TINY.vocab, 24)]
    G = 20
    got, ns = dec.generate(prompt, G)
    om = oracle_model(TINY, w, [])
    om.make_substitutes(dm.substitute_layers, bits=bits)
    z = np.zeros((64, 4), np.int64)
    ref_sd, ref_ns = speculative_generate(om, prompt, G, 4, 0.0, 0.0, (z, z, np.zeros(64, np.int64)), 256)
    ref_ar = autoregressive_generate(om, prompt, G, 0.0, np.zeros(G, np.int64), 256)
    assert ref_sd == ref_ar
    assert got == ref_sd
    assert ns == ref_ns[:len(ns)]
