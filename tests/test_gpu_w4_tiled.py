"""Low-bit substitutes in 16-row tiles: the repack is the permutation the
header states (bit-exact, 4 and 2 bits), the matrix-core GEMV on tiles
matches the oracle (RMSNorm prologue, store / residual / SiLU * up
epilogues, short and long k, ragged last units, waves past the chunks, both
widths), and the skinny GEMM reads 4-bit tiles and rows to the same bits."""
import numpy as np
import pytest
import torch

from oracle.bf16 import round_bf16
from oracle.model import linear, rmsnorm, silu
from oracle.quant import dequantize, quantize as oq
from self_speculative_decoding_w4a16_amd import _lib
from synth import normal_tensor
from tests.gpu_util import log, rel_err
from tests.helpers import host

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _quant(w, bits=4):
    n, k = w.shape
    codes = torch.empty((n, k * bits // 8), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=w.device)
    _lib.quantize(w, codes, meta, bits=bits)
    tc, tm = torch.empty_like(codes), torch.empty_like(meta)
    _lib.tile_codes(codes, meta, tc, tm, bits=bits)
    torch.cuda.synchronize()
    return codes, meta, tc, tm


def _tile_ref(codes, meta, bits=4):
    """The tiled layout written out from its statement in include/subspec.h:
    with e = 8 / bits groups a 64-byte chunk, KiB (t, c) holds, at
    16 (16 g + r), bytes 64 c + 16 g .. + 15 of row 16 t + r; meta dword
    16 e (t c_n + c) + e r + f is row 16 t + r's dword e c + f."""
    n, rb = codes.shape
    cn, e = rb // 64, 8 // bits
    tc = np.empty(n * rb, np.uint8)
    md = meta.view(np.uint32).reshape(n, -1)
    tm = np.empty(md.size, np.uint32)
    for t in range(n // 16):
        for c in range(cn):
            b = t * cn + c
            for g in range(4):
                for r in range(16):
                    tc[1024 * b + 16 * (16 * g + r):1024 * b + 16 * (16 * g + r) + 16] = \
                        codes[16 * t + r, 64 * c + 16 * g:64 * c + 16 * g + 16]
            for r in range(16):
                for f in range(e):
                    tm[16 * e * b + e * r + f] = md[16 * t + r, e * c + f]
    return tc, tm


@pytest.mark.parametrize("n,k,bits", [(16, 128, 4), (48, 384, 4), (160, 1024, 4), (16, 256, 2), (48, 768, 2),
                                      (160, 1024, 2)])
def test_tile_layout_bit_exact(cuda, n, k, bits):
    log(f"tile {n}x{k} bits={bits}")
    w = normal_tensor((n, k), 0.02, 3, cuda)
    codes, meta, tc, tm = _quant(w, bits)
    rc, rm = _tile_ref(codes.cpu().numpy(), meta.cpu().numpy().view(np.uint16), bits)
    np.testing.assert_array_equal(tc.cpu().numpy().reshape(-1), rc)
    np.testing.assert_array_equal(tm.cpu().numpy().view(np.uint32).reshape(-1), rm)


def test_tile_full_shape_sampled_tiles(cuda):
    n, k = 37888, 3584
    log("w4 tile full gate_up")
    w = normal_tensor((n, k), 0.02, 4, cuda)
    codes, meta, tc, tm = _quant(w)
    cn = k // 128
    for t in (0, 1, 1183, 2367):
        rc, rm = _tile_ref(codes[16 * t:16 * t + 16].cpu().numpy(), meta[16 * t:16 * t + 16].cpu().numpy().view(np.uint16))
        got_c = tc.view(-1)[1024 * cn * t:1024 * cn * (t + 1)].cpu().numpy()
        got_m = tm.view(-1).view(torch.int32)[32 * cn * t:32 * cn * (t + 1)].cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got_c, rc)
        np.testing.assert_array_equal(got_m, rm)


def _fused_ref(wd, x, g, eps, epilogue, resid):
    xn = rmsnorm(x[None, :], g, eps) if g is not None else x[None, :]
    y = linear(xn, wd)[0]
    if epilogue == 1:
        return round_bf16(resid + y)
    if epilogue == 2:
        F = wd.shape[0] // 2
        return round_bf16(silu(y[:F]) * y[F:])
    return y


# (n, k, norm, epilogue): 7B sites, k of 2 and 5 chunks (waves past the
# chunks), a ragged last unit of two tiles (n % 32 == 16), every x-item count
# of the prologue (k up to 28672)
CASES = [(512, 512, True, 0), (512, 256, True, 2), (1024, 640, False, 1), (80, 1024, False, 0),
         (4608, 3584, True, 0), (3584, 3584, False, 1), (3584, 18944, False, 1), (1024, 5120, True, 2),
         (512, 14336, False, 1), (272, 28672, False, 1), (96, 12288, False, 0), (64, 6144, True, 2)]


# 2 bits: chunks of 256 k (k = 256 is one chunk: waves past the chunks)
CASES_2 = [(512, 256, True, 0), (512, 512, True, 2), (1024, 1280, False, 1), (80, 1024, False, 0),
           (4608, 3584, True, 0), (3584, 18944, False, 1), (1024, 5120, True, 2), (272, 28672, False, 1)]


@pytest.mark.parametrize("n,k,norm,epilogue,bits", [c + (4,) for c in CASES] + [c + (2,) for c in CASES_2])
def test_tiled_gemv_matches_oracle(cuda, n, k, norm, epilogue, bits):
    log(f"tiled gemv {n}x{k} bits={bits} norm={norm} epilogue={epilogue}")
    w = normal_tensor((n, k), 0.02, 50, cuda)
    x = normal_tensor((k,), 1.0, 51, cuda)
    g = normal_tensor((k,), 1.0, 52, cuda) if norm else None
    resid = normal_tensor((n,), 1.0, 53, cuda) if epilogue == 1 else None
    _, _, tc, tm = _quant(w, bits)
    lin = _lib.linear(codes=tc, meta=tm, bits=bits, layout=1)
    y = torch.empty(n // 2 if epilogue == 2 else n, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(lin, x, y, norm_w=g, eps=1e-6, epilogue=epilogue, resid=resid)
    torch.cuda.synchronize()
    rc, rm = oq(host(w), bits=bits)
    ref = _fused_ref(dequantize(rc, rm, bits=bits), host(x), None if g is None else host(g), 1e-6, epilogue,
                     None if resid is None else host(resid))
    assert rel_err(host(y), ref) < TOL


def test_tiled_gemv_gate_up_full_shape_sampled_rows(cuda):
    F, k = 18944, 3584
    log("tiled gate_up full")
    w = normal_tensor((2 * F, k), 0.02, 60, cuda)
    x = normal_tensor((k,), 1.0, 61, cuda)
    g = normal_tensor((k,), 1.0, 62, cuda)
    _, _, tc, tm = _quant(w)
    y = torch.empty(F, dtype=torch.bfloat16, device=cuda)
    _lib.gemv(_lib.linear(codes=tc, meta=tm, layout=1), x, y, norm_w=g, eps=1e-6, epilogue=2)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, F - 1, np.random.default_rng(5).integers(0, F, 256)])
    rc, rm = oq(host(w[np.r_[rows, F + rows]]))
    ref = _fused_ref(dequantize(rc, rm), host(x), host(g), 1e-6, 2, None)
    assert rel_err(host(y)[rows], ref) < TOL


def test_tiled_gemv_two_calls_same_bits(cuda):
    """The tiled GEMV is deterministic: two calls give the same bits."""
    n, k = 3584, 18944
    w = normal_tensor((n, k), 0.02, 70, cuda)
    x = normal_tensor((k,), 1.0, 71, cuda)
    _, _, tc, tm = _quant(w)
    lin = _lib.linear(codes=tc, meta=tm, layout=1)
    y0 = torch.empty(n, dtype=torch.bfloat16, device=cuda)
    y1 = torch.empty_like(y0)
    _lib.gemv(lin, x, y0)
    _lib.gemv(lin, x, y1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("n,k,m", [(512, 256, 1), (4608, 3584, 5), (3584, 18944, 16), (37888, 3584, 3)])
def test_tiled_w4_gemm_equals_rows(cuda, n, k, m):
    log(f"w4 gemm tiled vs rows {n}x{k} m={m}")
    w = normal_tensor((n, k), 0.02, 80, cuda)
    x = normal_tensor((m, k), 1.0, 81, cuda)
    codes, meta, tc, tm = _quant(w)
    ws = torch.zeros(_lib.w4_gemm_workspace_bytes(n, k, m), dtype=torch.uint8, device=cuda)
    y0 = torch.empty(m, n, dtype=torch.bfloat16, device=cuda)
    y1 = torch.empty_like(y0)
    _lib.w4_gemm(_lib.linear(codes=codes, meta=meta), x, y0, ws)
    _lib.w4_gemm(_lib.linear(codes=tc, meta=tm, layout=1), x, y1, ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("tiled,bits", [(True, 4), (False, 4), (True, 2)])
def test_draft_step_on_either_layout_matches_oracle(cuda, tiled, bits):
    """One 7B-shaped substitute layer (layer 0: the embedding prologue on the
    low-bit QKV site) through a draft step with the substitutes tiled or
    row-major, at 4 or 2 bits: logits within 1e-2 of the oracle."""
    from oracle.model import forward
    from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    from synth import kv_history, model_weights, token_ids
    from synth.configs import QWEN7B
    from tests.helpers import oracle_model
    shape, kv_len, cap = QWEN7B.with_(n_layers=1, n_shared=0), 700, 768
    log(f"draft step, substitutes tiled={tiled} bits={bits}")
    w = model_weights(shape, 9, cuda)
    dm = DeviceModel(shape, w, tiled=tiled, bits=bits)
    assert all(v == int(tiled) for v in dm.layout[0].values())
    dec = SpecDecoder(dm, cap, 4)
    K, V = kv_history(shape.n_layers, shape.n_kv_heads, kv_len, shape.head_dim, cap, 16, cuda)
    dec.k_cache.copy_(K)
    dec.v_cache.copy_(V)
    tok = int(token_ids(1, shape.vocab, 12)[0])
    dec.reset(kv_len, tok)
    _lib.draft_step(dm.c, dec.c, 0, 0.0, None, dec.ws)
    torch.cuda.synchronize()
    om = oracle_model(shape, w, [])
    om.make_substitutes(dm.substitute_layers, bits=bits)
    kv = (host(K).astype(np.float64), host(V).astype(np.float64))
    ref = forward(om, kv, kv_len, [tok], draft=True)[0]
    assert rel_err(host(dec.draft_logits[0]), ref) < TOL
