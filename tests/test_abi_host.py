"""The C-ABI library loads, exports every symbol include/subspec.h declares,
and rejects bad arguments on the host before enqueuing anything (CPU only:
no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from self_speculative_decoding_w4a16_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "subspec.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(subspec_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_cycle_entry_points():
    names = _declared()
    for n in ("subspec_quantize", "subspec_draft_step", "subspec_verify", "subspec_reject",
              "subspec_kv_rollback"):
        assert n in names


def test_library_exports_every_declared_symbol():
    l = _lib.lib()
    for name in _declared():
        assert hasattr(l, name), name
    assert set(_declared()) == set(_lib.EXPORTS)
    assert _lib.abi_version() == 7  # subspec_state.attn_own_launch


V = ctypes.c_void_p


def test_quantize_argument_errors():
    l = _lib.lib()
    p = V(4096)
    assert l.subspec_quantize(None, 4, 64, 64, 4, p, p, None) == _lib.EINVAL
    assert l.subspec_quantize(p, 4, 64, 64, 5, p, p, None) == _lib.EUNSUPPORTED
    assert "bits" in _lib.last_error()
    assert l.subspec_quantize(p, 4, 64, 64, 1, p, p, None) == _lib.EUNSUPPORTED
    assert l.subspec_quantize(p, 4, 64, 64, 3, p, p, None) == _lib.ESHAPE  # 3 bits: k % 128
    assert "128" in _lib.last_error()
    assert l.subspec_quantize(p, 4, 64, 32, 4, p, p, None) == _lib.EUNSUPPORTED
    assert l.subspec_quantize(p, 4, 96, 64, 4, p, p, None) == _lib.ESHAPE
    assert l.subspec_quantize(p, 0, 64, 64, 4, p, p, None) == _lib.EINVAL


def test_tile_codes_and_layout_argument_errors():
    import ctypes
    l = _lib.lib()
    p = V(4096)
    assert l.subspec_tile_codes(None, p, 16, 128, 4, p, p, None) == _lib.EINVAL
    assert l.subspec_tile_codes(p, p, 16, 128, 4, p, None, None) == _lib.EINVAL
    assert l.subspec_tile_codes(p, p, 8, 128, 4, p, p, None) == _lib.ESHAPE     # n % 16
    assert l.subspec_tile_codes(p, p, 16, 192, 4, p, p, None) == _lib.ESHAPE    # 4 bits: k % 128
    assert l.subspec_tile_codes(p, p, 16, 128, 2, p, p, None) == _lib.ESHAPE    # 2 bits: k % 256
    assert "256" in _lib.last_error()
    assert l.subspec_tile_codes(p, p, 16, 256, 3, p, p, None) == _lib.EUNSUPPORTED
    assert l.subspec_tile_codes(p, p, 0, 128, 4, p, p, None) == _lib.EINVAL
    g = lambda lin, *a: l.subspec_gemv(ctypes.byref(lin), *a)
    tiled = lambda n, k, bits=4, layout=1: _lib.Linear(None, p, p, n, k, bits, layout)
    assert g(tiled(16, 128, layout=2), p, None, 0.0, 0, None, p, None) == _lib.EINVAL
    assert g(tiled(16, 256, bits=3), p, None, 0.0, 0, None, p, None) == _lib.EINVAL
    assert "4- or 2-bit" in _lib.last_error()
    assert g(tiled(24, 128), p, None, 0.0, 0, None, p, None) == _lib.ESHAPE     # n % 16
    assert g(tiled(16, 192), p, None, 0.0, 0, None, p, None) == _lib.ESHAPE     # k % 128
    assert g(tiled(16, 128, bits=2), p, None, 0.0, 0, None, p, None) == _lib.ESHAPE  # k % 256
    assert g(tiled(48, 128), p, p, 1e-6, 2, None, p, None) == _lib.ESHAPE       # SiLU: F % 16
    ws = (ctypes.c_uint8 * 4096)()
    assert l.subspec_w4_gemm(ctypes.byref(tiled(24, 128)), p, 1, p, ws, 4096, None) == _lib.ESHAPE
    assert l.subspec_w4_gemm(ctypes.byref(tiled(16, 256, bits=2)), p, 1, p, ws, 4096, None) == _lib.EINVAL


def test_gemv_gemm_sample_argument_errors():
    l = _lib.lib()
    p = V(4096)
    assert l.subspec_w4_gemv(p, p, 8, 96, p, p, None) == _lib.ESHAPE
    assert l.subspec_w4_gemv(p, p, 8, 64 * 1024, p, p, None) == _lib.EUNSUPPORTED
    assert l.subspec_bf16_gemv(p, 8, 12, p, p, None) == _lib.ESHAPE
    assert l.subspec_bf16_gemm(p, 8, 128, p, 513, p, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_bf16_gemm(p, 8, 100, p, 4, p, p, 1 << 20, None) == _lib.ESHAPE
    assert l.subspec_bf16_gemm(p, 4096, 4096, p, 17, p, None, 0, None) == _lib.EWORKSPACE
    assert l.subspec_sample(p, 0, 1.0, p, p, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_sample(p, 100, 1.0, None, p, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_sample(p, 100, 1.0, p, p, p, 16, None) == _lib.EWORKSPACE


def test_hbm_read_argument_errors():
    l = _lib.lib()
    p = V(4096)
    assert l.subspec_hbm_read(None, 64, p, None) == _lib.EINVAL
    assert l.subspec_hbm_read(p, 64, None, None) == _lib.EINVAL
    assert l.subspec_hbm_read(p, 0, p, None) == _lib.ESHAPE
    assert l.subspec_hbm_read(p, 40, p, None) == _lib.ESHAPE
    assert l.subspec_hbm_read(V(4100), 64, p, None) == _lib.EINVAL
    assert "aligned" in _lib.last_error()


def test_fused_gemv_argument_errors():
    import ctypes
    l = _lib.lib()
    p = V(4096)
    bf = _lib.Linear(p, None, None, 8, 128)
    both = _lib.Linear(p, p, p, 8, 128)
    odd = _lib.Linear(p, None, None, 7, 128)
    bad_bits = _lib.Linear(None, p, p, 8, 128, 5)
    three_64 = _lib.Linear(None, p, p, 8, 64, 3)
    wide = _lib.Linear(p, None, None, 8, 8192)
    g = lambda lin, *a: l.subspec_gemv(ctypes.byref(lin), *a)
    assert g(both, p, None, 0.0, 0, None, p, None) == _lib.EINVAL
    assert g(bf, p, None, 0.0, 3, None, p, None) == _lib.EINVAL
    assert g(bf, p, None, 0.0, 1, None, p, None) == _lib.EINVAL       # resid missing
    assert g(odd, p, p, 1e-6, 2, None, p, None) == _lib.ESHAPE        # odd gate/up rows
    assert g(_lib.Linear(p, None, None, 8, 96), p, None, 0.0, 0, None, p, None) == _lib.ESHAPE
    assert g(wide, p, p, 1e-6, 0, None, p, None) == _lib.EUNSUPPORTED  # norm above 6144
    assert g(bf, p, None, 0.0, 2, None, p, None) == _lib.EUNSUPPORTED  # SiLU needs the norm
    assert g(bf, None, p, 1e-6, 0, None, p, None) == _lib.EINVAL
    assert l.subspec_gemv(None, p, p, 1e-6, 0, None, p, None) == _lib.EINVAL
    assert g(bad_bits, p, None, 0.0, 0, None, p, None) == _lib.EINVAL   # width 5
    assert g(three_64, p, None, 0.0, 0, None, p, None) == _lib.ESHAPE   # 3 bits: k % 128


def test_reject_argument_errors():
    l = _lib.lib()
    p = V(4096)
    args = dict(vocab=100, T=1.0, Td=1.0)
    assert l.subspec_reject(65, 100, 1.0, 1.0, p, p, p, p, p, p, p, p, None, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_reject(4, 100, -1.0, 1.0, p, p, p, p, p, p, p, p, None, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_reject(4, 100, 1.0, 1.0, p, p, p, None, p, p, p, p, None, p, 1 << 20, None) == _lib.EINVAL
    assert l.subspec_reject(4, 100, 1.0, 1.0, p, p, p, p, p, p, p, p, None, p, 64, None) == _lib.EWORKSPACE
    assert l.subspec_reject(4, 1 << 25, 1.0, 1.0, p, p, p, p, p, p, p, p, None, p, 1 << 20, None) == _lib.EINVAL
    del args


def _fake_model(n_layers=1, head_dim=128, hidden=256, ffn=512, w4_bad=False):
    p = 4096
    H, F, Hq, Hkv = hidden, ffn, 2, 1
    qkv = (Hq + 2 * Hkv) * head_dim
    layers = (_lib.Layer * n_layers)()
    for l in range(n_layers):
        L = layers[l]
        L.attn_norm = L.ffn_norm = p
        L.qkv = _lib.Linear(p, None, None, qkv, H)
        L.o = _lib.Linear(p, None, None, H, Hq * head_dim)
        L.gate_up = _lib.Linear(p, None, None, 2 * F, H)
        L.down = _lib.Linear(p, None, None, H, F)
        L.qkv_d = _lib.Linear(None, p, p, qkv, H)
        L.o_d = _lib.Linear(None, p, p, H, Hq * head_dim)
        L.gate_up_d = _lib.Linear(None, p, p, 2 * F, H) if not w4_bad else _lib.Linear(p, p, p, 2 * F, H)
        L.down_d = _lib.Linear(p, None, None, H, F)
    m = _lib.Model(n_layers, H, F, Hq, Hkv, head_dim, 1000, 1e6, 1e-6, p, p, p,
                   ctypes.cast(layers, ctypes.POINTER(_lib.Layer)))
    return m, layers


def test_model_validation_and_workspace_size():
    l = _lib.lib()
    m, keep = _fake_model()
    n1 = l.subspec_workspace_bytes(ctypes.byref(m), 1, 1024)
    n17 = l.subspec_workspace_bytes(ctypes.byref(m), 17, 1024)
    assert n1 > 64 * 1024 and n17 > n1
    assert l.subspec_workspace_bytes(ctypes.byref(m), 65, 1024) == 0
    bad, keep2 = _fake_model(head_dim=64)
    assert l.subspec_workspace_bytes(ctypes.byref(bad), 1, 1024) == 0
    assert "head_dim" in _lib.last_error()
    bad2, keep3 = _fake_model(w4_bad=True)
    assert l.subspec_workspace_bytes(ctypes.byref(bad2), 1, 1024) == 0
    assert "gate_up_d" in _lib.last_error()


def test_draft_verify_argument_errors():
    l = _lib.lib()
    m, keep = _fake_model()
    p = 4096
    st = _lib.State(p, p, 1024, p, p, p, 4)
    ws = V(p)
    assert l.subspec_draft_step(ctypes.byref(m), ctypes.byref(st), 4, 0.0, None, ws, 1 << 30, None) == _lib.EINVAL
    assert l.subspec_draft_step(ctypes.byref(m), ctypes.byref(st), 0, 0.5, None, ws, 1 << 30, None) == _lib.EINVAL
    assert l.subspec_draft_step(ctypes.byref(m), ctypes.byref(st), 0, 0.0, None, ws, 128, None) == _lib.EWORKSPACE
    assert l.subspec_verify(ctypes.byref(m), ctypes.byref(st), 0, V(p), None, ws, 1 << 30, None) == _lib.EINVAL
    assert l.subspec_verify(ctypes.byref(m), ctypes.byref(st), 65, V(p), None, ws, 1 << 30, None) == _lib.EINVAL
    st_small = _lib.State(p, p, 8, p, p, p, 4)
    assert l.subspec_verify(ctypes.byref(m), ctypes.byref(st_small), 17, V(p), None, ws, 1 << 30, None) == _lib.ECAPACITY
    st_null = _lib.State(None, p, 1024, p, p, p, 4)
    assert l.subspec_verify(ctypes.byref(m), ctypes.byref(st_null), 4, V(p), None, ws, 1 << 30, None) == _lib.EINVAL
    assert l.subspec_kv_rollback(ctypes.byref(st), None, V(p), None) == _lib.EINVAL
    assert l.subspec_kv_advance(None, 1, None) == _lib.EINVAL


def test_multilevel_argument_errors():
    l = _lib.lib()
    m, keep = _fake_model()
    p = 4096
    st = _lib.State(p, p, 1024, p, p, p, 4)
    ws = V(p)
    dv = lambda st_, off, n, toks=V(p), nbytes=1 << 30: l.subspec_draft_verify(
        ctypes.byref(m), ctypes.byref(st_), off, n, toks, None, ws, nbytes, None)
    assert dv(st, 0, 0) == _lib.EINVAL
    assert dv(st, 0, 17) == _lib.EINVAL
    assert dv(st, 0, 4, toks=None) == _lib.EINVAL
    st_small = _lib.State(p, p, 8, p, p, p, 4)
    assert dv(st_small, 0, 9) == _lib.ECAPACITY
    assert dv(st_small, -1, 2) == _lib.ECAPACITY
    assert dv(st, 0, 4, nbytes=128) == _lib.EWORKSPACE
    ap = lambda at, max_n, n=V(p): l.subspec_draft_append(ctypes.byref(st), at, max_n, n, V(p), None)
    assert ap(-1, 2) == _lib.EINVAL
    assert ap(0, -1) == _lib.EINVAL
    assert ap(2, 3) == _lib.EINVAL  # past the gamma_max + 1 = 5 tokens
    assert ap(1, 2, n=None) == _lib.EINVAL
    assert "tokens buffer" in _lib.last_error() or "NULL" in _lib.last_error()


def test_tree_argument_errors():
    l = _lib.lib()
    m, keep = _fake_model()
    p = 4096
    st = _lib.State(p, p, 1024, p, p, p, 4)
    ws = V(p)
    big = 1 << 40
    by = ctypes.byref
    assert l.subspec_tree_workspace_bytes(by(m), 6, 48, 1024) > 64 * 1024
    assert l.subspec_tree_workspace_bytes(by(m), 17, 4, 1024) == 0  # k above 16
    assert l.subspec_tree_workspace_bytes(by(m), 8, 64, 1024) == 0  # 513 nodes
    assert l.subspec_tree_workspace_bytes(by(m), 2, 0, 1024) == 0
    # level outside [0, depth), sampled children without uniforms, a tree above the capacity
    assert l.subspec_tree_draft(by(m), by(st), 6, 8, 8, 0.0, None, ws, big, None) == _lib.EINVAL
    assert l.subspec_tree_draft(by(m), by(st), 6, 8, 0, 0.5, None, ws, big, None) == _lib.EINVAL
    st_small = _lib.State(p, p, 40, p, p, p, 4)
    assert l.subspec_tree_draft(by(m), by(st_small), 6, 8, 0, 0.0, None, ws, big, None) == _lib.ECAPACITY
    assert l.subspec_tree_verify(by(m), by(st_small), 6, 8, V(p), ws, big, None) == _lib.ECAPACITY
    assert l.subspec_tree_verify(by(m), by(st), 6, 8, None, ws, big, None) == _lib.EINVAL
    assert l.subspec_tree_verify(by(m), by(st), 6, 8, V(p), ws, 128, None) == _lib.EWORKSPACE
    # 3-bit draft weights: the tree's draft rows take bf16 or 4-bit only
    m3, keep3 = _fake_model()
    keep3[0].qkv_d = _lib.Linear(None, p, p, (2 + 2) * 128, 256, 3)
    assert l.subspec_tree_draft(by(m3), by(st), 2, 4, 0, 0.0, None, ws, big, None) == _lib.EUNSUPPORTED
    tr = l.subspec_tree_reject
    assert tr(6, 48, 1000, 1.0, 1.0, V(p), V(p), V(p), None, V(p), V(p), V(p), V(p), V(p), ws, big, None) == _lib.EINVAL
    assert tr(6, 48, 1000, -1.0, 1.0, V(p), V(p), V(p), V(p), V(p), V(p), V(p), V(p), V(p), ws, big, None) == _lib.EINVAL
    assert tr(0, 48, 1000, 0.0, 0.0, V(p), V(p), V(p), None, None, V(p), V(p), V(p), V(p), ws, big, None) == _lib.EINVAL
    assert tr(6, 48, 1000, 0.0, 0.0, V(p), V(p), V(p), None, None, V(p), V(p), V(p), V(p), ws, 64, None) == _lib.EWORKSPACE
    assert l.subspec_tree_commit(by(m), by(st), 6, 48, None, V(p), V(p), None) == _lib.EINVAL


def test_batch_argument_errors():
    l = _lib.lib()
    m, keep = _fake_model()
    p = 4096
    by = ctypes.byref
    big = 1 << 40
    ws = V(p)
    assert l.subspec_batch_workspace_bytes(by(m), 4, 17, 1024) > 64 * 1024
    assert l.subspec_batch_workspace_bytes(by(m), 17, 17, 1024) == 0  # batch above 16
    assert l.subspec_batch_workspace_bytes(by(m), 16, 64, 1024) == 0  # 1024 rows
    st = _lib.BatchState(p, p, 1024, 4, p, p, p, 4)
    assert l.subspec_batch_draft_step(by(m), by(st), 4, 0.0, None, ws, big, None) == _lib.EINVAL  # step >= gamma
    assert l.subspec_batch_draft_step(by(m), by(st), 0, 0.5, None, ws, big, None) == _lib.EINVAL  # no uniforms
    assert l.subspec_batch_draft_step(by(m), by(st), 0, 0.0, None, ws, 128, None) == _lib.EWORKSPACE
    bad = _lib.BatchState(p, p, 1024, 0, p, p, p, 4)
    assert l.subspec_batch_draft_step(by(m), by(bad), 0, 0.0, None, ws, big, None) == _lib.EINVAL
    assert l.subspec_batch_verify(by(m), by(st), 0, V(p), 5, None, ws, big, None) == _lib.EINVAL
    assert l.subspec_batch_verify(by(m), by(st), 5, V(p), 4, None, ws, big, None) == _lib.EINVAL  # ld < n
    assert l.subspec_batch_verify(by(m), by(st), 5, None, 5, None, ws, big, None) == _lib.EINVAL
    assert l.subspec_batch_reject(by(m), by(st), 1.0, 1.0, V(p), None, V(p), V(p), V(p), V(p), ws, big,
                                  None) == _lib.EINVAL
    assert l.subspec_batch_rollback(by(st), V(p), None, 0, None) == _lib.EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError):
        _lib.lib()


def test_index_count_matches_the_oracle_rule():
    # host-side arithmetic of the library (no device work): the list size of
    # the sparse draft index equals what the oracle's selection rule keeps
    from oracle.sparse import index_bounds
    for L in (0, 1, 3, 4, 67, 68, 69, 500, 4096, 60011):
        for sink, recent, budget in ((4, 64, 100), (0, 0, 1000), (4, 64, 0), (16, 8, 333), (4, 64, 1000)):
            s, r, K = index_bounds(L, sink, recent, budget)
            assert _lib.index_count(L, sink, recent, budget) == s + K + (L - r)
    for bad in ((-1, 4, 64, 100), (10, -1, 64, 100), (10, 4, -1, 100), (10, 4, 64, 1001)):
        with pytest.raises(_lib.SubspecError):
            _lib.index_count(*bad)
