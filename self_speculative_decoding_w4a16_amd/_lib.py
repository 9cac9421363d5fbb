"""ctypes binding of libsubspec.so (include/subspec.h).

Argument marshalling only: every function here forwards to the C ABI; the
work runs in the library's HIP kernels.  Importing this module does not load
the library; :func:`lib` does, and raises if it has not been built.
"""
import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsubspec.so")

OK = 0
EINVAL = -1
ESHAPE = -2
ECAPACITY = -3
EHIP = -4
EUNSUPPORTED = -5
EWORKSPACE = -6

STATUS_NONFINITE = 1
STATUS_ZERO_RESIDUAL = 2
STATUS_Q_ZERO = 4


class SubspecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libsubspec error {code}: {msg}")
        self.code = code


class Linear(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("codes", c_void_p), ("meta", c_void_p),
                ("n", c_int64), ("k", c_int64), ("bits", c_int32), ("layout", c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("ffn_norm", c_void_p),
                ("qkv", Linear), ("o", Linear), ("gate_up", Linear), ("down", Linear),
                ("qkv_d", Linear), ("o_d", Linear), ("gate_up_d", Linear), ("down_d", Linear)]


class Model(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("hidden", c_int32), ("ffn", c_int32),
                ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("vocab", c_int32), ("rope_theta", c_float), ("rms_eps", c_float),
                ("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers", POINTER(Layer))]


class State(ctypes.Structure):
    _fields_ = [("k_cache", c_void_p), ("v_cache", c_void_p), ("capacity", c_int32),
                ("kv_len", c_void_p), ("tokens", c_void_p), ("draft_logits", c_void_p),
                ("gamma_max", c_int32),
                ("kv_score", c_void_p), ("kv_index", c_void_p), ("kv_index_len", c_void_p),
                ("index_cap", c_int32), ("use_index", c_int32),
                ("n_sink", c_int32), ("n_recent", c_int32), ("score_window", c_int32),
                ("budget_permille", c_int32), ("draft_len", c_void_p), ("attn_own_launch", c_int32)]


class BatchState(ctypes.Structure):
    _fields_ = [("k_cache", c_void_p), ("v_cache", c_void_p), ("capacity", c_int32), ("batch", c_int32),
                ("kv_len", c_void_p), ("tokens", c_void_p), ("draft_logits", c_void_p), ("gamma_max", c_int32)]


class Control(ctypes.Structure):
    _fields_ = [("draft_len", c_void_p), ("state", c_void_p), ("entropy", c_void_p),
                ("c", ctypes.c_double), ("beta", ctypes.c_double), ("gamma_max", c_int32)]


_SIGS = {
    "subspec_abi_version": (c_int32, []),
    "subspec_last_error": (ctypes.c_char_p, []),
    "subspec_workspace_bytes": (c_size_t, [POINTER(Model), c_int32, c_int32]),
    "subspec_workspace_init": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "subspec_quantize": (c_int32, [c_void_p, c_int64, c_int64, c_int32, c_int32, c_void_p,
                                   c_void_p, c_void_p]),
    "subspec_tile_codes": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                     c_void_p]),
    "subspec_draft_step": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_float, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "subspec_verify": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "subspec_reject": (c_int32, [c_int32, c_int32, c_float, c_float, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "subspec_reject_len": (c_int32, [c_int32, c_int32, c_float, c_float, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "subspec_reject_batch": (c_int32, [c_int32, c_int32, c_int32, c_float, c_float, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_size_t, c_void_p]),
    "subspec_reject_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "subspec_control_init": (c_int32, [POINTER(Control), c_void_p]),
    "subspec_draft_control": (c_int32, [POINTER(Model), POINTER(State), c_int32, POINTER(Control), c_void_p,
                                        c_size_t, c_void_p]),
    "subspec_control_update": (c_int32, [POINTER(Control), c_void_p, c_void_p]),
    "subspec_reject_noalloc": (c_int32, [c_int32, c_int32, c_float, c_float, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
    "subspec_kv_rollback": (c_int32, [POINTER(State), c_void_p, c_void_p, c_void_p]),
    "subspec_kv_advance": (c_int32, [POINTER(State), c_int32, c_void_p]),
    "subspec_kv_select": (c_int32, [POINTER(Model), POINTER(State), c_void_p]),
    "subspec_index_count": (c_int64, [c_int64, c_int32, c_int32, c_int32]),
    "subspec_w4_gemv": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                  c_void_p]),
    "subspec_w4_gemm": (c_int32, [POINTER(Linear), c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "subspec_w4_gemm_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int32]),
    "subspec_bf16_gemv": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
    "subspec_gemv": (c_int32, [POINTER(Linear), c_void_p, c_void_p, c_float, c_int32, c_void_p,
                               c_void_p, c_void_p]),
    "subspec_bf16_gemm": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_int32, c_void_p,
                                    c_void_p, c_size_t, c_void_p]),
    "subspec_sample": (c_int32, [c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                 c_size_t, c_void_p]),
    "subspec_hbm_read": (c_int32, [c_void_p, c_int64, c_void_p, c_void_p]),
    "subspec_draft_verify": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "subspec_draft_append": (c_int32, [POINTER(State), c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "subspec_batch_workspace_bytes": (c_size_t, [POINTER(Model), c_int32, c_int32, c_int32]),
    "subspec_batch_draft_step": (c_int32, [POINTER(Model), POINTER(BatchState), c_int32, c_float, c_void_p, c_void_p,
                                           c_size_t, c_void_p]),
    "subspec_batch_verify": (c_int32, [POINTER(Model), POINTER(BatchState), c_int32, c_void_p, c_int64, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "subspec_batch_reject": (c_int32, [POINTER(Model), POINTER(BatchState), c_float, c_float, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "subspec_batch_rollback": (c_int32, [POINTER(BatchState), c_void_p, c_void_p, c_int32, c_void_p]),
    "subspec_tree_workspace_bytes": (c_size_t, [POINTER(Model), c_int32, c_int32, c_int32]),
    "subspec_tree_draft": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_int32, c_int32, c_float, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "subspec_tree_verify": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_int32, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    "subspec_tree_reject": (c_int32, [c_int32, c_int32, c_int32, c_float, c_float, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    "subspec_tree_commit": (c_int32, [POINTER(Model), POINTER(State), c_int32, c_int32, c_void_p, c_void_p,
                                      c_void_p, c_void_p]),
    "subspec_profile_start": (c_int32, [c_int32]),
    "subspec_profile_stop": (c_int32, []),
    "subspec_profile_read": (c_int32, [c_int32, POINTER(c_int64), POINTER(ctypes.c_double),
                                       POINTER(ctypes.c_double)]),
}

# Profiler classes (launch sites), in the order of the SUBSPEC_K_* enum.
K_NAMES = ("w4_qkv", "w4_o", "w4_gate_up", "w4_down",
           "bf16_qkv", "bf16_o", "bf16_gate_up", "bf16_down", "lm_head",
           "gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "gemm_lm_head",
           "attn_draft", "attn_verify", "sample", "reject", "misc", "scores", "select", "qkv_attn")
K = {name: i for i, name in enumerate(K_NAMES)}
# Groups of classes: every draft GEMV on a 4-bit substitute, every draft GEMV
# on bf16 weights, and every verify GEMM.
K_GROUPS = {"w4_gemv": K_NAMES[0:4], "bf16_gemv": K_NAMES[4:9], "verify_gemm": K_NAMES[9:14]}

EXPORTS = tuple(_SIGS)

_lib = None


def lib():
    """Load libsubspec.so (once).  Raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m self_speculative_decoding_w4a16_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def last_error():
    return lib().subspec_last_error().decode()


def check(code):
    if code != OK:
        raise SubspecError(code, last_error())
    return code


def _p(t):
    """Device (or host) pointer of a tensor, or None."""
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    return c_void_p(stream)


# ---------------------------------------------------------------- entry points
def abi_version():
    return lib().subspec_abi_version()


def workspace_bytes(model, max_tokens, capacity):
    n = lib().subspec_workspace_bytes(ctypes.byref(model), max_tokens, capacity)
    if n == 0:
        raise SubspecError(EINVAL, last_error())
    return n


def workspace_init(ws, stream=None):
    check(lib().subspec_workspace_init(_p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def code_row_bytes(k, bits):
    """Bytes of one row of codes at ``bits`` (layout of subspec_quantize)."""
    return {4: k // 2, 2: k // 4, 3: 3 * k // 8}[bits]


def quantize(w, codes, meta, group=64, bits=4, stream=None):
    n, k = w.shape
    check(lib().subspec_quantize(_p(w), n, k, group, bits, _p(codes), _p(meta), _stream(stream)))


def tile_codes(codes, meta, tcodes, tmeta, bits=4, stream=None):
    """4- or 2-bit codes [n][k bits/8] + meta [n][k/64][2] -> the 16-row tiles
    of subspec_tile_codes (same sizes)."""
    n, k = codes.shape[0], 64 * meta.shape[1]
    check(lib().subspec_tile_codes(_p(codes), _p(meta), n, k, bits, _p(tcodes), _p(tmeta), _stream(stream)))


def draft_step(model, state, step, draft_temp, u_codes, ws, stream=None):
    check(lib().subspec_draft_step(ctypes.byref(model), ctypes.byref(state), step, draft_temp,
                                   _p(u_codes), _p(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def verify(model, state, n_tokens, tokens, logits, ws, stream=None):
    check(lib().subspec_verify(ctypes.byref(model), ctypes.byref(state), n_tokens, _p(tokens),
                               _p(logits), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def reject(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
           u_code, n_accepted, out_tokens, status, probs, ws, stream=None):
    check(lib().subspec_reject(gamma, vocab, temp, draft_temp, _p(target_logits), _p(draft_logits),
                               _p(draft_tokens), _p(r_codes), _p(u_code), _p(n_accepted),
                               _p(out_tokens), _p(status), _p(probs), _p(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))


def reject_len(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
               u_code, gamma_len, n_accepted, out_tokens, status, probs, ws, stream=None):
    check(lib().subspec_reject_len(gamma, vocab, temp, draft_temp, _p(target_logits), _p(draft_logits),
                                   _p(draft_tokens), _p(r_codes), _p(u_code), _p(gamma_len), _p(n_accepted),
                                   _p(out_tokens), _p(status), _p(probs), _p(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def reject_workspace_bytes(batch, gamma, vocab):
    n = lib().subspec_reject_workspace_bytes(batch, gamma, vocab)
    if n == 0:
        raise SubspecError(EINVAL, last_error())
    return n


def reject_batch(batch, gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
                 u_codes, gamma_len, n_accepted, out_tokens, status, probs, ws, stream=None):
    check(lib().subspec_reject_batch(batch, gamma, vocab, temp, draft_temp, _p(target_logits), _p(draft_logits),
                                     _p(draft_tokens), _p(r_codes), _p(u_codes), _p(gamma_len), _p(n_accepted),
                                     _p(out_tokens), _p(status), _p(probs), _p(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def control_init(ctl, stream=None):
    check(lib().subspec_control_init(ctypes.byref(ctl), _stream(stream)))


def draft_control(model, state, step, ctl, ws, stream=None):
    check(lib().subspec_draft_control(ctypes.byref(model), ctypes.byref(state), step, ctypes.byref(ctl), _p(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def control_update(ctl, n_accepted, stream=None):
    check(lib().subspec_control_update(ctypes.byref(ctl), _p(n_accepted), _stream(stream)))


def reject_noalloc(gamma, vocab, temp, draft_temp, target_logits, draft_logits, draft_tokens, r_codes,
                   u_code, n_accepted, out_tokens, status, probs, stream=None):
    check(lib().subspec_reject_noalloc(gamma, vocab, temp, draft_temp, _p(target_logits),
                                       _p(draft_logits), _p(draft_tokens), _p(r_codes), _p(u_code),
                                       _p(n_accepted), _p(out_tokens), _p(status), _p(probs),
                                       _stream(stream)))


def kv_rollback(state, n_accepted, out_tokens, stream=None):
    check(lib().subspec_kv_rollback(ctypes.byref(state), _p(n_accepted), _p(out_tokens),
                                    _stream(stream)))


def kv_select(model, state, stream=None):
    check(lib().subspec_kv_select(ctypes.byref(model), ctypes.byref(state), _stream(stream)))


def index_count(L, n_sink, n_recent, budget_permille):
    """Entries of every sparse index list at kv_len = L (subspec_index_count)."""
    n = lib().subspec_index_count(L, n_sink, n_recent, budget_permille)
    if n < 0:
        raise SubspecError(EINVAL, last_error())
    return n


def kv_advance(state, delta, stream=None):
    check(lib().subspec_kv_advance(ctypes.byref(state), delta, _stream(stream)))


def w4_gemv(codes, meta, n, k, x, y, stream=None):
    check(lib().subspec_w4_gemv(_p(codes), _p(meta), n, k, _p(x), _p(y), _stream(stream)))


def w4_gemm_workspace_bytes(n, k, m):
    b = lib().subspec_w4_gemm_workspace_bytes(n, k, m)
    if b == 0:
        raise SubspecError(EINVAL, last_error())
    return b


def w4_gemm(lin, x, y, ws, stream=None):
    """Y [m][n] = X [m][k] W^T on 4-bit weights (m <= 16), matrix cores."""
    check(lib().subspec_w4_gemm(ctypes.byref(lin), _p(x), x.shape[0], _p(y), _p(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def bf16_gemv(w, x, y, stream=None):
    n, k = w.shape
    check(lib().subspec_bf16_gemv(_p(w), n, k, _p(x), _p(y), _stream(stream)))


def hbm_read(buf, sink, stream=None):
    """One streaming read of the device tensor buf (the HBM read ceiling);
    the int32 device scalar sink is XORed with every 32-bit word of buf."""
    check(lib().subspec_hbm_read(_p(buf), buf.numel() * buf.element_size(), _p(sink), _stream(stream)))


def linear(w=None, codes=None, meta=None, n=None, k=None, bits=4, layout=0):
    """A subspec_linear for bf16 weights w [n][k], or low-bit codes + meta
    [n][k/64][2] at ``bits`` = 4, 3 or 2 (k from meta when not given);
    ``layout`` 1: codes + meta in the tiles of tile_codes."""
    if w is not None:
        n, k = w.shape
        return Linear(_p(w), None, None, n, k, 0, 0)
    n = codes.shape[0] if n is None else n
    k = 64 * meta.shape[1] if k is None else k
    return Linear(None, _p(codes), _p(meta), n, k, bits, layout)


GEMV_STORE, GEMV_RESID, GEMV_SILU = 0, 1, 2


def gemv(lin, x, y, norm_w=None, eps=0.0, epilogue=GEMV_STORE, resid=None, stream=None):
    check(lib().subspec_gemv(ctypes.byref(lin), _p(x), _p(norm_w), eps, epilogue, _p(resid), _p(y),
                             _stream(stream)))


def bf16_gemm(w, x, y, ws, stream=None):
    n, k = w.shape
    m = x.shape[0]
    check(lib().subspec_bf16_gemm(_p(w), n, k, _p(x), m, _p(y), _p(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def sample(logits, temp, u_code, token, ws, stream=None):
    check(lib().subspec_sample(_p(logits), logits.numel(), temp, _p(u_code), _p(token), _p(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))


def draft_verify(model, state, pos_offset, n_tokens, tokens, logits, ws, stream=None):
    check(lib().subspec_draft_verify(ctypes.byref(model), ctypes.byref(state), pos_offset, n_tokens, _p(tokens),
                                     _p(logits), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def draft_append(state, at, max_n, n_accepted, out_tokens, stream=None):
    check(lib().subspec_draft_append(ctypes.byref(state), at, max_n, _p(n_accepted), _p(out_tokens),
                                     _stream(stream)))


def batch_workspace_bytes(model, batch, max_tokens, capacity):
    n = lib().subspec_batch_workspace_bytes(ctypes.byref(model), batch, max_tokens, capacity)
    if n == 0:
        raise SubspecError(EINVAL, last_error())
    return n


def batch_draft_step(model, state, step, draft_temp, u_codes, ws, stream=None):
    check(lib().subspec_batch_draft_step(ctypes.byref(model), ctypes.byref(state), step, draft_temp, _p(u_codes),
                                         _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def batch_verify(model, state, n_tokens, tokens, ld_tokens, logits, ws, stream=None):
    check(lib().subspec_batch_verify(ctypes.byref(model), ctypes.byref(state), n_tokens, _p(tokens), ld_tokens,
                                     _p(logits), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def batch_reject(model, state, temp, draft_temp, target_logits, r_codes, u_codes, n_accepted, out_tokens, status,
                 ws, stream=None):
    check(lib().subspec_batch_reject(ctypes.byref(model), ctypes.byref(state), temp, draft_temp, _p(target_logits),
                                     _p(r_codes), _p(u_codes), _p(n_accepted), _p(out_tokens), _p(status), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def batch_rollback(state, n_accepted, out_tokens, delta=0, stream=None):
    check(lib().subspec_batch_rollback(ctypes.byref(state), _p(n_accepted), _p(out_tokens), delta, _stream(stream)))


def tree_workspace_bytes(model, k, depth, capacity):
    n = lib().subspec_tree_workspace_bytes(ctypes.byref(model), k, depth, capacity)
    if n == 0:
        raise SubspecError(EINVAL, last_error())
    return n


def tree_draft(model, state, k, depth, level, draft_temp, u_codes, ws, stream=None):
    check(lib().subspec_tree_draft(ctypes.byref(model), ctypes.byref(state), k, depth, level, draft_temp,
                                   _p(u_codes), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def tree_verify(model, state, k, depth, logits, ws, stream=None):
    check(lib().subspec_tree_verify(ctypes.byref(model), ctypes.byref(state), k, depth, _p(logits), _p(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def tree_reject(k, depth, vocab, temp, draft_temp, target_logits, draft_logits, tokens, r_codes, u_code,
                n_accepted, chain, out_tokens, status, ws, stream=None):
    check(lib().subspec_tree_reject(k, depth, vocab, temp, draft_temp, _p(target_logits), _p(draft_logits),
                                    _p(tokens), _p(r_codes), _p(u_code), _p(n_accepted), _p(chain),
                                    _p(out_tokens), _p(status), _p(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def tree_commit(model, state, k, depth, n_accepted, chain, out_tokens, stream=None):
    check(lib().subspec_tree_commit(ctypes.byref(model), ctypes.byref(state), k, depth, _p(n_accepted),
                                    _p(chain), _p(out_tokens), _stream(stream)))


def profile_start(max_records=200000):
    check(lib().subspec_profile_start(max_records))


def profile_stop():
    check(lib().subspec_profile_stop())


def profile_read(cls):
    """(launches, total_ms, algorithmic bytes) recorded for kernel class cls."""
    n, ms, b = c_int64(), ctypes.c_double(), ctypes.c_double()
    check(lib().subspec_profile_read(cls, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(b)))
    return n.value, ms.value, b.value
