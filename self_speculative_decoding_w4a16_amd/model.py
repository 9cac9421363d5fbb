"""Device-resident model: bf16 target weights, low-bit substitute copies
(4 bits by default, or 3 / 2 bits per layer) built with the library's
quantiser, and the C structs that describe them.

The draft is the target itself with the layers [n_shared, n_layers) replaced
by their substitutes and the layers [0, n_shared) shared bit for bit
("SubSpec: Speculate Deep and Accurate" paper note, Method details).  Torch
only allocates device memory here; the quantisation runs in the HIP kernel.
"""
import ctypes

import torch

from . import _lib

MATS = ("qkv", "o", "gate_up", "down")


MAX_TILED_K = 28672
TILE_K = {4: 128, 2: 256}  # k of one 64-byte tile chunk per code width


class DeviceModel:
    def __init__(self, shape, weights, substitute_layers=None, stream=None, bits=4, tiled=True):
        """``weights``: dict from synth.model_weights (bf16 tensors on the GPU).
        ``substitute_layers``: indices quantised for the draft (default: all
        layers from ``shape.n_shared`` on).  ``bits``: code width of the
        substitutes, 4, 3 or 2 (an int, or a dict layer -> width).
        ``tiled``: keep 4- and 2-bit substitutes in the 16-row tiles of
        subspec_tile_codes (the matrix-core draft GEMV) where the shape
        allows; otherwise (and at 3 bits) row-major."""
        self.shape = shape
        self.w = weights
        L = len(weights["layers"])
        if substitute_layers is None:
            substitute_layers = range(shape.n_shared, L)
        self.substitute_layers = sorted(set(substitute_layers))
        self.bits = {l: (bits[l] if isinstance(bits, dict) else bits) for l in self.substitute_layers}
        self.q = [None] * L
        self.layout = [None] * L
        for l in self.substitute_layers:
            self.q[l], self.layout[l] = {}, {}
            b = self.bits[l]
            for name in MATS:
                wt = weights["layers"][l][name]
                n, k = wt.shape
                codes = torch.empty((n, _lib.code_row_bytes(k, b)), dtype=torch.uint8, device=wt.device)
                meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=wt.device)
                _lib.quantize(wt, codes, meta, bits=b, stream=stream)
                lay = int(tiled and b in TILE_K and n % 16 == 0 and k % TILE_K[b] == 0 and k <= MAX_TILED_K)
                if lay:
                    tc, tm = torch.empty_like(codes), torch.empty_like(meta)
                    _lib.tile_codes(codes, meta, tc, tm, bits=b, stream=stream)
                    codes, meta = tc, tm
                self.q[l][name] = (codes, meta)
                self.layout[l][name] = lay
        self._build_structs()

    def _lin_bf16(self, t):
        n, k = t.shape
        return _lib.Linear(t.data_ptr(), None, None, n, k, 0, 0)

    def _lin_w4(self, codes, meta, bits, layout):
        n = codes.shape[0]
        return _lib.Linear(None, codes.data_ptr(), meta.data_ptr(), n, 64 * meta.shape[1], bits, layout)

    def linear_d(self, l, name):
        """The draft's subspec_linear of matrix ``name`` of layer ``l``."""
        if self.q[l] is not None:
            return self._lin_w4(*self.q[l][name], self.bits[l], self.layout[l][name])
        return self._lin_bf16(self.w["layers"][l][name])

    def _build_structs(self):
        s = self.shape
        L = len(self.w["layers"])
        self.layer_array = (_lib.Layer * L)()
        for l, lw in enumerate(self.w["layers"]):
            st = self.layer_array[l]
            st.attn_norm = lw["attn_norm"].data_ptr()
            st.ffn_norm = lw["ffn_norm"].data_ptr()
            for name in MATS:
                setattr(st, name, self._lin_bf16(lw[name]))
                setattr(st, name + "_d", self.linear_d(l, name))
        self.c = _lib.Model(L, s.hidden, s.ffn, s.n_q_heads, s.n_kv_heads, s.head_dim, s.vocab,
                            s.rope_theta, s.rms_eps, self.w["embed"].data_ptr(),
                            self.w["final_norm"].data_ptr(), self.w["lm_head"].data_ptr(),
                            ctypes.cast(self.layer_array, ctypes.POINTER(_lib.Layer)))

    @property
    def n_layers(self):
        return len(self.w["layers"])

    def weight_bytes(self, draft):
        """Bytes of weights one forward streams (draft: W4 codes + fp16 meta for
        substitutes, bf16 otherwise; lm_head included)."""
        total = 0
        for l, lw in enumerate(self.w["layers"]):
            for name in MATS:
                if draft and self.q[l] is not None:
                    c, m = self.q[l][name]
                    total += c.numel() + 2 * m.numel()
                else:
                    total += 2 * lw[name].numel()
        return total + 2 * self.w["lm_head"].numel()
