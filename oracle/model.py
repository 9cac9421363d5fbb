"""O2/O3: the decoder forward used by both the draft and the verifier.

[SSN] Method details: the draft is the target itself - every layer keeps its
structure, the offloaded layers are replaced by their low-precision
substitutes, the resident layers are shared bit-for-bit, and draft and target
read and write one KV cache.  [SD] Module 2: the verifier runs all gamma+1
positions in one causal forward and returns gamma+1 distributions.

The pages give no architecture details; the reading is a Qwen/Llama-style
decoder with no biases: embed -> L x [RMSNorm -> QKV -> rotate-half RoPE ->
KV store -> causal GQA attention (scale 1/sqrt(d)) -> O + residual ->
RMSNorm -> SiLU(gate) * up -> down + residual] -> RMSNorm -> lm_head.
Math runs in float64; values are rounded to bfloat16 at the storage points:
norm outputs, each GEMV/GEMM output, Q and K after RoPE, the KV cache,
attention output, each residual sum, the SiLU*up product and the logits.
A residual-add projection is rounded once: bf16(h + W x).

Summation precision: the sums of every projection are float64 by default.
``acc=np.float32`` evaluates the same definition with float32 sums (the
definition fixes the storage points, not the order or precision of a sum;
the GPU sums in float32 in its own order).  Over one layer the two agree to
well inside the logits tolerance; over many random-init layers the bf16
roundings they take differently compound, and their distance measures how
far two equally valid evaluations of a deep model part.

Pinned by: verify row j equals the one-token decode at the same position,
attention equal to the masked full-matrix softmax, RMSNorm of a constant
vector, RoPE's norm preservation and relative-position property, the W4
special case where every code is equal, and greedy speculative decoding
equal to greedy autoregressive decoding (cycle.py).
"""
from dataclasses import dataclass, field

import numpy as np

from .bf16 import round_bf16
from .quant import quantize, dequantize


@dataclass
class OracleModel:
    n_layers: int
    hidden: int
    ffn: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rope_theta: float
    rms_eps: float
    embed: np.ndarray            # [V][H] bf16 values
    final_norm: np.ndarray       # [H]
    lm_head: np.ndarray          # [V][H]
    layers: list                 # dicts: attn_norm, ffn_norm, qkv, o, gate_up, down
    substitute: list = field(default_factory=list)  # per layer: None or dict name -> (codes, meta, bits)

    def make_substitutes(self, layer_ids, bits=4):
        """Quantise every matrix of the listed layers (O1) at ``bits`` (an int,
        or a list giving each listed layer its width); others stay shared."""
        self.substitute = [None] * self.n_layers
        layer_ids = list(layer_ids)
        widths = bits if isinstance(bits, (list, tuple)) else [bits] * len(layer_ids)
        for l, b in zip(layer_ids, widths):
            self.substitute[l] = {name: quantize(self.layers[l][name], bits=b) + (b,)
                                  for name in ("qkv", "o", "gate_up", "down")}

    def weight(self, l, name, draft):
        """Float64 weight matrix used by the draft (substitute) or the target."""
        if draft and self.substitute and self.substitute[l] is not None:
            codes, meta, bits = self.substitute[l][name]
            return dequantize(codes, meta, bits=bits)
        return np.asarray(self.layers[l][name], dtype=np.float64)


def new_kv(model, capacity):
    shape = (model.n_layers, model.n_kv_heads, capacity, model.head_dim)
    return np.zeros(shape, dtype=np.float64), np.zeros(shape, dtype=np.float64)


def rmsnorm(h, g, eps):
    """bf16(h / sqrt(mean(h^2) + eps) * g) for each row of h."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return round_bf16(h / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64))


def linear(x, w, acc=np.float64):
    """bf16(x W^T): rows of x against rows of W (sums in float64, or acc)."""
    return round_bf16((np.asarray(x, dtype=acc) @ np.asarray(w, dtype=acc).T).astype(np.float64))


def project(x, w, acc=np.float64):
    """x W^T with sums in float64 (or acc), not rounded."""
    return (np.asarray(x, dtype=acc) @ np.asarray(w, dtype=acc).T).astype(np.float64)


def rope(x, pos, theta):
    """Rotate-half RoPE of one head vector x [d] at integer position pos."""
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:half], x[half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s])


def silu(x):
    return x / (1.0 + np.exp(-x))


def attend(q, K, V, n_keys):
    """softmax(q K[:n]^T / sqrt(d)) V[:n] for one query head (float64)."""
    d = q.shape[0]
    s = (K[:n_keys] @ q) / np.sqrt(d)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ V[:n_keys]


def forward(model, kv, kv_len, tokens, draft=False, keep_logits=True, sparse=None, scores=None,
            score_window=16, acc=np.float64):
    """Run tokens[j] at position kv_len + j, j = 0..n-1, through the decoder.

    Writes the K/V of those positions into ``kv`` and returns the logits
    [n][V] (bf16 values as float64).  Row j attends to positions
    [0, kv_len + j].  ``draft`` selects the substitute weights.

    ``sparse = (index, base)``: row j of layer l, query head h attends only
    to the positions index[l][h // group] (ascending, all < base) and the
    speculative positions [base, kv_len + j] (sparse.py).
    ``scores``: a list that receives, per layer, the importance scores
    [n_kv_heads][kv_len + n] of this pass (sparse.py, importance_scores).
    ``acc``: precision of the projection sums (float64, or float32).
    """
    K, V = kv
    n = len(tokens)
    Hq, Hkv, d = model.n_q_heads, model.n_kv_heads, model.head_dim
    group = Hq // Hkv
    h = np.stack([np.asarray(model.embed[t], dtype=np.float64) for t in tokens])
    for l in range(model.n_layers):
        lw = model.layers[l]
        x = rmsnorm(h, lw["attn_norm"], model.rms_eps)
        qkv = linear(x, model.weight(l, "qkv", draft), acc)
        attn = np.zeros((n, Hq * d))
        for j in range(n):
            pos = kv_len + j
            for hk in range(Hkv):
                k = qkv[j, (Hq + hk) * d:(Hq + hk + 1) * d]
                v = qkv[j, (Hq + Hkv + hk) * d:(Hq + Hkv + hk + 1) * d]
                K[l, hk, pos] = round_bf16(rope(k, pos, model.rope_theta))
                V[l, hk, pos] = v
        if scores is not None:
            from .sparse import attention_probs
            sc = np.zeros((Hkv, kv_len + n))
        for j in range(n):
            pos = kv_len + j
            for hq in range(Hq):
                q = round_bf16(rope(qkv[j, hq * d:(hq + 1) * d], pos, model.rope_theta))
                hk = hq // group
                if sparse is None:
                    attn[j, hq * d:(hq + 1) * d] = attend(q, K[l, hk], V[l, hk], pos + 1)
                else:
                    index, base = sparse
                    keys = np.concatenate([np.asarray(index[l][hk], dtype=np.int64),
                                           np.arange(base, pos + 1)])
                    attn[j, hq * d:(hq + 1) * d] = attend(q, K[l, hk][keys], V[l, hk][keys], len(keys))
                if scores is not None and j >= n - score_window:
                    sc[hk, :pos + 1] += attention_probs(q, K[l, hk], pos + 1)
        if scores is not None:
            scores.append(sc)
        attn = round_bf16(attn)
        h = round_bf16(h + project(attn, model.weight(l, "o", draft), acc))
        x = rmsnorm(h, lw["ffn_norm"], model.rms_eps)
        gu = linear(x, model.weight(l, "gate_up", draft), acc)
        F = model.ffn
        act = round_bf16(silu(gu[:, :F]) * gu[:, F:])
        h = round_bf16(h + project(act, model.weight(l, "down", draft), acc))
    if not keep_logits:
        return None
    x = rmsnorm(h, model.final_norm, model.rms_eps)
    return linear(x, model.lm_head, acc)
