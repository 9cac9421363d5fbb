"""Seeded random draws.

* Weights and activations: ``torch.Generator`` on the requested device, so that a
  GPU run draws its inputs in HBM without a host round trip; the oracle receives
  a host copy of the same tensors.
* Uniforms for the sampling decisions: integers U in [0, 2**24) from numpy's
  PCG64, handed out together with their float32 value U * 2**-24 (exact).
"""
import numpy as np
import torch

UNIFORM_BITS = 24


def normal_tensor(shape, std, seed, device="cpu", dtype=torch.bfloat16, mean=0.0):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def uniform_codes(n, seed):
    """Return (U int64 array, u float32 array) with u = U / 2**24 exactly."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    U = rng.integers(0, 1 << UNIFORM_BITS, size=n, dtype=np.int64)
    u = (U.astype(np.float64) / float(1 << UNIFORM_BITS)).astype(np.float32)
    return U, u


def token_ids(n, vocab, seed):
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def model_weights(shape, seed, device="cpu", std=0.02, layers=None):
    """Random-init decoder weights (bf16) of ``shape``.

    Returns a dict: embed [V][H], final_norm [H], lm_head [V][H] and
    ``layers``: list of dicts with attn_norm [H], ffn_norm [H], qkv
    [(Hq+2Hkv)d][H], o [H][Hq d], gate_up [2F][H] (gate rows then up rows),
    down [H][F].  Norm weights are ones.  Each matrix gets its own seed.
    """
    H, F = shape.hidden, shape.ffn
    base = int(seed) * 1000
    w = {
        "embed": normal_tensor((shape.vocab, H), std, base + 1, device),
        "final_norm": torch.ones(H, dtype=torch.bfloat16, device=device),
        "lm_head": normal_tensor((shape.vocab, H), std, base + 2, device),
        "layers": [],
    }
    idx = range(shape.n_layers) if layers is None else layers
    for l in idx:
        s = base + 10 + 10 * l
        w["layers"].append({
            "attn_norm": torch.ones(H, dtype=torch.bfloat16, device=device),
            "ffn_norm": torch.ones(H, dtype=torch.bfloat16, device=device),
            "qkv": normal_tensor((shape.qkv_rows, H), std, s + 1, device),
            "o": normal_tensor((H, shape.q_dim), std, s + 2, device),
            "gate_up": normal_tensor((2 * F, H), std, s + 3, device),
            "down": normal_tensor((H, F), std, s + 4, device),
        })
    return w


def kv_history(n_layers, n_kv_heads, length, head_dim, capacity, seed, device="cpu"):
    """Synthetic bf16 K and V caches [L][Hkv][capacity][d]; the first ``length``
    positions hold N(0,1) draws, the rest zeros."""
    k = torch.zeros((n_layers, n_kv_heads, capacity, head_dim), dtype=torch.bfloat16, device=device)
    v = torch.zeros_like(k)
    if length > 0:
        k[:, :, :length] = normal_tensor((n_layers, n_kv_heads, length, head_dim), 1.0, seed, device)
        v[:, :, :length] = normal_tensor((n_layers, n_kv_heads, length, head_dim), 1.0, seed + 1, device)
    return k, v


def logits_pair(gamma, vocab, seed, target_std=3.0, draft_noise=0.5, device="cpu"):
    """Target logits [gamma+1][V] ~ N(0, target_std^2) and draft logits
    [gamma][V] = target[:gamma] + N(0, draft_noise^2), both rounded to bf16."""
    t = normal_tensor((gamma + 1, vocab), target_std, seed, device, dtype=torch.float32)
    noise = normal_tensor((gamma, vocab), draft_noise, seed + 1, device, dtype=torch.float32)
    d = t[:gamma] + noise
    return t.to(torch.bfloat16), d.to(torch.bfloat16)
