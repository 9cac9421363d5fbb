"""Test-side glue: host copies of synthetic weights handed to the oracle."""
import numpy as np

from oracle.model import OracleModel


def host(t):
    return t.detach().float().cpu().numpy()


def oracle_model(shape, w, substitute_layers=()):
    m = OracleModel(
        n_layers=len(w["layers"]), hidden=shape.hidden, ffn=shape.ffn,
        n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim,
        vocab=shape.vocab, rope_theta=shape.rope_theta, rms_eps=shape.rms_eps,
        embed=host(w["embed"]), final_norm=host(w["final_norm"]), lm_head=host(w["lm_head"]),
        layers=[{k: host(v) for k, v in lw.items()} for lw in w["layers"]],
    )
    m.make_substitutes(list(substitute_layers))
    return m


def memo_weights(om):
    """The oracle's weight matrices converted once (the same float64 values;
    the oracle dequantises substitutes on every call), for tests that run
    many forwards of one large layer."""
    cache, orig = {}, om.weight

    def weight(l, name, draft):
        key = (l, name, bool(draft and om.substitute and om.substitute[l] is not None))
        if key not in cache:
            cache[key] = orig(l, name, draft)
        return cache[key]
    om.weight = weight
    return om
