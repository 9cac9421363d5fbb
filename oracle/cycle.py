"""O6: the speculative cycle, KV sharing and rollback; plain AR decoding.

[SD] overall flow and pseudo-code: draft gamma tokens autoregressively, verify
gamma+1 positions in one target forward, run the rejection round, repeat; the
KV of rejected positions and everything after them is discarded (Module 2).
[SSN] Method details: draft and target share one KV cache.

State convention: committed tokens y_0..y_{c-1}; the cache holds target K/V
for positions 0..c-2, so kv_len = c - 1 and y_{c-1} is the next input.
Draft step i (i = 0..gamma-1) feeds tokens[i] at position kv_len + i and
writes draft K/V there; verify feeds tokens[0..gamma] at kv_len..kv_len+gamma
and overwrites those positions with target K/V, so committed K/V is always
the target's.  Rollback: kv_len += n + 1.

Uniform codes of cycle c: U_draft[c][i], R[c][i], U_final[c].

Pinned by: greedy speculative decoding == greedy autoregressive decoding of
the target (the lossless property at T = 0) and kv_len == committed - 1.
"""
import numpy as np

from .model import forward, new_kv
from .reject import reject
from .sampling import sample
from .sparse import build_index
from .adaptive import Controller, entropy


def prefill(model, kv, prompt):
    """Process prompt[:-1]; returns kv_len = len(prompt) - 1."""
    if len(prompt) > 1:
        forward(model, kv, 0, list(prompt[:-1]), draft=False, keep_logits=False)
    return len(prompt) - 1


def draft_tokens(model, kv, kv_len, last_token, gamma, draft_temp, U_draft, index=None):
    """gamma draft steps; with ``index`` the draft attends sparsely (sparse.py)."""
    toks = [int(last_token)]
    logits = []
    sparse = None if index is None else (index, kv_len)
    for i in range(gamma):
        z = forward(model, kv, kv_len + i, [toks[i]], draft=True, sparse=sparse)[0]
        logits.append(z)
        toks.append(sample(z.astype(np.float32), draft_temp, U_draft[i]))
    return toks, np.array(logits)


def speculative_cycle(model, kv, kv_len, last_token, gamma, temp, draft_temp, U_draft, R, U_final):
    toks, dlogits = draft_tokens(model, kv, kv_len, last_token, gamma, draft_temp, U_draft)
    tlogits = forward(model, kv, kv_len, toks, draft=False)
    n, out, status = reject(tlogits, dlogits, toks[1:], R, U_final, temp, draft_temp)
    return n, out, status, toks, dlogits, tlogits


def sparse_speculative_cycle(model, kv, kv_len, last_token, gamma, temp, draft_temp, U_draft, R,
                             U_final, index, n_sink, n_recent, window, budget_permille):
    """One cycle with a sparse-KV draft ([SSL] sections 3.1-3.2): the draft
    attends to ``index`` (None: dense, the first cycle), the verify pass
    yields the importance scores of its last ``window`` rows, and the index
    of the next cycle is rebuilt over the committed positions
    [0, kv_len + n + 1)."""
    toks, dlogits = draft_tokens(model, kv, kv_len, last_token, gamma, draft_temp, U_draft, index)
    scores = []
    tlogits = forward(model, kv, kv_len, toks, draft=False, scores=scores, score_window=window)
    n, out, status = reject(tlogits, dlogits, toks[1:], R, U_final, temp, draft_temp)
    new_index = build_index(scores, kv_len + n + 1, n_sink, n_recent, budget_permille)
    return n, out, status, toks, dlogits, tlogits, scores, new_index


def speculative_generate(model, prompt, n_generate, gamma, temp, draft_temp, uniforms, capacity):
    """Generate at least n_generate tokens; returns (tokens[:n_generate], per-cycle n)."""
    U_draft, R, U_final = uniforms
    kv = new_kv(model, capacity)
    kv_len = prefill(model, kv, prompt)
    committed = list(prompt)
    out, ns = [], []
    c = 0
    while len(out) < n_generate:
        n, emitted, _, _, _, _ = speculative_cycle(
            model, kv, kv_len, committed[-1], gamma, temp, draft_temp, U_draft[c], R[c], U_final[c])
        kv_len += n + 1
        committed += emitted
        out += emitted
        ns.append(n)
        assert kv_len == len(committed) - 1
        c += 1
    return out[:n_generate], ns


def autoregressive_generate(model, prompt, n_generate, temp, U, capacity):
    """Plain target decoding, one token per forward."""
    kv = new_kv(model, capacity)
    kv_len = prefill(model, kv, prompt)
    last = prompt[-1]
    out = []
    for t in range(n_generate):
        z = forward(model, kv, kv_len, [last], draft=False)[0]
        last = sample(z.astype(np.float32), temp, U[t])
        out.append(last)
        kv_len += 1
    return out


def adaptive_speculative_cycle(model, kv, kv_len, last_token, ctl, temp, draft_temp, U_draft, R, U_final,
                               entropies=None):
    """One cycle with the entropy-adaptive draft length ([SSL] section 3.3,
    oracle/adaptive.py): tokens are drafted one at a time until the
    controller stops (gamma_eff <= gamma_max), the gamma_eff + 1 positions are
    verified and judged, and the controller's centres are updated with the
    outcome.  ``entropies``: the entropies to feed the controller instead of
    the oracle's own (teacher forcing on another evaluation's values)."""
    toks = [int(last_token)]
    dlogits = []
    for i in range(ctl.gamma_max):
        z = forward(model, kv, kv_len + i, [toks[i]], draft=True)[0]
        dlogits.append(z)
        toks.append(sample(z.astype(np.float32), draft_temp, U_draft[i]))
        h = entropy(z) if entropies is None else float(entropies[i])
        if not ctl.after_token(h):
            break
    g = ctl.gamma_eff
    tlogits = forward(model, kv, kv_len, toks[:g + 1], draft=False)
    n, out, status = reject(tlogits, np.array(dlogits[:g]), toks[1:g + 1], R[:g], U_final, temp, draft_temp)
    ctl.after_round(n)
    return n, out, status, toks[:g + 1], np.array(dlogits[:g]), tlogits, g


def adaptive_generate(model, prompt, n_generate, gamma_max, c, temp, draft_temp, uniforms, capacity,
                      beta=None):
    """Speculative decoding with the entropy-adaptive draft length; returns
    (tokens[:n_generate], per-cycle n, per-cycle gamma_eff)."""
    U_draft, R, U_final = uniforms
    ctl = Controller(gamma_max, c) if beta is None else Controller(gamma_max, c, beta)
    kv = new_kv(model, capacity)
    kv_len = prefill(model, kv, prompt)
    committed = list(prompt)
    out, ns, gs = [], [], []
    c_i = 0
    while len(out) < n_generate:
        n, emitted, _, _, _, _, g = adaptive_speculative_cycle(
            model, kv, kv_len, committed[-1], ctl, temp, draft_temp, U_draft[c_i], R[c_i], U_final[c_i])
        kv_len += n + 1
        committed += emitted
        out += emitted
        ns.append(n)
        gs.append(g)
        c_i += 1
    return out[:n_generate], ns, gs
