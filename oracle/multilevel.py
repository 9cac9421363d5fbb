"""O10: multi-level substitutes - a 2-bit draft for the 4-bit draft.

[SSR] section 10.3, item (9): a 2-bit substitute drafts for the 4-bit
substitute, which drafts for the bf16 target (ML-SpecQD's multi-level
scheme).  Reading (the report names the scheme, not its steps): nested
speculative decoding.  One outer cycle needs gamma tokens of the 4-bit draft
and the 4-bit distributions they were drawn from; inner rounds produce them:

  * the 2-bit model (the same substituted layers at 2 bits, the same shared
    bf16 layers) drafts up to gamma2 tokens from the last middle token;
  * the 4-bit model runs those positions in one pass (its logits at every
    row) and the plain round of reject.py judges them with p = the 4-bit
    distribution at T_mid and q = the 2-bit one at T2;
  * the accepted tokens and the round's residual / bonus token are appended
    to the middle tokens, with the 4-bit logits of the rows that predicted
    them; rounds repeat until gamma middle tokens exist (the last round's
    surplus is dropped).

The outer round then judges the gamma middle tokens against the bf16 target
with q = those 4-bit logits at T_mid - the plain cycle's round.  It stays
lossless because every middle token is an exact sample of the 4-bit model's
conditional given the earlier middle tokens (the inner round samples its p
exactly), so the middle tokens are distributed as a plain 4-bit draft's.

Cache: the three levels share one KV cache; the 2-bit drafts write their K/V
at the speculative positions, each 4-bit pass overwrites the positions it
runs, and the target's verify overwrites all gamma + 1 of them.

Uniform codes of one outer cycle: inner round r (r < gamma) draws its i-th
draft token with U2[r][i], tests with R2[r][i] and draws its last token with
F2[r]; the outer round uses R[0..gamma) and U.

Pinned by: greedy multi-level decoding equal to greedy autoregressive
decoding of the target; a 2-bit model equal to the 4-bit one accepting every
inner draft; the middle tokens equal to plain speculative decoding of the
4-bit model with the 2-bit draft; the first emitted token's law equal to the
target's softmax (chi-square).
"""
import numpy as np

from .model import forward
from .reject import reject
from .sampling import sample


def middle_tokens(om4, om2, kv, kv_len, last_token, gamma, gamma2, T_mid, T2, U2, R2, F2):
    """The gamma middle tokens after last_token (positions kv_len ..), their
    4-bit logits [gamma][V], and each inner round's (drafted, n, status)."""
    toks = [int(last_token)]
    mlog = []
    rounds = []
    r = 0
    while len(toks) - 1 < gamma:
        base = len(toks) - 1
        g = min(gamma2, gamma - base)
        d = [toks[-1]]
        dlog = []
        for i in range(g):
            z = forward(om2, kv, kv_len + base + i, [d[i]], draft=True)[0]
            dlog.append(z)
            d.append(sample(z.astype(np.float32), T2, U2[r][i]))
        L = forward(om4, kv, kv_len + base, d, draft=True)
        n, out, status = reject(L, np.array(dlog), d[1:], list(R2[r][:g]), F2[r], T_mid, T2)
        take = min(n + 1, gamma - base)
        toks += out[:take]
        mlog += [L[i] for i in range(take)]
        rounds.append((g, n, status))
        r += 1
    return toks, np.array(mlog), rounds


def multilevel_cycle(om4, om2, kv, kv_len, last_token, gamma, gamma2, T, T_mid, T2, U2, R2, F2, R, U):
    """One outer cycle; om4 is also the target (draft=False reads its bf16
    weights).  Returns (n, emitted tokens, status, middle tokens, middle
    logits, target logits, inner rounds)."""
    toks, mlog, rounds = middle_tokens(om4, om2, kv, kv_len, last_token, gamma, gamma2, T_mid, T2, U2, R2, F2)
    tlog = forward(om4, kv, kv_len, toks, draft=False)
    n, out, status = reject(tlog, mlog, toks[1:], list(R), U, T, T_mid)
    return n, out, status, toks, mlog, tlog, rounds


def multilevel_generate(om4, om2, prompt, n_generate, gamma, gamma2, T, T_mid, T2, uniforms, capacity):
    """Generate at least n_generate tokens; uniforms = (U2 [C][gamma][gamma2],
    R2 [C][gamma][gamma2], F2 [C][gamma], R [C][gamma], U [C]).  Returns
    (tokens[:n_generate], per-cycle n)."""
    from .cycle import prefill
    from .model import new_kv
    U2, R2, F2, R, U = uniforms
    kv = new_kv(om4, capacity)
    kv_len = prefill(om4, kv, prompt)
    committed = list(prompt)
    out, ns = [], []
    c = 0
    while len(out) < n_generate:
        n, emitted, *_ = multilevel_cycle(om4, om2, kv, kv_len, committed[-1], gamma, gamma2, T, T_mid, T2,
                                          U2[c], R2[c], F2[c], R[c], U[c])
        kv_len += n + 1
        committed += emitted
        out += emitted
        ns.append(n)
        c += 1
    return out[:n_generate], ns
