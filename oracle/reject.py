"""O5: one verification round - accept, residual resample, bonus token.

[SD] pseudo-code and Module 3: for i = 1..gamma, draft token x_i is accepted
when r_i < min(1, p_i(x_i) / q_i(x_i)); at the first rejection every later
draft is dropped and one token is drawn from norm(max(0, p_i - q_i)); when all
gamma are accepted one bonus token is drawn from p_{gamma+1}.  Every round
therefore emits between 1 and gamma+1 tokens.  Greedy verification (T = 0,
[SSR] section 3.2, Table 1) makes p one-hot at the target argmax.

Readings where the pages are silent:
  * q_i is the distribution the draft token was actually drawn from, i.e. the
    sharpened softmax(z_d / T_d) (one-hot at the draft argmax when T_d = 0);
    this is the only reading under which the round stays lossless.
  * r_i and u are caller-given uniforms R_i / 2**24 and U / 2**24; one u
    serves the residual draw or the bonus draw, whichever happens.
  * Exact arithmetic: with the integer weights of oracle.sampling,
    p_i(x)/q_i(x) = (Wt_x * Sd) / (Wd_x * St), so the test
    r < p/q  <=>  R * Wd_x * St < 2**24 * Wt_x * Sd  is decided on integers.
  * Residual: D_j = max(0, Wt_j * Sd - Wd_j * St) >> (bitlength(Sd) - 1),
    i.e. max(0, p - q) up to the positive factor St*Sd, kept to 41 bits; it
    is sampled with the same inverse CDF.  If its total is 0 the token is
    drawn from p instead and status bit 2 is set.
  * status bit 1: a non-finite logit in a row that was read (such logits
    carry no probability, see oracle.sampling); bit 4: a draft token with
    q(x) = 0 (then it is accepted iff p(x) > 0).
  * A draft token outside [0, V) (the device marks a draft step it had to
    skip with -1) has q(x) = p(x) = 0: it is rejected, with status bit 4,
    at any temperature.
  * A draw whose total weight is 0 (residual and p both without mass, i.e.
    a target row with no finite logit) gives token 0.

Pinned by: q = p gives n = gamma; greedy gives the longest prefix of draft
tokens equal to the target argmax; at least one token per round; exact
enumeration over tiny vocabularies (first token distributed as p_1,
P(n >= m) = prod_{i<=m} sum_x min(p_i, q_i)); a chi-square test on V = 8.
"""
import numpy as np

from .sampling import argmax_lowest, fixed_weights, inverse_cdf, UNIFORM_BITS

STATUS_NONFINITE = 1
STATUS_ZERO_RESIDUAL = 2
STATUS_Q_ZERO = 4


def _draft_weights(zd, x, draft_temp):
    """Integer weights of q and their sum (one-hot at the draft argmax if T_d = 0)."""
    if draft_temp == 0:
        W = np.zeros(np.asarray(zd).shape[0], dtype=np.int64)
        W[argmax_lowest(zd)] = 1
        return W, 1
    return fixed_weights(zd, draft_temp)


def residual_weights(Wt, St, Wd, Sd):
    """max(0, p - q) scaled by St*Sd and shifted to 41 bits, as int64."""
    shift = max(int(Sd).bit_length() - 1, 0)
    out = np.zeros(len(Wt), dtype=np.int64)
    for j in range(len(Wt)):
        d = int(Wt[j]) * int(Sd) - int(Wd[j]) * int(St)
        if d > 0:
            out[j] = d >> shift
    return out


def accept_test(R, Wt_x, St, Wd_x, Sd):
    """r < p(x)/q(x) decided exactly on integers."""
    return int(R) * int(Wd_x) * int(St) < (int(Wt_x) * int(Sd)) << UNIFORM_BITS


def reject(target_logits, draft_logits, draft_tokens, R, U, temp, draft_temp):
    """Run one round.

    target_logits [gamma+1][V], draft_logits [gamma][V] (bf16 values),
    draft_tokens [gamma], R [gamma] and U: uniform codes in [0, 2**24).
    Returns (n_accepted, tokens emitted (length n+1), status).
    """
    zt = np.asarray(target_logits, dtype=np.float32)
    zd = np.asarray(draft_logits, dtype=np.float32)
    gamma = len(draft_tokens)
    status = 0
    n = gamma
    V = zt.shape[1]
    for i in range(gamma):
        x = int(draft_tokens[i])
        if not np.all(np.isfinite(zt[i])) or not np.all(np.isfinite(zd[i])):
            status |= STATUS_NONFINITE
        if not 0 <= x < V:
            status |= STATUS_Q_ZERO
            ok = False
        elif temp == 0:
            ok = x == argmax_lowest(zt[i])
        else:
            Wt, St = fixed_weights(zt[i], temp)
            Wd, Sd = _draft_weights(zd[i], x, draft_temp)
            if Wd[x] == 0:
                status |= STATUS_Q_ZERO
            ok = accept_test(R[i], Wt[x], St, Wd[x], Sd)
        if not ok:
            n = i
            break
    row = zt[n]
    if not np.all(np.isfinite(row)):
        status |= STATUS_NONFINITE
    if temp == 0:
        y = argmax_lowest(row)
    else:
        Wt, St = fixed_weights(row, temp)
        if n < gamma:
            Wd, Sd = _draft_weights(zd[n], int(draft_tokens[n]), draft_temp)
            D = residual_weights(Wt, St, Wd, Sd)
            if D.sum() > 0:
                y = inverse_cdf(D, U)
            else:
                status |= STATUS_ZERO_RESIDUAL
                y = inverse_cdf(Wt, U)
        else:
            y = inverse_cdf(Wt, U)
    out = [int(t) for t in draft_tokens[:n]] + [int(y)]
    return n, out, status


def acceptance_probabilities(target_logits, draft_logits, draft_tokens, temp, draft_temp):
    """Float64 p_i(x_i) and q_i(x_i) of each draft token (for reporting)."""
    from .sampling import softmax_f64
    p = [softmax_f64(target_logits[i], temp)[int(x)] for i, x in enumerate(draft_tokens)]
    q = [softmax_f64(draft_logits[i], draft_temp)[int(x)] for i, x in enumerate(draft_tokens)]
    return np.array(p), np.array(q)
