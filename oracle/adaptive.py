"""Entropy-adaptive draft length.  TEST INFRASTRUCTURE ONLY (see
oracle/__init__.py).

[SSL] section 3.3: the acceptance rate drifts with the task and the stage of
generation, so a fixed draft length loses either way.  Every draft token
records the entropy H_i of its output distribution; after verification it is
known whether the token was accepted; an exponential moving average keeps the
mean entropy of accepted tokens (H_acc) and of rejected tokens (H_rej) as two
class centres; a new draft token is classified softly by its distances to the
two centres, giving an acceptance probability p_i and, for a draft of length
k, the expected output sum_{m=1..k} prod_{i<=m} p_i; the controller picks the
candidate length of highest expected efficiency,
    k* = argmax_k (1 + sum_{m=1..k} prod_{i=1..m} p_i) / (k C_d + C_v).
Low entropy (a confident draft) bets long; a spike of uncertainty cuts the
draft short at once.

Readings (the page leaves these steps open):
  R1 entropy: H_i = -sum_j q_j ln q_j with q = softmax of the draft logits at
     temperature 1 (the model's own output distribution, whatever temperature
     the token is drawn at); non-finite logits carry no probability.
  R2 centres: EMA with rate beta (default 1/8): H <- H + beta (H_i - H); a
     centre starts at the first entropy of its class.
  R3 soft class: p_i = d_rej / (d_acc + d_rej) with d = |H_i - centre|; 1/2
     when both distances are 0; p_i = 1 while either centre is unseen.
  R4 online use: tokens are drafted one at a time and p_i exists only after
     token i.  After token i the draft goes on iff some longer candidate
     k > i, with the tokens not yet drafted forecast at p_i, is more
     efficient than stopping at i: E_f(k) > E(i).  The round's draft length
     gamma_eff is the i where it stops (at most gamma_max); every drafted
     token is verified.
  R5 candidates: every length 1 .. gamma_max.
  R6 costs: c = C_d / C_v is given (the caller measures its own draft step
     and verify pass); E(k) = (1 + sum_{m<=k} P_m) / (k c + 1), P_m the
     running product.
  R7 updates: after the rejection round with n accepted, tokens 1..n update
     H_acc in order and token n+1, if it was drafted (n < gamma_eff), updates
     H_rej; later tokens were never judged and update nothing.
  Arithmetic: float64, in the order written below, so that the decisions
  are reproducible from the same entropies (the device controller runs the
  same operations in the same order).

Pinned by: the entropy of a uniform row (ln V), of a one-hot row (0) and of a
two-valued row (closed form); the soft class at and between the centres; the
stop rule against brute force over every length when all p are equal
(the first-order condition of S(k) = (alpha k + 1)/(k c + 1) of [SSL]
section 1: with p = 1 the longest draft wins when c < 1), the stop on a
spike; the EMA closed form; and greedy adaptive speculative decoding equal
to greedy autoregressive decoding (oracle/cycle.py).
"""
import numpy as np

BETA = 0.125


def entropy(z):
    """-sum q ln q of softmax(z) at temperature 1, float64 (non-finite logits
    excluded; 0 for a row with no finite logit)."""
    z = np.asarray(z, dtype=np.float64)
    z = z[np.isfinite(z)]
    if z.size == 0:
        return 0.0
    e = np.exp(z - z.max())
    S = e.sum()
    q = e / S
    nz = q > 0
    return float(-(q[nz] * np.log(q[nz])).sum())


class Controller:
    """The class centres and the state of the round being drafted."""

    def __init__(self, gamma_max, c, beta=BETA):
        self.gamma_max = int(gamma_max)
        self.c = float(c)
        self.beta = float(beta)
        self.h_acc = 0.0
        self.h_rej = 0.0
        self.seen_acc = False
        self.seen_rej = False
        self.start_round()

    def start_round(self):
        self.P = 1.0       # prod_{i<=m} p_i of the tokens drafted so far
        self.A = 1.0       # 1 + sum_m P_m
        self.gamma_eff = self.gamma_max
        self.H = []

    def p_of(self, h):
        """Soft acceptance probability of a token of entropy h (R3)."""
        if not (self.seen_acc and self.seen_rej):
            return 1.0
        da = abs(h - self.h_acc)
        dr = abs(h - self.h_rej)
        if da + dr == 0.0:
            return 0.5
        return dr / (da + dr)

    def after_token(self, h):
        """Token i = len(H) + 1 was drafted with entropy h: returns True iff
        the draft goes on (R4); sets gamma_eff when it stops."""
        h = float(h)
        self.H.append(h)
        i = len(self.H)
        p = self.p_of(h)
        self.P = self.P * p
        self.A = self.A + self.P
        if i >= self.gamma_max:
            self.gamma_eff = self.gamma_max
            return False
        e_stop = self.A / (i * self.c + 1.0)
        P, A = self.P, self.A
        go = False
        for k in range(i + 1, self.gamma_max + 1):
            P = P * p
            A = A + P
            if A / (k * self.c + 1.0) > e_stop:
                go = True
                break
        if not go:
            self.gamma_eff = i
        return go

    def _ema(self, centre, seen, h):
        if not seen:
            return h
        return centre + self.beta * (h - centre)

    def after_round(self, n):
        """Rejection round done with n accepted (R7); starts the next round."""
        for i in range(min(n, len(self.H))):
            self.h_acc = self._ema(self.h_acc, self.seen_acc, self.H[i])
            self.seen_acc = True
        if n < self.gamma_eff and n < len(self.H):
            self.h_rej = self._ema(self.h_rej, self.seen_rej, self.H[n])
            self.seen_rej = True
        self.start_round()
