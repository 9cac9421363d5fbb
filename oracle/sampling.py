"""O4: temperature softmax weights, argmax and inverse-CDF sampling.

[SD] pseudo-code and Module 1: the drafter samples each candidate from its own
distribution q and hands q(x) to the verifier; [SSR] sections 2.2 and 3.4
(Table 5): the SubSpec draft samples from a sharpened distribution
(temperature 0.2).  The pages do not say how a token is drawn from a
distribution; the reading used here is the inverse CDF in ascending vocabulary
order with a caller-given uniform, defined so that the decision is exact:

  * M = max_j z_j over the (bf16) logits of the row;
  * w_j = exp(fl32(fl32(z_j - M) / T)) evaluated in float32;
  * W_j = floor(w_j * 2**40), an integer (so every sum below is exact);
  * with a uniform u = U / 2**24 (U an integer in [0, 2**24)), the token is
    the smallest j with C_j > floor(U * S / 2**24), where C is the inclusive
    prefix sum of W and S = C_{V-1}.
  * T = 0 means greedy: the token is the argmax, lowest index on ties.

Non-finite logits (the pages never meet them; reading): a NaN or +-Inf logit
carries no probability and never wins the argmax, so a row samples exactly
like the row with those entries removed.  M is the largest finite logit.  A
row with no finite logit has no mass at all; its argmax and every draw from
it are token 0 (the deterministic fallback).  The rejection round reports
such rows in its status word.

Pinned by: a chi-square test of the sampled frequencies against softmax(z/T)
computed in float64, the exact interval lengths of the inverse CDF on tiny
vocabularies, and the tie rule of the argmax.
"""
import numpy as np

FIX_BITS = 40
UNIFORM_BITS = 24


def argmax_lowest(z):
    """Index of the largest finite value; the lowest index wins ties; 0 when
    no value is finite."""
    z = np.asarray(z)
    best = None
    for j in range(z.shape[0]):
        if np.isfinite(z[j]) and (best is None or z[j] > z[best]):
            best = j
    return 0 if best is None else best


def tempered_weights_f32(z, temp):
    """w_j = exp((z_j - M) / T), every operation in float32, M the largest
    finite logit; non-finite logits get w_j = 0."""
    z = np.asarray(z, dtype=np.float32)
    finite = np.isfinite(z)
    if not finite.any():
        return np.zeros(z.shape, dtype=np.float32)
    m = z[finite].max()
    zf = np.where(finite, z, m).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        t = ((zf - m).astype(np.float32) / np.float32(temp)).astype(np.float32)
        w = np.exp(t).astype(np.float32)
    return np.where(finite, w, np.float32(0.0)).astype(np.float32)


def fixed_point(w):
    """floor(w * 2**40) as int64 (w in [0, 1])."""
    return np.floor(np.asarray(w, dtype=np.float64) * float(1 << FIX_BITS)).astype(np.int64)


def fixed_weights(z, temp):
    """(W, S): integer weights of softmax(z / T) and their exact sum."""
    W = fixed_point(tempered_weights_f32(z, temp))
    return W, int(W.sum())


def inverse_cdf(W, U):
    """Smallest j with C_j > floor(U * S / 2**24); W non-negative integers.
    A zero total weight (a row without finite logits) gives token 0."""
    W = np.asarray(W, dtype=np.int64)
    if (W < 0).any():
        raise ValueError("inverse_cdf needs non-negative weights")
    S = int(W.sum())
    if S == 0:
        return 0
    th = (int(U) * S) >> UNIFORM_BITS
    C = np.cumsum(W)
    return int(np.searchsorted(C, th, side="right"))


def sample(z, temp, U):
    """Draw one token from softmax(z / T) with uniform code U (greedy if T == 0)."""
    if temp == 0:
        return argmax_lowest(z)
    W, _ = fixed_weights(z, temp)
    return inverse_cdf(W, U)


def softmax_f64(z, temp):
    """Plain float64 softmax(z / T); used for reporting probabilities."""
    z = np.asarray(z, dtype=np.float64)
    p = np.zeros_like(z)
    finite = np.isfinite(z)
    if temp == 0 or not finite.any():
        p[argmax_lowest(z)] = 1.0 if finite.any() else 0.0
        return p
    e = np.exp((z[finite] - z[finite].max()) / temp)
    p[finite] = e / e.sum()
    return p
