"""O7: sparse-KV drafting - importance scores, index selection, gathered
draft attention.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[SSL] section 3.1: while drafting, every layer and attention head reads only
an index of about a tenth of the positions - a few sink positions at the
start, a few recent positions at the end, and the remaining budget filled
with the positions of highest importance - gathered from the dense cache.
[SSL] section 3.2: the importance of a past position is the attention the
most recent W = 16 query positions of the verify pass gave it (the verify
pass computes dense attention anyway); the cache itself is never pruned, and
the index is rebuilt from fresh statistics after every verify.

Readings (where the page leaves a step open):
  * GQA: one index per KV head; its score sums the probabilities of the
    query heads that share the KV head.
  * Window: the verify pass's last min(W, rows) rows (a gamma + 1 = 12 row
    pass contributes all of its rows); the scores are rebuilt, not carried.
  * Index over the committed positions [0, L), L = kv_len after rollback:
    sink = [0, n_sink), recent = [L - n_recent, L), and from the middle
    [n_sink, L - n_recent) the K = ceil(budget * L) - n_sink - n_recent
    positions of highest score (score descending, position ascending on
    ties), K clipped to [0, middle size).  The budget is given in thousandths
    so that ceil() is exact integer arithmetic.  The index is ascending.
  * The draft step at position p attends to the index plus the speculative
    positions [L, p] (its own fresh draft K/V).
  * The first cycle (no verify yet) drafts densely.

Pinned by: scores of one row and head summing to 1 (the window's scores
summing to rows x group), the one-hot-V identity (attention output equals
the probability vector), uniform probabilities for a zero query, the
characterisation of top-K (every chosen middle position outranks every
unchosen one, in (score desc, position asc) order), full budget giving the
dense draft exactly, and a gathered attention equal to dense attention on
the compacted cache.  Parity with the pages is otherwise unpinned: they
print no worked example.
"""
import numpy as np


def attention_probs(q, K, n_keys):
    """softmax over positions [0, n_keys) of (K q) / sqrt(d), float64."""
    q = np.asarray(q, dtype=np.float64)
    logits = np.asarray(K[:n_keys], dtype=np.float64) @ q / np.sqrt(q.shape[0])
    w = np.exp(logits - np.max(logits))
    return w / np.sum(w)


def index_bounds(L, n_sink, n_recent, budget_permille):
    """(sink end, recent start, K): sink = [0, s), recent = [r, L), and K
    middle positions chosen from [s, r)."""
    s = min(n_sink, L)
    r = max(s, L - n_recent)
    total = -(-budget_permille * L // 1000)  # ceil(budget * L), exact
    K = min(max(total - s - (L - r), 0), r - s)
    return s, r, K


def select_index(score, L, n_sink, n_recent, budget_permille):
    """Ascending positions of the draft index over committed positions [0, L)."""
    s, r, K = index_bounds(L, n_sink, n_recent, budget_permille)
    score = np.asarray(score, dtype=np.float64)
    middle = sorted(range(s, r), key=lambda j: (-score[j], j))
    chosen = sorted(middle[:K])
    return np.array(list(range(s)) + chosen + list(range(r, L)), dtype=np.int64)


def build_index(scores, L, n_sink, n_recent, budget_permille):
    """index[l][hk] for every layer and KV head from per-layer scores."""
    return [[select_index(sc[hk], L, n_sink, n_recent, budget_permille) for hk in range(sc.shape[0])]
            for sc in scores]
