"""O9: the static deep/narrow token tree (k chains of depth D).

[SSR] section 6.3: SubSpec keeps SpecInfer's token-tree verification (every
path of the tree verified by one target forward) but shapes the tree deep and
narrow, k = 6 and D = 48; section 6.4: the tree is static (a fixed shape, in
place of EAGLE-2's context-dependent tree); section 3.7: D = 48.

Reading (the pages give only the width k and the depth D, no topology): the
static tree of width k and depth D is k chains that share the root.  The root
is the last committed token; chain c in [0, k) holds one node at each depth
d in [1, D].  Node numbers, cache slots and positions:

    t = 0                       root          slot kv_len       position kv_len
    t = 1 + c D + (d - 1)       chain c, d    slot kv_len + t   position kv_len + d

Node t attends to the slots [0, kv_len] (the committed prefix and the root)
and to the slots of its own chain up to itself - exactly what it would see if
its chain were decoded as a plain sequence.  With k = 1 the tree is the chain
of the plain speculative cycle (gamma = D).

Drafting: level 0 runs the root through the draft; its distribution gives the
k depth-1 tokens: the k largest logits when T_d = 0 (lowest index first on
ties), or k independent draws from q_root when T_d > 0 (SpecInfer's children
are samples of the draft distribution).  Level d = 1..D-1 runs the k depth-d
nodes at once; each chain's depth-(d+1) token is drawn from that chain's own
distribution (its argmax when T_d = 0).

Verification: one target forward over all 1 + k D nodes with the visibility
above.  The root is judged by SpecInfer's multi-step speculative sampling:
the depth-1 children are tested in chain order, child c accepted when
r_c < p_c(x_c) / q_c(x_c), with p_0 = p_root and, after a rejection,
p_{c+1} = norm(max(0, p_c - q_c)); if every child is rejected one token is
drawn from the last p_c and the round ends.  q_c is q_root (sampled children)
or, for children chosen greedily (T_d = 0), the one-hot distribution at x_c
(the chain reading of reject.py: q one-hot at the draft's choice), under
which the residual is p_c with x_c removed - both keep the round lossless.
Greedy verification (T = 0) accepts the first child equal to the target's
argmax at the root.  After the root, the accepted chain's depth-2..D tokens
are judged by the chain rule of reject.py against the target rows of its
depth-1..D nodes and the draft rows of its depth-1..D-1 nodes.

Readings where the pages are silent (integer arithmetic as in reject.py):
  * the residual of a multi-step round is taken again from the previous
    residual, max(0, W S_d - W_d S) shifted right by bitlength(S_d) - 1 when
    W are p_root's own weights (below 2^40, the shift of reject.py) and by
    one bit more when W is already a residual (below 2^41), so every weight
    stays below 2^41 and every sum below 2^59; a residual without mass is
    replaced by p_root (status bit 2) and the round goes on;
  * a child outside [0, V) is skipped: not tested, the residual unchanged,
    status bit 4;
  * with fewer than k finite logits at the root, the greedy children past
    the finite ones are token 0;
  * uniforms: U_draft [k D] - root draw c is U_draft[c], chain c's draw at
    level d is U_draft[k + c (D - 1) + d - 1]; R [k + D - 1] - R[c] tests
    child c, R[k + i] the chain's i-th test; U the one final draw.

Commit: the accepted chain's first n nodes hold the committed K/V; they move
to the slots kv_len + 1 .. kv_len + n, and kv_len += n + 1 (the cycle's
convention: the last emitted token is the next input).

Pinned by: k = 1 equal to the plain cycle (every temperature pair); each
node's logits equal a plain forward of its path; greedy tree decoding equal to
greedy autoregressive decoding; the first emitted token distributed as p_root
(exact enumeration over children, accept uniforms and the final draw); the
committed K/V equal to those of autoregressive decoding; top-k brute force.
"""
import numpy as np

from .bf16 import round_bf16
from .model import rmsnorm, linear, project, rope, silu, attend
from .reject import (reject, residual_weights, accept_test, STATUS_NONFINITE, STATUS_Q_ZERO,
                     STATUS_ZERO_RESIDUAL)
from .sampling import argmax_lowest, fixed_weights, inverse_cdf, sample


def node(c, d, D):
    """Node number of chain c at depth d (d >= 1)."""
    return 1 + c * D + (d - 1)


def depth(t, D):
    return 0 if t == 0 else (t - 1) % D + 1


def chain_of(t, D):
    return -1 if t == 0 else (t - 1) // D


def n_nodes(k, D):
    return 1 + k * D


def visible_slots(t, kv_len, D):
    """Cache slots node t attends to, ascending."""
    own = [] if t == 0 else list(range(kv_len + 1 + chain_of(t, D) * D, kv_len + t + 1))
    return list(range(kv_len + 1)) + own


def tree_forward(model, kv, kv_len, nodes, tokens, D, draft=False, logit_rows=None, acc=np.float64):
    """Run the listed tree nodes (with their tokens) through the decoder.

    Node t is embedded from its token, rotated at position kv_len + depth(t),
    writes its K/V to slot kv_len + t and attends to visible_slots(t).  All
    listed nodes write their K/V before any of them attends (one pass, as the
    verifier runs it).  Returns the logits of the rows in ``logit_rows``
    (all rows by default) as [len(logit_rows)][V].
    """
    K, Vc = kv
    n = len(nodes)
    Hq, Hkv, d = model.n_q_heads, model.n_kv_heads, model.head_dim
    group = Hq // Hkv
    h = np.stack([np.asarray(model.embed[t], dtype=np.float64) for t in tokens])
    for l in range(model.n_layers):
        lw = model.layers[l]
        x = rmsnorm(h, lw["attn_norm"], model.rms_eps)
        qkv = linear(x, model.weight(l, "qkv", draft), acc)
        for j, t in enumerate(nodes):
            pos, slot = kv_len + depth(t, D), kv_len + t
            for hk in range(Hkv):
                k = qkv[j, (Hq + hk) * d:(Hq + hk + 1) * d]
                v = qkv[j, (Hq + Hkv + hk) * d:(Hq + Hkv + hk + 1) * d]
                K[l, hk, slot] = round_bf16(rope(k, pos, model.rope_theta))
                Vc[l, hk, slot] = v
        attn = np.zeros((n, Hq * d))
        for j, t in enumerate(nodes):
            pos = kv_len + depth(t, D)
            keys = np.asarray(visible_slots(t, kv_len, D), dtype=np.int64)
            for hq in range(Hq):
                q = round_bf16(rope(qkv[j, hq * d:(hq + 1) * d], pos, model.rope_theta))
                hk = hq // group
                attn[j, hq * d:(hq + 1) * d] = attend(q, K[l, hk][keys], Vc[l, hk][keys], len(keys))
        attn = round_bf16(attn)
        h = round_bf16(h + project(attn, model.weight(l, "o", draft), acc))
        x = rmsnorm(h, lw["ffn_norm"], model.rms_eps)
        gu = linear(x, model.weight(l, "gate_up", draft), acc)
        F = model.ffn
        act = round_bf16(silu(gu[:, :F]) * gu[:, F:])
        h = round_bf16(h + project(act, model.weight(l, "down", draft), acc))
    rows = list(range(n)) if logit_rows is None else list(logit_rows)
    if not rows:
        return np.zeros((0, model.vocab))
    x = rmsnorm(h[rows], model.final_norm, model.rms_eps)
    return linear(x, model.lm_head, acc)


def top_k_lowest(z, k):
    """The k largest finite values' indices, larger first, lower index first
    on ties; positions past the number of finite values are token 0."""
    z = np.asarray(z)
    finite = [j for j in range(z.shape[0]) if np.isfinite(z[j])]
    order = sorted(finite, key=lambda j: (-float(z[j]), j))
    out = order[:k]
    return out + [0] * (k - len(out))


def root_children(z, k, draft_temp, U):
    """The k depth-1 tokens from the root's draft logits."""
    z = np.asarray(z, dtype=np.float32)
    if draft_temp == 0:
        return top_k_lowest(z, k)
    W, _ = fixed_weights(z, draft_temp)
    return [inverse_cdf(W, U[c]) for c in range(k)]


def draft_tree(model, kv, kv_len, root_token, k, D, draft_temp, U_draft, acc=np.float64):
    """Draft the whole tree: returns (node tokens [1 + k D], draft logits
    [1 + k (D - 1)][V]: row 0 the root, row 1 + c (D - 1) + d - 1 chain c's
    depth-d node)."""
    tokens = np.zeros(n_nodes(k, D), dtype=np.int64)
    tokens[0] = int(root_token)
    dlogits = np.zeros((1 + k * (D - 1), model.vocab))
    z0 = tree_forward(model, kv, kv_len, [0], [tokens[0]], D, draft=True, acc=acc)[0]
    dlogits[0] = z0
    for c, x in enumerate(root_children(z0, k, draft_temp, U_draft[:k])):
        tokens[node(c, 1, D)] = x
    for d in range(1, D):
        nodes = [node(c, d, D) for c in range(k)]
        z = tree_forward(model, kv, kv_len, nodes, [tokens[t] for t in nodes], D, draft=True, acc=acc)
        for c in range(k):
            dlogits[1 + c * (D - 1) + d - 1] = z[c]
            u = U_draft[k + c * (D - 1) + d - 1]
            tokens[node(c, d + 1, D)] = sample(z[c].astype(np.float32), draft_temp, u)
    return tokens, dlogits


def _residual(W, S, Wd, Sd, from_p):
    """max(0, p_c - q) as weights below 2^41: residual_weights' shift for p's
    own weights (below 2^40), one bit more for a residual (below 2^41)."""
    if from_p:
        return residual_weights(W, S, Wd, Sd)
    shift = max(int(Sd).bit_length() - 1, 0) + 1
    out = np.zeros(len(W), dtype=np.int64)
    for j in range(len(W)):
        d = int(W[j]) * int(Sd) - int(Wd[j]) * int(S)
        if d > 0:
            out[j] = d >> shift
    return out


def _onehot(V, x):
    W = np.zeros(V, dtype=np.int64)
    W[x] = 1
    return W, 1


def tree_reject(tlogits, dlogits, tokens, k, D, R, U, temp, draft_temp):
    """Judge one tree.  tlogits [1 + k D][V] (node order), dlogits
    [1 + k (D - 1)][V], tokens [1 + k D], R [k + D - 1], U.
    Returns (n accepted, emitted tokens (n + 1), status, accepted chain or -1)."""
    zt = np.asarray(tlogits, dtype=np.float32)
    zd = np.asarray(dlogits, dtype=np.float32)
    V = zt.shape[1]
    status = 0
    if not np.all(np.isfinite(zt[0])) or not np.all(np.isfinite(zd[0])):
        status |= STATUS_NONFINITE
    xs = [int(tokens[node(c, 1, D)]) for c in range(k)]
    chosen = -1
    if temp == 0:
        y = argmax_lowest(zt[0])
        for c, x in enumerate(xs):
            if not 0 <= x < V:
                status |= STATUS_Q_ZERO
                continue
            if x == y:
                chosen = c
                break
    else:
        Wp, Sp = fixed_weights(zt[0], temp)
        W, S = Wp, Sp
        for c, x in enumerate(xs):
            if not 0 <= x < V:
                status |= STATUS_Q_ZERO
                continue
            Wd, Sd = _onehot(V, x) if draft_temp == 0 else fixed_weights(zd[0], draft_temp)
            if Wd[x] == 0:
                status |= STATUS_Q_ZERO
            if accept_test(R[c], W[x], S, Wd[x], Sd):
                chosen = c
                break
            W = _residual(W, S, Wd, Sd, W is Wp)
            S = int(W.sum())
            if S == 0:
                status |= STATUS_ZERO_RESIDUAL
                W, S = Wp, Sp
        if chosen < 0:
            y = inverse_cdf(W, U)
    if chosen < 0:
        return 0, [int(y)], status, -1
    c = chosen
    t1 = node(c, 1, D)
    n, out, st = reject(zt[t1:t1 + D], zd[1 + c * (D - 1):1 + c * (D - 1) + D - 1],
                        [int(t) for t in tokens[t1 + 1:t1 + D]], list(R[k:k + D - 1]), U, temp, draft_temp)
    return 1 + n, [xs[c]] + out, status | st, c


def tree_commit(kv, kv_len, n, c, D):
    """Move the accepted chain's first n nodes' K/V to slots kv_len + 1 ..
    kv_len + n; returns the new kv_len."""
    K, Vc = kv
    for i in range(1, n + 1):
        src, dst = kv_len + node(c, i, D), kv_len + i
        if src != dst:
            K[:, :, dst] = K[:, :, src]
            Vc[:, :, dst] = Vc[:, :, src]
    return kv_len + n + 1


def tree_cycle(model, kv, kv_len, last_token, k, D, temp, draft_temp, U_draft, R, U, acc=np.float64):
    """Draft, verify, judge and commit one tree.  Returns (n, emitted tokens,
    status, chain, node tokens, draft logits, target logits, new kv_len)."""
    tokens, dlogits = draft_tree(model, kv, kv_len, last_token, k, D, draft_temp, U_draft, acc=acc)
    nodes = list(range(n_nodes(k, D)))
    tlogits = tree_forward(model, kv, kv_len, nodes, list(tokens), D, draft=False, acc=acc)
    n, out, status, c = tree_reject(tlogits, dlogits, tokens, k, D, R, U, temp, draft_temp)
    new_len = tree_commit(kv, kv_len, n, max(c, 0), D)
    return n, out, status, c, tokens, dlogits, tlogits, new_len


def tree_generate(model, prompt, n_generate, k, D, temp, draft_temp, uniforms, capacity):
    """Speculative decoding with the static tree; returns (tokens[:n_generate],
    per-cycle n).  uniforms = (U_draft [cycles][k D], R [cycles][k + D - 1],
    U [cycles])."""
    from .cycle import prefill
    from .model import new_kv
    U_draft, R, U = uniforms
    kv = new_kv(model, capacity)
    kv_len = prefill(model, kv, prompt)
    committed = list(prompt)
    out, ns = [], []
    c = 0
    while len(out) < n_generate:
        if kv_len + n_nodes(k, D) > capacity:
            raise ValueError("the KV capacity cannot hold another tree")
        n, emitted, _, _, _, _, _, kv_len = tree_cycle(model, kv, kv_len, committed[-1], k, D, temp,
                                                       draft_temp, U_draft[c], R[c], U[c])
        committed += emitted
        out += emitted
        ns.append(n)
        assert kv_len == len(committed) - 1
        c += 1
    return out[:n_generate], ns
