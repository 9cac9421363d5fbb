"""The speculative cycle on one GPU ("How speculative decoding makes LLMs go
brrr", overall flow and pseudo-code): gamma draft steps, one verify pass over
gamma+1 positions, the rejection round, KV rollback.  Every step is a call
into libsubspec; this class only owns the device buffers and the call order.
State lives on the device (kv_len, tokens), so a cycle needs no host sync;
the host reads back the emitted tokens once per cycle.

With ``graphs`` a whole cycle (every kernel of the draft steps, the verify
pass, the rejection round, the rollback and the index rebuild) is recorded
once in a HIP graph and replayed: launch arguments are fixed and all state
lives on the device, so replays need no host work per kernel.  The first
cycle of each kind runs eagerly (it also warms the library's caches).

With ``sparse`` the draft reads a sparse KV index ("The second ledger of
speculative decoding", sections 3.1-3.2): every verify writes importance
scores, and after the rollback the index is rebuilt; the first cycle after
a reset drafts densely.

With ``adaptive`` the draft length follows the entropy controller of the
same blog's section 3.3: after every draft step the library measures the
token's entropy and decides on the device whether the draft goes on; later
steps skip themselves, the rejection round judges only the drafted tokens,
and the controller's class centres are updated from its outcome.  gamma is
then the longest draft.  With graphs the draft is recorded in segments of
1, 1, 2, 4, 8 ... steps and the host reads the device draft length after
each, so the segments past the stop are not launched.
"""
import torch

from . import _lib


class SpecDecoder:
    def __init__(self, model, capacity, gamma, temp=0.0, draft_temp=0.0, max_tokens=64,
                 device="cuda", sparse=None, graphs=False, adaptive=None):
        """``sparse``: None (dense drafting) or dict(n_sink, n_recent, window,
        budget_permille).  ``graphs``: replay recorded cycles (see above).
        ``adaptive``: None (fixed length gamma) or dict(c = C_d / C_v,
        beta = EMA rate)."""
        s = model.shape
        self.model = model
        self.gamma = gamma
        self.temp = float(temp)
        self.draft_temp = float(draft_temp)
        self.capacity = capacity
        self.max_tokens = max(max_tokens, gamma + 1)
        L, V = model.n_layers, s.vocab
        kv_shape = (L, s.n_kv_heads, capacity, s.head_dim)
        self.k_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.tokens = torch.zeros(gamma + 1, dtype=torch.int32, device=device)
        self.draft_logits = torch.zeros((max(gamma, 1), V), dtype=torch.bfloat16, device=device)
        self.target_logits = torch.zeros((gamma + 1, V), dtype=torch.bfloat16, device=device)
        self.n_accepted = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.zeros(gamma + 1, dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.probs = torch.zeros((max(gamma, 1), 2), dtype=torch.float32, device=device)
        self.prefill_tokens = torch.zeros(self.max_tokens, dtype=torch.int32, device=device)
        self._zero = torch.zeros(1, dtype=torch.int32, device=device)
        # fixed homes of a cycle's uniform codes (the recorded graph reads them)
        self.ud_buf = torch.zeros(max(gamma, 1), dtype=torch.int32, device=device)
        self.r_buf = torch.zeros(max(gamma, 1), dtype=torch.int32, device=device)
        self.uf_buf = torch.zeros(1, dtype=torch.int32, device=device)
        self.use_graphs = graphs
        self._graphs = {}
        self._warm = set()
        nbytes = _lib.workspace_bytes(model.c, self.max_tokens, capacity)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _lib.workspace_init(self.ws)
        self.c = _lib.State(self.k_cache.data_ptr(), self.v_cache.data_ptr(), capacity,
                            self.kv_len.data_ptr(), self.tokens.data_ptr(),
                            self.draft_logits.data_ptr(), gamma)
        self.adaptive = dict(adaptive) if adaptive else None
        self.ctl = None
        if self.adaptive:
            if sparse:
                raise ValueError("the adaptive draft length is built for dense drafting")
            self.draft_len = torch.full((1,), gamma, dtype=torch.int32, device=device)
            self.ctl_state = torch.zeros(8, dtype=torch.float64, device=device)
            self.entropy = torch.zeros(max(gamma, 1), dtype=torch.float32, device=device)
            self.ctl = _lib.Control(self.draft_len.data_ptr(), self.ctl_state.data_ptr(),
                                    self.entropy.data_ptr(), float(self.adaptive["c"]),
                                    float(self.adaptive.get("beta", 0.125)), gamma)
            self.c.draft_len = self.draft_len.data_ptr()
            _lib.control_init(self.ctl)
        self.sparse = dict(sparse) if sparse else None
        if self.sparse:
            sp = self.sparse
            self.index_cap = _lib.index_count(capacity, sp["n_sink"], sp["n_recent"],
                                              sp["budget_permille"])
            self.kv_score = torch.zeros((L, s.n_kv_heads, capacity), dtype=torch.float32, device=device)
            self.kv_index = torch.zeros((L, s.n_kv_heads, self.index_cap), dtype=torch.int32,
                                        device=device)
            self.kv_index_len = torch.zeros(1, dtype=torch.int32, device=device)
            c = self.c
            c.kv_score = self.kv_score.data_ptr()
            c.kv_index = self.kv_index.data_ptr()
            c.kv_index_len = self.kv_index_len.data_ptr()
            c.index_cap = self.index_cap
            c.use_index = 0
            c.n_sink, c.n_recent = sp["n_sink"], sp["n_recent"]
            c.score_window, c.budget_permille = sp["window"], sp["budget_permille"]

    # ------------------------------------------------------------ state
    def reset(self, kv_len, last_token):
        self.kv_len.fill_(int(kv_len))
        self.tokens[0] = int(last_token)
        self.c.use_index = 0  # the first cycle drafts densely

    def load_kv(self, k, v, kv_len, last_token):
        """Start from a given KV history (bf16 [L][Hkv][>= kv_len][d])."""
        n = k.shape[2]
        self.k_cache[:, :, :n].copy_(k)
        self.v_cache[:, :, :n].copy_(v)
        self.reset(kv_len, last_token)

    def prefill(self, prompt):
        """Run prompt[:-1] through the target (chunks of max_tokens positions);
        afterwards kv_len = len(prompt) - 1 and tokens[0] = prompt[-1]."""
        prompt = [int(t) for t in prompt]
        self.reset(0, prompt[-1])
        body = prompt[:-1]
        score = self.c.kv_score
        self.c.kv_score = None  # no importance scores for prefill chunks
        try:
            for c0 in range(0, len(body), self.max_tokens):
                chunk = body[c0:c0 + self.max_tokens]
                self.prefill_tokens[:len(chunk)] = torch.tensor(chunk, dtype=torch.int32)
                _lib.verify(self.model.c, self.c, len(chunk), self.prefill_tokens, None, self.ws)
                _lib.kv_advance(self.c, len(chunk))
        finally:
            self.c.kv_score = score

    # ------------------------------------------------------------ one cycle
    def _draft_steps(self, a, b, u_draft):
        for i in range(a, b):
            _lib.draft_step(self.model.c, self.c, i, self.draft_temp, u_draft, self.ws)
            if self.ctl is not None:
                _lib.draft_control(self.model.c, self.c, i, self.ctl, self.ws)

    def draft(self, u_draft=None):
        self._draft_steps(0, self.gamma, u_draft)

    def verify(self):
        _lib.verify(self.model.c, self.c, self.gamma + 1, self.tokens, self.target_logits, self.ws)

    def reject(self, r_codes=None, u_code=None):
        if self.ctl is not None:
            _lib.reject_len(self.gamma, self.model.shape.vocab, self.temp, self.draft_temp,
                            self.target_logits, self.draft_logits, self.tokens[1:], r_codes, u_code,
                            self.draft_len, self.n_accepted, self.out_tokens, self.status, self.probs, self.ws)
            _lib.control_update(self.ctl, self.n_accepted)
            return
        _lib.reject(self.gamma, self.model.shape.vocab, self.temp, self.draft_temp,
                    self.target_logits, self.draft_logits, self.tokens[1:], r_codes, u_code,
                    self.n_accepted, self.out_tokens, self.status, self.probs, self.ws)

    def last_draft_len(self):
        """Draft length of the last completed cycle (adaptive length only)."""
        return int(self.ctl_state[6].item())

    def commit(self):
        _lib.kv_rollback(self.c, self.n_accepted, self.out_tokens)
        if self.sparse:
            _lib.kv_select(self.model.c, self.c)
            self.c.use_index = 1

    def ar_step(self):
        """One plain autoregressive step of the draft model (a full-precision
        model when no layer is substituted): run tokens[0] at kv_len, draw
        tokens[1], then commit it (kv_len += 1, tokens[0] = tokens[1])."""
        _lib.draft_step(self.model.c, self.c, 0, self.draft_temp, None, self.ws)
        self._zero.zero_()
        _lib.kv_rollback(self.c, self._zero, self.tokens[1:])

    def _cycle_body(self, stochastic):
        self.draft(self.ud_buf if stochastic else None)
        self.verify()
        self.reject(self.r_buf if stochastic else None, self.uf_buf if stochastic else None)
        self.commit()

    def _replay(self, key, body):
        """body() eagerly the first time, recorded into a HIP graph the
        second, replayed from then on."""
        if key not in self._warm:
            body()
            self._warm.add(key)
            return
        g = self._graphs.get(key)
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                body()
            self._graphs[key] = g
        g.replay()

    def _segments(self):
        """Draft steps in segments [0, 1), [1, 2), [2, 4), [4, 8), ..."""
        segs, a, b = [], 0, 1
        while a < self.gamma:
            segs.append((a, min(b, self.gamma)))
            a, b = b, 2 * b
        return segs

    def _cycle_segmented(self, stochastic):
        """Adaptive length with graphs: the draft runs as recorded segments and
        the host reads the device draft length after each, so the segments
        after the controller's stop are not launched at all (they would only
        skip themselves); then verify, reject and commit as one graph."""
        u = self.ud_buf if stochastic else None
        for a, b in self._segments():
            self._replay(("draft", stochastic, a), lambda a=a, b=b: self._draft_steps(a, b, u))
            if b < self.gamma and int(self.draft_len.item()) <= b:
                break

        def tail():
            self.verify()
            self.reject(self.r_buf if stochastic else None, self.uf_buf if stochastic else None)
            self.commit()
        self._replay(("tail", stochastic), tail)

    def cycle(self, u_draft=None, r_codes=None, u_code=None):
        """One speculative cycle; uniform codes (device int32) are copied into
        the decoder's own buffers first."""
        stochastic = u_draft is not None or r_codes is not None or u_code is not None
        if stochastic:
            if u_draft is not None:
                self.ud_buf[:self.gamma].copy_(u_draft[:self.gamma])
            if r_codes is not None:
                self.r_buf[:self.gamma].copy_(r_codes[:self.gamma])
            if u_code is not None:
                self.uf_buf.copy_(u_code.reshape(-1)[:1])
        if self.use_graphs and self.ctl is not None:
            self._cycle_segmented(stochastic)
            return
        key = (stochastic, int(self.c.use_index))
        if not self.use_graphs or key not in self._warm:
            self._cycle_body(stochastic)
            self._warm.add(key)
            return
        g = self._graphs.get(key)
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._cycle_body(stochastic)
            self.c.use_index = key[1]  # the recorded commit set it on the host
            self._graphs[key] = g
        g.replay()
        if self.sparse:
            self.c.use_index = 1

    def generate(self, prompt, n_generate, uniforms=None, on_cycle=None):
        """Speculative decoding of at least n_generate tokens after ``prompt``.
        ``uniforms`` = (U_draft [C][gamma], R [C][gamma], U_final [C]) uint32
        device tensors, or None for greedy runs.  Returns (tokens, per-cycle n)."""
        kv = len(prompt) - 1
        if kv + self.gamma + 1 > self.capacity:
            raise ValueError(f"prompt of {len(prompt)} tokens leaves no room for a cycle of "
                             f"{self.gamma + 1} positions in a KV capacity of {self.capacity}")
        self.prefill(prompt)
        out, ns = [], []
        c = 0
        while len(out) < n_generate:
            # a cycle writes positions kv .. kv + gamma; stop before the cache
            # would overflow instead of letting rollback move past capacity
            if kv + self.gamma + 1 > self.capacity:
                raise ValueError(f"KV capacity {self.capacity} reached after {len(out)} of "
                                 f"{n_generate} tokens (kv_len {kv}, gamma {self.gamma})")
            if uniforms is not None:
                ud, rr, uf = uniforms
                self.cycle(ud[c], rr[c], uf[c:c + 1])
            else:
                self.cycle()
            n = int(self.n_accepted.item())
            out += self.out_tokens[:n + 1].tolist()
            ns.append(n)
            kv += n + 1
            if on_cycle:
                on_cycle(c, n)
            c += 1
        return out[:n_generate], ns


class TreeDecoder:
    """Speculative decoding with SubSpec's static deep/narrow token tree
    ("SubSpec" report, sections 6.3, 6.4 and 3.7): k chains of depth D share
    the root; one cycle drafts the tree level by level (all chains of a level
    in one pass over the draft weights), verifies all 1 + k D nodes in one
    target pass, judges the root by multi-step rejection and the accepted
    chain by the plain round, and moves that chain's K/V next to the prefix.
    Every step is a call into libsubspec; with ``graphs`` a whole cycle is
    recorded once and replayed."""

    def __init__(self, model, capacity, k, depth, temp=0.0, draft_temp=0.0, device="cuda", graphs=False):
        s = model.shape
        self.model = model
        self.k, self.depth = int(k), int(depth)
        self.temp, self.draft_temp = float(temp), float(draft_temp)
        self.capacity = capacity
        self.n_nodes = 1 + self.k * self.depth
        L, V = model.n_layers, s.vocab
        kv_shape = (L, s.n_kv_heads, capacity, s.head_dim)
        self.k_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.tokens = torch.zeros(self.n_nodes, dtype=torch.int32, device=device)
        self.draft_logits = torch.zeros((1 + self.k * (self.depth - 1), V), dtype=torch.bfloat16, device=device)
        self.target_logits = torch.zeros((self.n_nodes, V), dtype=torch.bfloat16, device=device)
        self.n_accepted = torch.zeros(1, dtype=torch.int32, device=device)
        self.chain = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.zeros(self.depth + 1, dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.max_tokens = 64
        self.prefill_tokens = torch.zeros(self.max_tokens, dtype=torch.int32, device=device)
        self.ud_buf = torch.zeros(self.k * self.depth, dtype=torch.int32, device=device)
        self.r_buf = torch.zeros(self.k + self.depth - 1, dtype=torch.int32, device=device)
        self.uf_buf = torch.zeros(1, dtype=torch.int32, device=device)
        nbytes = max(_lib.workspace_bytes(model.c, self.max_tokens, capacity),
                     _lib.tree_workspace_bytes(model.c, self.k, self.depth, capacity))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _lib.workspace_init(self.ws)
        self.c = _lib.State(self.k_cache.data_ptr(), self.v_cache.data_ptr(), capacity,
                            self.kv_len.data_ptr(), self.tokens.data_ptr(),
                            self.draft_logits.data_ptr(), self.depth)
        self.use_graphs = graphs
        self._graphs = {}
        self._warm = set()

    def reset(self, kv_len, last_token):
        self.kv_len.fill_(int(kv_len))
        self.tokens[0] = int(last_token)

    def load_kv(self, k, v, kv_len, last_token):
        n = k.shape[2]
        self.k_cache[:, :, :n].copy_(k)
        self.v_cache[:, :, :n].copy_(v)
        self.reset(kv_len, last_token)

    def prefill(self, prompt):
        prompt = [int(t) for t in prompt]
        self.reset(0, prompt[-1])
        body = prompt[:-1]
        for c0 in range(0, len(body), self.max_tokens):
            chunk = body[c0:c0 + self.max_tokens]
            self.prefill_tokens[:len(chunk)] = torch.tensor(chunk, dtype=torch.int32)
            _lib.verify(self.model.c, self.c, len(chunk), self.prefill_tokens, None, self.ws)
            _lib.kv_advance(self.c, len(chunk))

    # ------------------------------------------------------------ one cycle
    def draft(self, u_draft=None):
        for level in range(self.depth):
            _lib.tree_draft(self.model.c, self.c, self.k, self.depth, level, self.draft_temp, u_draft, self.ws)

    def verify(self):
        _lib.tree_verify(self.model.c, self.c, self.k, self.depth, self.target_logits, self.ws)

    def reject(self, r_codes=None, u_code=None):
        _lib.tree_reject(self.k, self.depth, self.model.shape.vocab, self.temp, self.draft_temp,
                         self.target_logits, self.draft_logits, self.tokens, r_codes, u_code, self.n_accepted,
                         self.chain, self.out_tokens, self.status, self.ws)

    def commit(self):
        _lib.tree_commit(self.model.c, self.c, self.k, self.depth, self.n_accepted, self.chain, self.out_tokens)

    def _cycle_body(self, stochastic):
        self.draft(self.ud_buf if stochastic else None)
        self.verify()
        self.reject(self.r_buf if stochastic else None, self.uf_buf if stochastic else None)
        self.commit()

    def cycle(self, u_draft=None, r_codes=None, u_code=None):
        stochastic = u_draft is not None or r_codes is not None or u_code is not None
        if stochastic:
            if u_draft is not None:
                self.ud_buf.copy_(u_draft[:self.ud_buf.numel()])
            if r_codes is not None:
                self.r_buf.copy_(r_codes[:self.r_buf.numel()])
            if u_code is not None:
                self.uf_buf.copy_(u_code.reshape(-1)[:1])
        if not self.use_graphs or stochastic not in self._warm:
            self._cycle_body(stochastic)
            self._warm.add(stochastic)
            return
        g = self._graphs.get(stochastic)
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._cycle_body(stochastic)
            self._graphs[stochastic] = g
        g.replay()

    def generate(self, prompt, n_generate, uniforms=None, on_cycle=None):
        """At least n_generate tokens after ``prompt``; ``uniforms`` =
        (U_draft [C][k D], R [C][k + D - 1], U [C]) device int32, or None
        (greedy).  Returns (tokens, per-cycle n)."""
        kv = len(prompt) - 1
        self.prefill(prompt)
        out, ns = [], []
        c = 0
        while len(out) < n_generate:
            if kv + self.n_nodes > self.capacity:
                raise ValueError(f"KV capacity {self.capacity} cannot hold another tree of {self.n_nodes} "
                                 f"nodes after kv_len {kv}")
            if uniforms is not None:
                ud, rr, uf = uniforms
                self.cycle(ud[c], rr[c], uf[c:c + 1])
            else:
                self.cycle()
            n = int(self.n_accepted.item())
            out += self.out_tokens[:n + 1].tolist()
            ns.append(n)
            kv += n + 1
            if on_cycle:
                on_cycle(c, n)
            c += 1
        return out[:n_generate], ns


class BatchDecoder:
    """B independent sequences decoded together on shared weights ("SubSpec"
    report, section 10.3, item 11: the substitutes serve several users): every
    draft step runs the B rows through the draft in one weight stream (4-bit
    layers on the matrix-core skinny GEMM), one verify pass covers the
    gamma + 1 positions of every sequence, and each sequence has its own
    rejection round and rollback.  Every step is a call into libsubspec; with
    ``graphs`` a whole cycle is recorded once and replayed."""

    def __init__(self, model, batch, capacity, gamma, temp=0.0, draft_temp=0.0, device="cuda", graphs=False):
        s = model.shape
        self.model = model
        self.batch, self.gamma = int(batch), int(gamma)
        self.temp, self.draft_temp = float(temp), float(draft_temp)
        self.capacity = capacity
        L, V, B = model.n_layers, s.vocab, self.batch
        self.k_cache = torch.zeros((L, B, s.n_kv_heads, capacity, s.head_dim), dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros_like(self.k_cache)
        self.kv_len = torch.zeros(B, dtype=torch.int32, device=device)
        self.tokens = torch.zeros((B, gamma + 1), dtype=torch.int32, device=device)
        self.draft_logits = torch.zeros((B, max(gamma, 1), V), dtype=torch.bfloat16, device=device)
        self.target_logits = torch.zeros((B, gamma + 1, V), dtype=torch.bfloat16, device=device)
        self.n_accepted = torch.zeros(B, dtype=torch.int32, device=device)
        self.out_tokens = torch.zeros((B, gamma + 1), dtype=torch.int32, device=device)
        self.status = torch.zeros(B, dtype=torch.int32, device=device)
        self.zeros = torch.zeros(B, dtype=torch.int32, device=device)
        self.chunk = max(1, min(64, 512 // B))
        self.prefill_tokens = torch.zeros((B, self.chunk), dtype=torch.int32, device=device)
        self.ud_buf = torch.zeros((B, max(gamma, 1)), dtype=torch.int32, device=device)
        self.r_buf = torch.zeros((B, max(gamma, 1)), dtype=torch.int32, device=device)
        self.uf_buf = torch.zeros(B, dtype=torch.int32, device=device)
        nbytes = _lib.batch_workspace_bytes(model.c, B, max(gamma + 1, self.chunk), capacity)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _lib.workspace_init(self.ws)
        self.c = _lib.BatchState(self.k_cache.data_ptr(), self.v_cache.data_ptr(), capacity, B,
                                 self.kv_len.data_ptr(), self.tokens.data_ptr(), self.draft_logits.data_ptr(), gamma)
        self.use_graphs = graphs
        self._graphs = {}
        self._warm = set()

    def reset(self, kv_len, last_tokens):
        self.kv_len.copy_(torch.as_tensor(kv_len, dtype=torch.int32).expand(self.batch))
        self.tokens[:, 0] = torch.as_tensor(last_tokens, dtype=torch.int32)

    def prefill(self, prompts):
        """prompts: B token lists of one length P; afterwards kv_len = P - 1
        and tokens[b][0] = prompts[b][-1]."""
        P = len(prompts[0])
        if any(len(p) != P for p in prompts):
            raise ValueError("batched prefill takes prompts of one length")
        self.reset(0, [p[-1] for p in prompts])
        body = torch.tensor([list(p[:-1]) for p in prompts], dtype=torch.int32)
        for c0 in range(0, P - 1, self.chunk):
            n = min(self.chunk, P - 1 - c0)
            self.prefill_tokens[:, :n].copy_(body[:, c0:c0 + n])
            _lib.batch_verify(self.model.c, self.c, n, self.prefill_tokens, self.chunk, None, self.ws)
            _lib.batch_rollback(self.c, None, None, n)

    def draft(self, u_draft=None):
        for i in range(self.gamma):
            _lib.batch_draft_step(self.model.c, self.c, i, self.draft_temp, u_draft, self.ws)

    def verify(self):
        _lib.batch_verify(self.model.c, self.c, self.gamma + 1, self.tokens, self.gamma + 1, self.target_logits, self.ws)

    def reject(self, r_codes=None, u_codes=None):
        _lib.batch_reject(self.model.c, self.c, self.temp, self.draft_temp, self.target_logits, r_codes, u_codes,
                          self.n_accepted, self.out_tokens, self.status, self.ws)

    def commit(self):
        _lib.batch_rollback(self.c, self.n_accepted, self.out_tokens)

    def ar_step(self):
        """One plain autoregressive step of every sequence on the draft
        weights (the target itself when nothing is substituted): step 0 of the
        draft, then kv_len += 1 and tokens[b][0] = tokens[b][1]."""
        _lib.batch_draft_step(self.model.c, self.c, 0, self.draft_temp, None, self.ws)
        _lib.batch_rollback(self.c, self.zeros, self.tokens[:, 1:])

    def _cycle_body(self, stochastic):
        self.draft(self.ud_buf if stochastic else None)
        self.verify()
        self.reject(self.r_buf if stochastic else None, self.uf_buf if stochastic else None)
        self.commit()

    def cycle(self, u_draft=None, r_codes=None, u_codes=None):
        stochastic = u_draft is not None or r_codes is not None or u_codes is not None
        if stochastic:
            if u_draft is not None:
                self.ud_buf.copy_(u_draft)
            if r_codes is not None:
                self.r_buf.copy_(r_codes)
            if u_codes is not None:
                self.uf_buf.copy_(u_codes)
        if not self.use_graphs or stochastic not in self._warm:
            self._cycle_body(stochastic)
            self._warm.add(stochastic)
            return
        g = self._graphs.get(stochastic)
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._cycle_body(stochastic)
            self._graphs[stochastic] = g
        g.replay()

    def generate(self, prompts, n_generate, uniforms=None):
        """At least n_generate tokens for every sequence; ``uniforms`` =
        (U_draft [C][B][gamma], R [C][B][gamma], U [C][B]) device int32, or
        None (greedy).  Returns (per-sequence tokens, per-cycle n lists)."""
        kv = len(prompts[0]) - 1
        self.prefill(prompts)
        outs = [[] for _ in range(self.batch)]
        ns = []
        c = 0
        lens = [kv] * self.batch
        while min(len(o) for o in outs) < n_generate:
            if max(lens) + self.gamma + 1 > self.capacity:
                raise ValueError(f"KV capacity {self.capacity} reached")
            if uniforms is not None:
                self.cycle(uniforms[0][c], uniforms[1][c], uniforms[2][c])
            else:
                self.cycle()
            n = self.n_accepted.tolist()
            out = self.out_tokens.tolist()
            for b in range(self.batch):
                outs[b] += out[b][:n[b] + 1]
                lens[b] += n[b] + 1
            ns.append(n)
            c += 1
        return [o[:n_generate] for o in outs], ns


class MultiLevelDecoder:
    """Multi-level substitutes ("SubSpec" report, section 10.3, item 9): the
    4-bit draft's gamma tokens come from inner rounds in which a model with
    2-bit substitutes drafts up to gamma2 tokens, the 4-bit draft runs them
    in one pass and the plain round keeps the accepted ones plus one drawn
    token; the bf16 target then verifies the gamma tokens with q = their
    4-bit logits.  All levels share one KV cache.  Every step is a call into
    libsubspec; the host reads each inner round's length (one sync a round)."""

    def __init__(self, model4, model2, capacity, gamma, gamma2, temp=0.0, mid_temp=0.0, draft_temp=0.0,
                 device="cuda"):
        s = model4.shape
        self.m4, self.m2 = model4, model2
        self.gamma, self.gamma2 = int(gamma), int(gamma2)
        self.temp, self.mid_temp, self.draft_temp = float(temp), float(mid_temp), float(draft_temp)
        self.capacity = capacity
        L, V = model4.n_layers, s.vocab
        g_all = self.gamma + self.gamma2
        kv_shape = (L, s.n_kv_heads, capacity, s.head_dim)
        self.k_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros(kv_shape, dtype=torch.bfloat16, device=device)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.tokens = torch.zeros(g_all + 1, dtype=torch.int32, device=device)
        self.inner_logits = torch.zeros((g_all, V), dtype=torch.bfloat16, device=device)  # 2-bit, by step
        self.mid_logits = torch.zeros((g_all + 1, V), dtype=torch.bfloat16, device=device)  # 4-bit, by position
        self.target_logits = torch.zeros((self.gamma + 1, V), dtype=torch.bfloat16, device=device)
        self.n_accepted = torch.zeros(1, dtype=torch.int32, device=device)
        self.out_tokens = torch.zeros(self.gamma + 1, dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.in_n = torch.zeros(1, dtype=torch.int32, device=device)
        self.in_out = torch.zeros(self.gamma2 + 1, dtype=torch.int32, device=device)
        self.in_status = torch.zeros(1, dtype=torch.int32, device=device)
        self.probs = torch.zeros((max(g_all, 1), 2), dtype=torch.float32, device=device)
        self.u2_buf = torch.zeros(g_all, dtype=torch.int32, device=device)
        self.r2_buf = torch.zeros(max(self.gamma2, 1), dtype=torch.int32, device=device)
        self.f2_buf = torch.zeros(1, dtype=torch.int32, device=device)
        self.r_buf = torch.zeros(max(self.gamma, 1), dtype=torch.int32, device=device)
        self.uf_buf = torch.zeros(1, dtype=torch.int32, device=device)
        self.max_tokens = 64
        self.prefill_tokens = torch.zeros(self.max_tokens, dtype=torch.int32, device=device)
        nbytes = _lib.workspace_bytes(model4.c, self.max_tokens, capacity)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _lib.workspace_init(self.ws)
        ptrs = (self.k_cache.data_ptr(), self.v_cache.data_ptr(), capacity, self.kv_len.data_ptr(),
                self.tokens.data_ptr())
        self.c = _lib.State(*ptrs, self.mid_logits.data_ptr(), g_all)
        self.c2 = _lib.State(*ptrs, self.inner_logits.data_ptr(), g_all)
        self.rounds = []  # (base, drafted, n, status) of the last cycle's inner rounds

    def reset(self, kv_len, last_token):
        self.kv_len.fill_(int(kv_len))
        self.tokens[0] = int(last_token)

    def prefill(self, prompt):
        prompt = [int(t) for t in prompt]
        self.reset(0, prompt[-1])
        body = prompt[:-1]
        for c0 in range(0, len(body), self.max_tokens):
            chunk = body[c0:c0 + self.max_tokens]
            self.prefill_tokens[:len(chunk)] = torch.tensor(chunk, dtype=torch.int32)
            _lib.verify(self.m4.c, self.c, len(chunk), self.prefill_tokens, None, self.ws)
            _lib.kv_advance(self.c, len(chunk))

    # ------------------------------------------------------------ one cycle
    def inner_round(self, base, g):
        """Draft g tokens after middle token `base` with the 2-bit model, run
        the 4-bit draft over them, judge them; returns the round's n (host)."""
        stoch = self.draft_temp > 0
        for i in range(g):
            _lib.draft_step(self.m2.c, self.c2, base + i, self.draft_temp, self.u2_buf if stoch else None, self.ws)
        _lib.draft_verify(self.m4.c, self.c, base, g + 1, self.tokens[base:], self.mid_logits[base:], self.ws)
        stoch_p = self.mid_temp > 0
        _lib.reject(g, self.m4.shape.vocab, self.mid_temp, self.draft_temp, self.mid_logits[base:],
                    self.inner_logits[base:], self.tokens[base + 1:], self.r2_buf if stoch_p else None,
                    self.f2_buf if stoch_p else None, self.in_n, self.in_out, self.in_status, self.probs, self.ws)
        _lib.draft_append(self.c, base + 1, g, self.in_n, self.in_out)
        return int(self.in_n.item())

    def middle(self, cycle_uniforms=None):
        """The gamma middle tokens (tokens[1..gamma]) and their 4-bit logits
        (mid_logits[0..gamma)); cycle_uniforms = (U2 [gamma][gamma2],
        R2 [gamma][gamma2], F2 [gamma]) host int arrays, or None."""
        base, r = 0, 0
        self.rounds = []
        while base < self.gamma:
            g = min(self.gamma2, self.gamma - base)
            if cycle_uniforms is not None:
                U2, R2, F2 = cycle_uniforms
                self.u2_buf[base:base + g] = torch.as_tensor(U2[r][:g], dtype=torch.int32)
                self.r2_buf[:g] = torch.as_tensor(R2[r][:g], dtype=torch.int32)
                self.f2_buf[0] = int(F2[r])
            n = self.inner_round(base, g)
            self.rounds.append((base, g, n, int(self.in_status.item())))
            base += min(n + 1, self.gamma - base)
            r += 1

    def verify(self):
        _lib.verify(self.m4.c, self.c, self.gamma + 1, self.tokens, self.target_logits, self.ws)

    def reject(self, r_codes=None, u_code=None):
        _lib.reject(self.gamma, self.m4.shape.vocab, self.temp, self.mid_temp, self.target_logits, self.mid_logits,
                    self.tokens[1:], r_codes, u_code, self.n_accepted, self.out_tokens, self.status, self.probs,
                    self.ws)

    def commit(self):
        _lib.kv_rollback(self.c, self.n_accepted, self.out_tokens)

    def cycle(self, cycle_uniforms=None):
        """cycle_uniforms = (U2, R2, F2, R [gamma], U) host int arrays, or None."""
        self.middle(None if cycle_uniforms is None else cycle_uniforms[:3])
        self.verify()
        if cycle_uniforms is not None and self.temp > 0:
            self.r_buf[:self.gamma] = torch.as_tensor(cycle_uniforms[3][:self.gamma], dtype=torch.int32)
            self.uf_buf[0] = int(cycle_uniforms[4])
            self.reject(self.r_buf, self.uf_buf)
        else:
            self.reject()
        self.commit()

    def generate(self, prompt, n_generate, uniforms=None):
        """uniforms = (U2 [C][gamma][gamma2], R2, F2 [C][gamma], R [C][gamma],
        U [C]) host int arrays, or None (greedy)."""
        kv = len(prompt) - 1
        self.prefill(prompt)
        out, ns = [], []
        c = 0
        while len(out) < n_generate:
            if kv + self.gamma + self.gamma2 + 1 > self.capacity:
                raise ValueError(f"KV capacity {self.capacity} reached")
            self.cycle(None if uniforms is None else tuple(u[c] for u in uniforms))
            n = int(self.n_accepted.item())
            out += self.out_tokens[:n + 1].tolist()
            ns.append(n)
            kv += n + 1
            c += 1
        return out[:n_generate], ns
