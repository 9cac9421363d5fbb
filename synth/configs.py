"""Model shapes and decode settings of the five synthetic workloads.

Shapes follow the decoder families the pages measure on: a Qwen2.5-7B-shaped
model for the SubSpec numbers (SubSpec report, section 3.2, Table 1), a
Qwen2.5-32B shape (same report, section 2.1) and a Llama-3.1-8B shape for the
long-context variant (SparseSpec-L blog, section 2).  All weights are
random-init; no checkpoint is read.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    ffn: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rope_theta: float
    rms_eps: float
    # layers [0, n_shared) keep their bf16 weights in the draft; the rest are
    # replaced by 4-bit group-64 substitutes.
    n_shared: int = 0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_params(self) -> int:
        h, f = self.hidden, self.ffn
        return self.qkv_rows * h + h * self.q_dim + 2 * f * h + h * f

    def with_(self, **kw) -> "ModelShape":
        return replace(self, **kw)


QWEN7B = ModelShape("qwen2.5-7b-shape", 28, 3584, 18944, 28, 4, 128, 152064,
                    1.0e6, 1e-6, n_shared=11)
QWEN32B = ModelShape("qwen2.5-32b-shape", 64, 5120, 27648, 40, 8, 128, 152064,
                     1.0e6, 1e-6, n_shared=0)
LLAMA8B = ModelShape("llama-3.1-8b-shape", 32, 4096, 14336, 32, 8, 128, 128256,
                     5.0e5, 1e-5, n_shared=0)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    gamma: int
    temp: float          # target temperature T (0 = greedy)
    draft_temp: float    # draft temperature T_d (0 = greedy)
    prompt: int
    generate: int
    extra: dict = field(default_factory=dict)


CONFIGS = {
    # one 512x512 linear + a V=1000, gamma=4 rejection step
    "tiny": Workload("tiny", QWEN7B.with_(n_layers=0, hidden=512, vocab=1000), 4, 1.0, 1.0, 0, 0,
                     {"gemv_n": 512, "gemv_k": 512}),
    # one 7B-shaped decoder layer, 4-bit draft vs bf16 verify of 17 positions, KV 1024
    "layer7b": Workload("layer7b", QWEN7B.with_(n_layers=1, n_shared=0), 16, 0.0, 0.0, 1024, 0),
    # full 28-layer 7B shape: 11 shared bf16 + 17 W4 substitutes, gamma 16
    "full7b": Workload("full7b", QWEN7B, 16, 0.0, 0.0, 512, 256),
    "full7b_sharp": Workload("full7b_sharp", QWEN7B, 16, 0.0, 0.2, 512, 256),
    # 64-layer 32B shape, all W4 substitutes, gamma 48, T = T_d = 0.6
    "full32b": Workload("full32b", QWEN32B, 48, 0.6, 0.6, 2048, 128),
    # long-context 8B shape with a gathered 10% KV index for the draft
    "longctx8b": Workload("longctx8b", LLAMA8B, 11, 0.0, 0.0, 60000, 128,
                          {"n_sink": 4, "n_recent": 64, "budget": 0.1, "budget_permille": 100, "window": 16}),
}


def shape_by_name(name: str) -> ModelShape:
    return {s.name: s for s in (QWEN7B, QWEN32B, LLAMA8B)}[name]
