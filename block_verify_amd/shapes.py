"""Decoder shapes and run configurations of the block-verify workloads.

The shapes are the Qwen2.5-shaped random-init decoders the workloads name
(tiny, 0.5B, 1.5B, 7B).  Architectural details the pages leave open are read
as the plainest Qwen2-style decoder: pre-norm RMSNorm (eps 1e-6, unit gain),
rotate-half RoPE with theta 1e6, no biases, SwiGLU MLP, untied LM head.

Nothing in this module computes any part of the method; it only names sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def tensor_specs(self):
        """Canonical tensor list: (name, shape, kind).

        Order: embed; per layer [attn_norm, wq, wk, wv, wo, mlp_norm, wgate,
        wup, wdown]; final_norm; lm_head.  Linear weights are [out, in]
        row-major, as every decoder checkpoint stores them.
        """
        H, F, V = self.hidden, self.ffn, self.vocab
        specs = [("embed", (V, H), "embed")]
        for l in range(self.n_layers):
            specs += [
                (f"l{l}.attn_norm", (H,), "norm"),
                (f"l{l}.wq", (self.q_dim, H), "linear"),
                (f"l{l}.wk", (self.kv_dim, H), "linear"),
                (f"l{l}.wv", (self.kv_dim, H), "linear"),
                (f"l{l}.wo", (H, self.q_dim), "linear"),
                (f"l{l}.mlp_norm", (H,), "norm"),
                (f"l{l}.wgate", (F, H), "linear"),
                (f"l{l}.wup", (F, H), "linear"),
                (f"l{l}.wdown", (H, F), "linear"),
            ]
        specs += [("final_norm", (H,), "norm"), ("lm_head", (V, H), "linear")]
        return specs

    def n_params(self) -> int:
        n = 0
        for _, shp, _ in self.tensor_specs():
            p = 1
            for s in shp:
                p *= s
            n += p
        return n

    def weight_bytes_bf16(self) -> int:
        return 2 * self.n_params()

    def kv_bytes_per_token(self) -> int:
        """bf16 K and V of every layer for one position."""
        return 2 * 2 * self.n_layers * self.kv_dim


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 1024, 4096)
QWEN_1_5B = ModelShape("qwen2.5-1.5b-shape", 28, 1536, 12, 2, 128, 8960, 151936)
QWEN_0_5B = ModelShape("qwen2.5-0.5b-shape", 24, 896, 14, 2, 64, 4864, 151936)
QWEN_7B = ModelShape("qwen2.5-7b-shape", 28, 3584, 28, 4, 128, 18944, 152064)

SHAPES = {s.name: s for s in (TINY, QWEN_1_5B, QWEN_0_5B, QWEN_7B)}

# Seeds of the synthetic inputs.
SEED_TARGET = 0
SEED_CORRUPT = 1
SEED_NOISE = 2
SEED_PHILOX = 3
SEED_DRAFT = 10
SEED_PROMPT = 20


@dataclass(frozen=True)
class RunConfig:
    """One workload: a target (and optionally a draft), a prompt, a draft source."""
    name: str
    target: ModelShape
    prompt_len: int
    n_new: int
    k: int
    mode: str = "greedy"            # "greedy" | "stochastic"
    draft_source: str = "table"     # "table" | "model" | "noisy_self" | "q4_self"
    corrupt_p: float = 0.0          # per-position replacement probability of the table
    draft: ModelShape | None = None  # independent draft model (own cache)
    prefill_chunk: int = 2048
    depth: int = 0                  # sequential draft depth D (q4 draft), 0 = k
    notes: dict = field(default_factory=dict)


CONFIGS = [
    RunConfig("tiny", TINY, 128, 16, 4, corrupt_p=0.4),
    RunConfig("1.5b-2k", QWEN_1_5B, 2048, 64, 4, corrupt_p=0.46),
    RunConfig("1.5b-8k+0.5b-draft", QWEN_1_5B, 8192, 64, 4, corrupt_p=0.51,
              draft_source="model", draft=QWEN_0_5B),
    RunConfig("1.5b-4k-stochastic", QWEN_1_5B, 4096, 64, 4, mode="stochastic",
              draft_source="noisy_self"),
    RunConfig("7b-2k-q4-draft", QWEN_7B, 2048, 64, 8, draft_source="q4_self", depth=8),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}
