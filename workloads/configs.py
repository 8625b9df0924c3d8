"""The five seeded RLT replay workloads (model shape + batch shape).

Shapes follow the configurations the build is measured on.  Where a prompt
split is not given it is taken as T/2; the split never changes replay outputs
(prompt/response split invariance, Proposition 3.1 on the feinterview page
"普林斯顿提出 RLT：跨 Token 携带解码器状态的循环 Transformer", model-RL co-design
principle) and is used only by split-invariance tests.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelConfig:
    vocab: int
    d_model: int
    n_heads: int
    n_layers: int          # L_E = L_D (encoder and decoder layers are tied pairwise)
    ffn_dim: int
    ffn_kind: str          # "gelu" or "swiglu"
    window: int            # W >= 1, includes the current token; W-1 cached entries
    mem_groups: int        # G: 1 (shared memory) or n_layers (one per decoder layer)
    dtype: str             # "fp32" or "bf16" (bf16 storage, fp32 accumulate)
    norm_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int             # 1..5; weights seed = index, tokens seed = 100 + index
    model: ModelConfig
    batch: int             # B independent sequences
    seq_len: int           # T
    prompt_len: int        # prompt/response split (tests only)
    token_dist: str        # "uniform" or "zipf1.1"

    @property
    def weight_seed(self) -> int:
        return self.index

    @property
    def token_seed(self) -> int:
        return 100 + self.index


CONFIGS = {
    "tiny": Workload(
        "tiny", 1,
        ModelConfig(vocab=256, d_model=64, n_heads=4, n_layers=2, ffn_dim=256,
                    ffn_kind="gelu", window=8, mem_groups=1, dtype="fp32"),
        batch=4, seq_len=64, prompt_len=32, token_dist="uniform"),
    "small": Workload(
        "small", 2,
        ModelConfig(vocab=512, d_model=64, n_heads=4, n_layers=4, ffn_dim=256,
                    ffn_kind="gelu", window=32, mem_groups=4, dtype="bf16"),
        batch=64, seq_len=1024, prompt_len=512, token_dist="uniform"),
    "300m": Workload(
        "300m", 3,
        ModelConfig(vocab=32000, d_model=1024, n_heads=16, n_layers=12, ffn_dim=4096,
                    ffn_kind="swiglu", window=128, mem_groups=12, dtype="bf16"),
        batch=512, seq_len=2048, prompt_len=1024, token_dist="zipf1.1"),
    "ref48": Workload(
        "ref48", 4,
        ModelConfig(vocab=32000, d_model=2048, n_heads=16, n_layers=48, ffn_dim=5632,
                    ffn_kind="swiglu", window=256, mem_groups=1, dtype="bf16"),
        batch=64, seq_len=4096, prompt_len=3072, token_dist="zipf1.1"),
    "long": Workload(
        "long", 5,
        ModelConfig(vocab=32000, d_model=1024, n_heads=16, n_layers=48, ffn_dim=2816,
                    ffn_kind="swiglu", window=512, mem_groups=1, dtype="bf16"),
        batch=16, seq_len=32768, prompt_len=16384, token_dist="zipf1.1"),
}


def get_workload(name: str) -> Workload:
    return CONFIGS[name]
