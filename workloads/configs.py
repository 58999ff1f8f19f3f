"""The five workload shapes of the verification step.

Shapes follow the workloads the source pages discuss: a Llama-3-8B-shaped
layer (32 query / 8 KV heads, head dim 128, vocabulary 128256, [SD]
"Heterogeneous Vocabulary Alignment"), an EAGLE-style static tree (60 total
tokens), the SPEED-Bench Throughput Split ISL buckets 1k..32k at batch 1..256
with three entropy levels, and ECHO's high-concurrency super-tree (vocabulary
151936, batch 256). Synthetic data stands in for every dataset.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    index: int              # 1-based config number, used in seeds
    B: int
    tree: str               # 'chain' | 'eagle60' | 'super'
    K: int                  # chain length (chain), or total nodes (super)
    Hq: int
    Hkv: int
    D: int
    dtype: str              # 'f32' | 'bf16' (Q/K/V element type)
    L: int                  # committed context per request
    V: int
    logit_sigma: float      # target logits ~ N(0, sigma^2)
    draft_sigma: float      # draft logits = target + N(0, draft_sigma^2)
    temperature: float
    max_T: int = 64         # super-tree: largest per-request tree
    bucket: int = 0         # C4 bucket index (seed offset)
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.index + self.bucket * 0x100

    @property
    def lib_seed(self) -> int:
        return 0xC0FFEE + self.index + self.bucket * 0x100


CONFIGS = {
    "c1_tiny_chain": WorkloadConfig("c1_tiny_chain", 1, B=1, tree="chain", K=4, Hq=1, Hkv=1, D=64, dtype="f32",
                                    L=128, V=1000, logit_sigma=2.0, draft_sigma=0.5, temperature=1.0),
    "c2_llama8b_chain": WorkloadConfig("c2_llama8b_chain", 2, B=8, tree="chain", K=5, Hq=32, Hkv=8, D=128,
                                       dtype="bf16", L=2048, V=128256, logit_sigma=3.0, draft_sigma=1.0,
                                       temperature=1.0),
    "c3_eagle_tree": WorkloadConfig("c3_eagle_tree", 3, B=16, tree="eagle60", K=60, Hq=32, Hkv=8, D=128,
                                    dtype="bf16", L=4096, V=128256, logit_sigma=3.0, draft_sigma=0.7,
                                    temperature=1.0),
    "c5_super_tree": WorkloadConfig("c5_super_tree", 5, B=256, tree="super", K=2048, Hq=64, Hkv=4, D=128,
                                    dtype="bf16", L=4096, V=151936, logit_sigma=3.0, draft_sigma=1.0,
                                    temperature=1.0, max_T=32),
}

# Throughput buckets: ISL in {1k, 2k, 8k, 16k, 32k} x batch {1, 8, 32} x temperature
# {0.5, 1, 2} (entropy levels), K = 3 chain, Llama-8B attention shape.
C4_BUCKETS = []
_i = 0
for _L in (1024, 2048, 8192, 16384, 32768):
    for _B in (1, 8, 32):
        for _T in (0.5, 1.0, 2.0):
            C4_BUCKETS.append(WorkloadConfig(f"c4_L{_L}_B{_B}_T{_T:g}", 4, B=_B, tree="chain", K=3, Hq=32, Hkv=8,
                                             D=128, dtype="bf16", L=_L, V=128256, logit_sigma=3.0,
                                             draft_sigma=1.0, temperature=_T, bucket=_i))
            _i += 1
for _c in C4_BUCKETS:
    CONFIGS[_c.name] = _c


def get_config(name: str) -> WorkloadConfig:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    return CONFIGS[name]


def scaled(cfg: WorkloadConfig, **overrides) -> WorkloadConfig:
    """A copy of cfg with some sizes replaced (smaller cases for oracle-speed parity)."""
    return dataclasses.replace(cfg, **overrides)
