"""Layer configurations for the synthetic FlexPrefill workloads.

Each entry describes one attention layer's causal prefill: the attention
shape (batch, query heads, key/value heads, sequence length, head dim),
the input precision, the method's hyper-parameters (block size, cumulative
threshold gamma, divergence threshold tau, minimum budget in tokens) and
the mix of planted head types the generator in ``synth.workload`` builds.

The shapes stand in for the models the FlexPrefill pages evaluate
(Llama-3.1-8B: 32 query / 8 key-value heads, head dim 128; GLM-4-9B: 32 / 2)
at the pages' headline context of 128k tokens ("Key results" on the
atlas.scime.ai summary page).  The hyper-parameter values are the ones the
pages' ablation table lists as defaults (gamma 0.95, tau 0.1, minimum budget
1024 tokens, block 128) and the variants it tests (gamma 0.9, block 64,
minimum budget 2048).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

# Head types planted by the generator.
VERTICAL, SLASH, QUERY_AWARE, NOISE = "V", "S", "QA", "N"
HEAD_TYPES = (VERTICAL, SLASH, QUERY_AWARE, NOISE)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str            # "fp32" or "bf16": the input and output precision
    block: int
    gamma: float
    tau: float
    min_budget: int
    # Head-type fractions (V, S, QA, N) or an explicit per-head tuple.
    mix: Tuple[float, float, float, float] = (0.4, 0.3, 0.2, 0.1)
    explicit_types: Tuple[str, ...] = ()
    sinks: int = 16
    slash_width: int = 1
    seed: int = 20250
    note: str = field(default="", compare=False)

    @property
    def nb(self) -> int:
        return self.N // self.block

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = [
    LayerConfig("tiny_fp32_4k", B=1, Hq=4, Hkv=4, N=4096, d=128, dtype="fp32",
                block=128, gamma=0.95, tau=0.1, min_budget=1024,
                explicit_types=(VERTICAL, SLASH, QUERY_AWARE, NOISE),
                seed=20250,
                note="tiny CPU-checkable layer, one head of each planted type"),
    LayerConfig("llama8b_32k", B=1, Hq=32, Hkv=8, N=32768, d=128, dtype="bf16",
                block=128, gamma=0.95, tau=0.1, min_budget=1024, seed=20251,
                note="Llama-3.1-8B-shaped layer, 32k context"),
    LayerConfig("llama8b_128k", B=1, Hq=32, Hkv=8, N=131072, d=128, dtype="bf16",
                block=128, gamma=0.95, tau=0.1, min_budget=1024, seed=20252,
                note="Llama-3.1-8B-shaped layer, 128k context (headline point)"),
    LayerConfig("llama8b_128k_sparse", B=1, Hq=32, Hkv=8, N=131072, d=128,
                dtype="bf16", block=128, gamma=0.9, tau=0.1, min_budget=1024,
                sinks=64, slash_width=4, seed=20253,
                note="gamma 0.9, 64 sinks, slash width 4"),
    LayerConfig("glm9b_64k_bs64", B=1, Hq=32, Hkv=2, N=65536, d=128, dtype="bf16",
                block=64, gamma=0.95, tau=0.1, min_budget=2048,
                mix=(0.25, 0.1875, 0.5, 0.0625),
                seed=20254,
                note="GLM-4-9B-shaped layer, block 64, half the heads query-aware"),
]

BY_NAME = {c.name: c for c in CONFIGS}
HEADLINE = BY_NAME["llama8b_128k"]
