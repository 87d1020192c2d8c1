"""Named synthetic decode workloads for the Slow-Fast Inference (SFI) decode path.

Each workload fixes the attention shape (batch, query/KV heads, head dim, storage dtype),
the context length, the decode-trajectory length, the sparse-memory sizes (sink, recent
window, selected K) and the Selector knobs.  The shapes follow the Qwen3-family models
the pages evaluate on (Slow-Fast Inference pages: "Resultados Principales" /
"Résultats Expérimentaux" / "实验结果"); the sink / recent / selected split follows the
fast-step memory description ("Pasos Rápidos", "Étapes Rapides", "2.1 慢快推理框架");
the Selector knobs (lambda, soft-NMS, cross-head exclusivity) follow "2.2 Selector".

This module holds sizes and knobs only: no arithmetic of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int            # independent sequences
    layers: int           # attention layers, each with its own KV
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # storage dtype of K/V: "bf16" or "f32"
    context: int          # KV length before the first decode step
    steps: int            # decode steps in the trajectory
    n_sink: int
    n_recent: int         # recent window W
    top_k: int            # selected positions per KV head
    p_boundary: float     # Bernoulli probability of a semantic-boundary flag per step
    refresh_budget: int   # max consecutive fast steps
    n_topics: int         # topic positions per query span
    key_scale_sigma: float  # per-position key scale ~ LogNormal(0, sigma)
    query_noise: float    # std of per-step query noise
    nms_radius: int
    alpha_soft: float
    alpha_cross: float
    lam: float
    page_size: int = 16
    evidence_window: int = 1  # decode queries whose attention the Selector pools
    sliding_recent: bool = False  # recent segment = newest W positions at every step
    lambda_clip: float = -1.0  # < 0: fusion weight lam; in [0, 1]: adaptive, clipped here
    nms_greedy: bool = False   # greedy soft-NMS instead of the one-pass reading

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_len(self) -> int:
        """KV positions generated: context plus one appended token per decode step."""
        return self.context + self.steps

    @property
    def pages_per_seq(self) -> int:
        return -(-self.total_len // self.page_size)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def seq_len(self, step: int) -> int:
        """KV length N_s at decode step s; position N_s-1 is the current token."""
        return self.context + step

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_SEL = dict(nms_radius=4, alpha_soft=0.5, alpha_cross=0.5, lam=0.3, query_noise=0.1)

WORKLOADS: Dict[str, Workload] = {
    # one tiny fp32 layer: 4 q heads / 2 KV heads, head_dim 64, 1K context, 16 steps
    "tiny_fp32_1k": Workload(
        name="tiny_fp32_1k", batch=1, layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
        dtype="f32", context=1024, steps=16, n_sink=4, n_recent=64, top_k=128,
        p_boundary=0.10, refresh_budget=8, n_topics=8, key_scale_sigma=0.5, **_SEL),
    # Qwen3-0.6B-shaped layer: 16/8 heads, head_dim 128, bf16, 8K context, 256 steps
    "qwen3_0p6b_8k": Workload(
        name="qwen3_0p6b_8k", batch=1, layers=1, num_q_heads=16, num_kv_heads=8, head_dim=128,
        dtype="bf16", context=8192, steps=256, n_sink=4, n_recent=256, top_k=1024,
        p_boundary=0.05, refresh_budget=32, n_topics=32, key_scale_sigma=0.5, **_SEL),
    # Qwen3-4B-shaped layer: 32/8 heads, batch 4, 32K context, 512 steps
    "qwen3_4b_32k_b4": Workload(
        name="qwen3_4b_32k_b4", batch=4, layers=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", context=32768, steps=512, n_sink=4, n_recent=512, top_k=4096,
        p_boundary=0.05, refresh_budget=32, n_topics=64, key_scale_sigma=0.7, **_SEL),
    # Qwen3-4B-shaped full stack: 36 layers, batch 1, 128K context, 256 steps
    "qwen3_4b_128k_36l": Workload(
        name="qwen3_4b_128k_36l", batch=1, layers=36, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", context=131072, steps=256, n_sink=4, n_recent=1024,
        top_k=19456, p_boundary=0.05, refresh_budget=32, n_topics=64, key_scale_sigma=0.7,
        **_SEL),
    # large-model-shaped layer: 64/4 heads (group 16), batch 8, 64K context, dense boundaries
    "g16_64k_b8": Workload(
        name="g16_64k_b8", batch=8, layers=1, num_q_heads=64, num_kv_heads=4, head_dim=128,
        dtype="bf16", context=65536, steps=256, n_sink=4, n_recent=512, top_k=9830,
        p_boundary=0.15, refresh_budget=16, n_topics=128, key_scale_sigma=0.7,
        **dict(_SEL, nms_radius=8)),
}

ORDER: List[str] = ["tiny_fp32_1k", "qwen3_0p6b_8k", "qwen3_4b_32k_b4",
                    "qwen3_4b_128k_36l", "g16_64k_b8"]

# Workload whose throughput the benchmark reports: the 128K-context 36-layer stack.
BENCH_WORKLOAD = "qwen3_4b_128k_36l"


def get(name: str) -> Workload:
    return WORKLOADS[name]
