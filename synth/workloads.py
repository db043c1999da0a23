"""The five synthetic decode workloads, with the shapes of the Prism Attention
kernel and end-to-end measurements (arXiv 2610.22985, Section 5.3 and
Appendix D, Tables 6-8: Qwen3/Llama-class GQA models, head dimension 128,
sparse budgets of 1K-4K tokens, contexts up to 128K).

A workload fixes shapes and the seed namespace only.  Nothing here computes
any part of the attention method itself.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                      # seed namespace; distinct per workload
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_layers: int
    anchor_stride: int            # layer l is an anchor (proposal) layer iff l % stride == 0
    kappa: int                    # sparse budget per KV head
    window: int                   # +-w neighbourhood used by refined layers
    rope_base: float
    context: Optional[int] = None               # fixed context length for every sequence
    len_range: Optional[Tuple[int, int]] = None  # else lengths drawn uniformly in this range
    lengths: Optional[Tuple[int, ...]] = None    # else these exact lengths (one per sequence)
    planted: bool = False         # sink tokens + query-aligned drifting clusters
    n_sinks: int = 4
    sink_scale: float = 4.0
    n_clusters: int = 64
    cluster_len: int = 32
    cluster_cos: float = 0.6
    drift: int = 16
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def is_anchor(self, layer: int) -> bool:
        return layer % self.anchor_stride == 0

    def anchor_of(self, layer: int) -> int:
        """The nearest preceding anchor layer (itself for an anchor)."""
        return layer - (layer % self.anchor_stride)


TINY_4K = Workload(
    name="tiny-4k-gqa4", wid=1, batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
    page_size=64, num_layers=2, anchor_stride=2, kappa=256, window=16, rope_base=10000.0,
    context=4096,
    note="batch 1, 2 layers (anchor, refined), 8q/2kv, ctx 4096, kappa 256, w 16, RoPE base 1e4",
)

LLAMA_32K = Workload(
    name="llama3-8b-32k", wid=2, batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
    page_size=64, num_layers=32, anchor_stride=8, kappa=2048, window=32, rope_base=500000.0,
    context=32768,
    note="Llama-3-8B-shaped, batch 1, 32 layers, anchor every 8, ctx 32768, kappa 2048, w 32",
)

LLAMA_128K_PLANTED = Workload(
    name="llama3-8b-128k-planted", wid=3, batch=1, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=64, num_layers=32, anchor_stride=8, kappa=2048, window=32,
    rope_base=500000.0, context=131072, planted=True,
    note="as llama3-8b-32k at ctx 131072 with 4 sinks and 64 drifting query-aligned clusters",
)

BATCHED_16 = Workload(
    name="batched-16x8k-64k", wid=4, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
    page_size=64, num_layers=32, anchor_stride=4, kappa=1024, window=16, rope_base=500000.0,
    len_range=(8192, 65536),
    note="batch 16, lengths U[8192, 65536] rounded to 64, anchor every 4, kappa 1024, w 16",
)

LONG_4x128K = Workload(
    name="long-4x128k-gqa8", wid=5, batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
    page_size=64, num_layers=80, anchor_stride=8, kappa=4096, window=64, rope_base=500000.0,
    context=131072, planted=True,
    note="batch 4, ctx 131072, 64q/8kv (GQA 8), 80 layers, anchor every 8, kappa 4096, w 64, planted",
)

WORKLOADS = (TINY_4K, LLAMA_32K, LLAMA_128K_PLANTED, BATCHED_16, LONG_4x128K)
BY_NAME = {w.name: w for w in WORKLOADS}


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (used for small test cases)."""
    d = {k: getattr(wl, k) for k in wl.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)
