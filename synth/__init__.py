"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU oracle's
callers.  Input generation only: no part of the attention method lives here."""
from .workloads import (Workload, WORKLOADS, BY_NAME, TINY_4K, LLAMA_32K, LLAMA_128K_PLANTED,
                        BATCHED_16, LONG_4x128K, scaled)
from .gen import (Paging, LayerInputs, paging, seq_lens, query, kv_head, layer_inputs,
                  cluster_starts, apply_rope, f32_to_bf16_bits, bf16_bits_to_f32,
                  default_threads)

__all__ = [
    "Workload", "WORKLOADS", "BY_NAME", "TINY_4K", "LLAMA_32K", "LLAMA_128K_PLANTED",
    "BATCHED_16", "LONG_4x128K", "scaled", "Paging", "LayerInputs", "paging", "seq_lens",
    "query", "kv_head", "layer_inputs", "cluster_starts", "apply_rope", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "default_threads",
]
