"""CPU oracle (test infrastructure only): a plain float64 reference of the
decode-step path.  Imported only by the tests, the package smoke check and the
benchmark's CPU-baseline leg; it shares no code with the HIP library."""
from .prism_oracle import (bf16_to_f64, cache_rows, relevance, top_kappa, window_pool,
                           rank_pool, attention_weights, sparse_attention, default_scale,
                           anchor_select, refine_in_pool, refined_select, attend, decode_layer,
                           decode_step, layer_roles, stride_role, cache_row_bits,
                           quantize_int2, dequantize_int2, proposal_rows, INT2_GROUP,
                           dense_attend)

__all__ = ["bf16_to_f64", "cache_rows", "relevance", "top_kappa", "window_pool", "rank_pool",
           "attention_weights", "sparse_attention", "default_scale", "anchor_select",
           "refine_in_pool", "refined_select", "attend", "decode_layer", "decode_step",
           "layer_roles", "stride_role", "cache_row_bits", "quantize_int2", "dequantize_int2",
           "proposal_rows", "INT2_GROUP", "dense_attend"]
