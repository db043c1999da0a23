"""Token-sparse GQA decode attention with proposal-refined cross-layer index
sharing (Prism Attention) for MI355X / gfx950.

The computation lives in the HIP library libprism.so (C ABI: include/prism.h);
this package is its ctypes binding.  Functions carry the C names.
"""
from ._lib import (PrismError, KVCache, params, lib, declared_functions, prism_workspace_size,
                   prism_score_topk, prism_refine_topk, prism_sparse_attn, prism_decode_layer,
                   prism_decode_layer_noalloc, PRISM_STATIC_WORKSPACE_BYTES,
                   prism_status_string, prism_last_error, prism_abi_version, prism_profile_events,
                   prism_profile_launches, prism_pattern_role, prism_decode_layer_role,
                   prism_quantize_keys, int2_shapes, prism_dense_attn,
                   KERNEL_KINDS, ROLES, PRISM_OK,
                   PRISM_ERR_INVALID_ARG, PRISM_ERR_UNSUPPORTED, PRISM_ERR_WORKSPACE,
                   PRISM_ERR_HIP, LIB_PATH)

__all__ = ["PrismError", "KVCache", "params", "lib", "declared_functions", "prism_workspace_size",
           "prism_score_topk", "prism_refine_topk", "prism_sparse_attn", "prism_decode_layer",
           "prism_decode_layer_noalloc", "PRISM_STATIC_WORKSPACE_BYTES",
           "prism_status_string", "prism_last_error", "prism_abi_version",
           "prism_profile_events", "prism_profile_launches", "prism_pattern_role",
           "prism_decode_layer_role", "prism_quantize_keys", "int2_shapes", "prism_dense_attn",
           "KERNEL_KINDS",
           "ROLES", "PRISM_OK",
           "PRISM_ERR_INVALID_ARG", "PRISM_ERR_UNSUPPORTED", "PRISM_ERR_WORKSPACE",
           "PRISM_ERR_HIP", "LIB_PATH"]
