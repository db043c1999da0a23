"""ctypes binding of libprism.so: argument marshalling only.  Every computation
happens in the HIP library; there is no fallback path.  Tensor arguments are
PyTorch device tensors (PyTorch is used for device memory and streams); bf16
arrays may be given as torch.bfloat16, torch.int16 or torch.uint16 tensors
holding the bit patterns."""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# PRISM_LIBRARY: another build of the same library (the host-sanitizer test loads one)
LIB_PATH = os.environ.get("PRISM_LIBRARY") or os.path.join(PKG_DIR, "libprism.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "prism.h")

PRISM_STATIC_WORKSPACE_BYTES = 64 << 20   # include/prism.h: the no-allocation call's workspace
PRISM_OK, PRISM_ERR_INVALID_ARG, PRISM_ERR_UNSUPPORTED, PRISM_ERR_WORKSPACE, PRISM_ERR_HIP = \
    0, -1, -2, -3, -4


class PrismError(RuntimeError):
    def __init__(self, status: int, fn: str, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


ABI_VERSION = 7   # PRISM_ABI_VERSION of include/prism.h that the structs below follow


class KVCacheStruct(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("min_seq_len", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("new_keys", ctypes.c_int32)]


class ParamsStruct(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("kappa", ctypes.c_int32),
                ("anchor_stride", ctypes.c_int32), ("window", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("pool_rho", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGS = {
    "prism_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(KVCacheStruct),
                                               ctypes.POINTER(ParamsStruct)]),
    "prism_score_topk": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), _P,
                                        ctypes.POINTER(ParamsStruct), _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "prism_refine_topk": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), _P,
                                         ctypes.POINTER(ParamsStruct), _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "prism_sparse_attn": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), _P,
                                         ctypes.POINTER(ParamsStruct), _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "prism_decode_layer": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(KVCacheStruct), _P,
                                          ctypes.POINTER(ParamsStruct), _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "prism_decode_layer_noalloc": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(KVCacheStruct),
                                                  _P, ctypes.POINTER(ParamsStruct), _P, _P, _P,
                                                  _P]),
    "prism_dense_attn": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), _P,
                                        ctypes.POINTER(ParamsStruct), _P, _P, ctypes.c_size_t, _P]),
    "prism_quantize_keys": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), ctypes.c_int32, _P, _P,
                                           _P]),
    "prism_pattern_role": (ctypes.c_int32, [ctypes.c_char_p, ctypes.c_int32, ctypes.c_int32]),
    "prism_decode_layer_role": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(KVCacheStruct), _P,
                                               ctypes.POINTER(ParamsStruct), _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "prism_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "prism_last_error": (ctypes.c_char_p, []),
    "prism_abi_version": (ctypes.c_int32, []),
    "prism_profile_events": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
    "prism_profile_launches": (ctypes.c_int64, [ctypes.c_int32]),
}

# prism_layer_role
ROLES = {"F": 0, "R": 1, "S": 2}

# prism_kernel_kind
KERNEL_KINDS = {"anchor_score": 0, "refine_score": 1, "select": 2, "attention": 3,
                "pool_build": 4, "classify": 5, "merge": 6, "quantize": 7, "dense": 8}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(token_sparse_attention_gqa_amd.build.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        version = int(handle.prism_abi_version())
        if version != ABI_VERSION:   # the structs above follow one layout only
            raise RuntimeError(f"{LIB_PATH} has ABI version {version}, this binding expects "
                               f"{ABI_VERSION}: rebuild the HIP library")
        _lib = handle
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/prism.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^PRISM_API\s+[\w\s\*]+?\b(prism_\w+)\s*\(", text, re.M)))


def _check(status: int, fn: str):
    if status != PRISM_OK:
        msg = lib().prism_last_error().decode(errors="replace")
        raise PrismError(status, fn, msg)


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t, name, *, itemsize=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):          # raw device address
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class KVCache:
    """One layer's paged cache: keeps the tensors alive and the C struct."""

    def __init__(self, k_pages, v_pages, block_table, seq_lens, *, max_seq_len, min_seq_len,
                 head_dim=None, page_size=None, k_codes=None, k_scales=None, new_keys=0):
        """k_codes / k_scales (optional, together): the INT2 proposal keys,
        uint8 [num_pages, Hkv, page, 32] and bf16 bits [num_pages, Hkv, page, 4, 2].
        new_keys: trailing positions of every sequence whose codes the scoring
        calls write before scoring them (a decode step's appended keys)."""
        self.tensors = (k_pages, v_pages, block_table, seq_lens, k_codes, k_scales)
        num_pages, hkv, ps, d = k_pages.shape
        if tuple(v_pages.shape) != tuple(k_pages.shape):
            raise ValueError("k_pages and v_pages must have the same shape")
        batch, max_pages = block_table.shape
        self.struct = KVCacheStruct(
            _ptr(k_pages, "k_pages", itemsize=2), _ptr(v_pages, "v_pages", itemsize=2),
            _ptr(block_table, "block_table", itemsize=4), _ptr(seq_lens, "seq_lens", itemsize=4),
            batch, hkv, head_dim if head_dim is not None else d,
            page_size if page_size is not None else ps, num_pages, max_pages, int(max_seq_len),
            int(min_seq_len), _ptr(k_codes, "k_codes", itemsize=1, optional=True),
            _ptr(k_scales, "k_scales", itemsize=2, optional=True), int(new_keys))

    def with_layer(self, k_pages, v_pages, k_codes=None, k_scales=None,
                   new_keys=0) -> "KVCache":
        """Same sequences and block table, another layer's K/V (and INT2) arrays."""
        bt, sl = self.tensors[2], self.tensors[3]
        s = self.struct
        return KVCache(k_pages, v_pages, bt, sl, max_seq_len=s.max_seq_len,
                       min_seq_len=s.min_seq_len, head_dim=s.head_dim, page_size=s.page_size,
                       k_codes=k_codes, k_scales=k_scales, new_keys=new_keys)

    def with_int2(self, k_codes, k_scales, new_keys=0) -> "KVCache":
        """The same cache with INT2 proposal keys (or without, given None)."""
        return self.with_layer(self.tensors[0], self.tensors[1], k_codes, k_scales, new_keys)

    def with_new_keys(self, new_keys) -> "KVCache":
        """The same cache whose last new_keys positions still lack INT2 codes."""
        t = self.tensors
        return self.with_layer(t[0], t[1], t[4], t[5], new_keys)


def params(num_q_heads, kappa, anchor_stride=1, window=0, softmax_scale=0.0,
           pool_rho=0) -> ParamsStruct:
    """prism_params; pool_rho >= 1 selects the rank-expanded pool (the anchor's
    top pool_rho * kappa tokens) instead of the window pool."""
    return ParamsStruct(int(num_q_heads), int(kappa), int(anchor_stride), int(window),
                        float(softmax_scale), int(pool_rho))


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# The C entry points, same names
# ---------------------------------------------------------------------------

def prism_workspace_size(kv: KVCache, p: ParamsStruct) -> int:
    return int(lib().prism_workspace_size(ctypes.byref(kv.struct), ctypes.byref(p)))


def prism_score_topk(kv, q, p, idx_out, scores_out=None, workspace=None, stream=None):
    ws, nbytes = _ws(workspace)
    _check(lib().prism_score_topk(ctypes.byref(kv.struct), _ptr(q, "q", itemsize=2),
                                  ctypes.byref(p), _ptr(idx_out, "idx_out", itemsize=4),
                                  _ptr(scores_out, "scores_out", itemsize=4, optional=True),
                                  ws, nbytes, _stream(stream)), "prism_score_topk")


def prism_refine_topk(kv, q, p, anchor_idx, idx_out, pool_out=None, pool_len_out=None,
                      pool_scores_out=None, workspace=None, stream=None):
    ws, nbytes = _ws(workspace)
    _check(lib().prism_refine_topk(
        ctypes.byref(kv.struct), _ptr(q, "q", itemsize=2), ctypes.byref(p),
        _ptr(anchor_idx, "anchor_idx", itemsize=4, optional=p.pool_rho >= 1),
        _ptr(idx_out, "idx_out", itemsize=4),
        _ptr(pool_out, "pool_out", itemsize=4, optional=True),
        _ptr(pool_len_out, "pool_len_out", itemsize=4, optional=True),
        _ptr(pool_scores_out, "pool_scores_out", itemsize=4, optional=True),
        ws, nbytes, _stream(stream)), "prism_refine_topk")


def prism_sparse_attn(kv, q, p, idx, out, workspace=None, stream=None):
    ws, nbytes = _ws(workspace)
    _check(lib().prism_sparse_attn(ctypes.byref(kv.struct), _ptr(q, "q", itemsize=2),
                                   ctypes.byref(p), _ptr(idx, "idx", itemsize=4),
                                   _ptr(out, "out", itemsize=4), ws, nbytes, _stream(stream)),
           "prism_sparse_attn")


def prism_decode_layer(layer, kv, q, p, anchor_idx, layer_idx_out, out, workspace=None,
                       stream=None):
    ws, nbytes = _ws(workspace)
    _check(lib().prism_decode_layer(int(layer), ctypes.byref(kv.struct), _ptr(q, "q", itemsize=2),
                                    ctypes.byref(p), _ptr(anchor_idx, "anchor_idx", itemsize=4),
                                    _ptr(layer_idx_out, "layer_idx_out", itemsize=4,
                                         optional=True),
                                    _ptr(out, "out", itemsize=4), ws, nbytes, _stream(stream)),
           "prism_decode_layer")


def prism_decode_layer_noalloc(layer, kv, q, p, anchor_idx, layer_idx_out, out, stream=None):
    """prism_decode_layer on the library's static per-GPU workspace (no
    allocation; shapes needing more than PRISM_STATIC_WORKSPACE_BYTES fail)."""
    _check(lib().prism_decode_layer_noalloc(int(layer), ctypes.byref(kv.struct),
                                            _ptr(q, "q", itemsize=2), ctypes.byref(p),
                                            _ptr(anchor_idx, "anchor_idx", itemsize=4),
                                            _ptr(layer_idx_out, "layer_idx_out", itemsize=4,
                                                 optional=True),
                                            _ptr(out, "out", itemsize=4), _stream(stream)),
           "prism_decode_layer_noalloc")


def prism_dense_attn(kv, q, p, out, workspace=None, stream=None):
    """Dense decode attention over every cached token into out [B, Hq, D]."""
    ws, nbytes = _ws(workspace)
    _check(lib().prism_dense_attn(ctypes.byref(kv.struct), _ptr(q, "q", itemsize=2),
                                  ctypes.byref(p), _ptr(out, "out", itemsize=4), ws, nbytes,
                                  _stream(stream)),
           "prism_dense_attn")


def prism_quantize_keys(kv, num_new, k_codes, k_scales, stream=None):
    """INT2 codes and scales of the last num_new positions' keys (all if <= 0)."""
    _check(lib().prism_quantize_keys(ctypes.byref(kv.struct), int(num_new),
                                     _ptr(k_codes, "k_codes", itemsize=1),
                                     _ptr(k_scales, "k_scales", itemsize=2), _stream(stream)),
           "prism_quantize_keys")


def int2_shapes(num_pages, num_kv_heads, page_size=64):
    """Shapes of the INT2 code and scale arrays for a cache of these pages."""
    return (num_pages, num_kv_heads, page_size, 32), (num_pages, num_kv_heads, page_size, 4, 2)


def prism_pattern_role(pattern: str, layer: int, table4: bool = False) -> int:
    """prism_layer_role of `layer` in a pattern string (-1 if invalid)."""
    return int(lib().prism_pattern_role(pattern.encode(), int(bool(table4)), int(layer)))


def prism_decode_layer_role(role, kv, q, p, set_idx, out, workspace=None, stream=None):
    """role: a prism_layer_role value, or one of the letters F, R, S."""
    if isinstance(role, str):
        role = ROLES.get(role, -1)
    ws, nbytes = _ws(workspace)
    _check(lib().prism_decode_layer_role(int(role), ctypes.byref(kv.struct),
                                         _ptr(q, "q", itemsize=2), ctypes.byref(p),
                                         _ptr(set_idx, "set_idx", itemsize=4),
                                         _ptr(out, "out", itemsize=4), ws, nbytes,
                                         _stream(stream)),
           "prism_decode_layer_role")


def prism_status_string(status: int) -> str:
    return lib().prism_status_string(int(status)).decode()


def prism_last_error() -> str:
    return lib().prism_last_error().decode(errors="replace")


def prism_abi_version() -> int:
    return int(lib().prism_abi_version())


def prism_profile_events(kind, start_events, stop_events):
    """start_events / stop_events: lists of torch.cuda.Event (timing enabled) or
    raw hipEvent_t handles; empty lists switch profiling of that kind off."""
    k = KERNEL_KINDS[kind] if isinstance(kind, str) else int(kind)
    n = len(start_events)
    if len(stop_events) != n:
        raise ValueError("need as many stop events as start events")

    def handle(e):
        if isinstance(e, int):
            return e
        if e.cuda_event == 0:        # torch creates the event lazily on first record
            e.record()
        return e.cuda_event

    arr_t = ctypes.c_void_p * max(n, 1)
    starts = arr_t(*[handle(e) for e in start_events])
    stops = arr_t(*[handle(e) for e in stop_events])
    _check(lib().prism_profile_events(k, starts if n else None, stops if n else None, n),
           "prism_profile_events")


def prism_profile_launches(kind) -> int:
    k = KERNEL_KINDS[kind] if isinstance(kind, str) else int(kind)
    return int(lib().prism_profile_launches(k))
