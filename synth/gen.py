"""Seeded synthetic inputs for the decode-step workloads.

Everything is drawn with numpy from seeds derived from
(workload id, stream, layer, sequence, kv head), so any single layer, sequence
or KV head can be regenerated on its own, in any order, bit for bit.

What is generated (per layer):
  * q      bf16 [B, Hq, D]          ~N(0, 1), taken as already position-rotated
  * K      bf16 paged [P, Hkv, S, D] ~N(0, 1), then rotated by RoPE at its position
  * V      bf16 paged [P, Hkv, S, D] ~N(0, 1)
and, per workload, the block table [B, max_pages] (a seeded permutation of the
physical pages) and the sequence lengths [B].

RoPE uses the half-split pairing (d, d + D/2) with angle m * base^(-2d/D), the
x*cos(m theta) + rotate(x)*sin(m theta) form of the rotary embedding as the
spectral block-sparse "Prism" blog states it (its "RoPE + Mean Pooling Problem"
section).

Planted structure (the 128K workloads): the first `n_sinks` positions hold K
scaled by `sink_scale`; `n_clusters` runs of `cluster_len` contiguous tokens
have stored (post-RoPE) keys at cosine `cluster_cos` to one query head of their
KV group (cluster c aligns to head g*G + c mod G), with the key norm kept; the
cluster starts perform a +-`drift` random walk from one layer to the next.

This module holds input generation only: nothing of the scoring, selection,
window expansion or attention the library computes.
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .workloads import Workload

STREAM_K, STREAM_V, STREAM_Q, STREAM_CLUSTER, STREAM_LENS, STREAM_PAGES, STREAM_DRIFT = range(7)


def _rng(wl: Workload, stream: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([wl.wid, stream, *[int(i) for i in ids]])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 to the nearest bfloat16, ties to even; returns the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Paging:
    seq_lens: np.ndarray     # int32 [B]
    block_table: np.ndarray  # int32 [B, max_pages]; entries past a sequence's pages are 0
    num_pages: int
    max_pages: int


def seq_lens(wl: Workload) -> np.ndarray:
    if wl.lengths is not None:
        assert len(wl.lengths) == wl.batch
        return np.array(wl.lengths, dtype=np.int32)
    if wl.context is not None:
        return np.full(wl.batch, wl.context, dtype=np.int32)
    lo, hi = wl.len_range
    x = _rng(wl, STREAM_LENS).integers(lo, hi + 1, size=wl.batch)
    ps = wl.page_size
    x = ((x + ps // 2) // ps) * ps            # nearest multiple of the page size
    return np.clip(x, lo, hi).astype(np.int32)


@functools.lru_cache(maxsize=8)
def paging(wl: Workload) -> Paging:
    lens = seq_lens(wl)
    ps = wl.page_size
    npg = (lens.astype(np.int64) + ps - 1) // ps
    total = int(npg.sum())
    perm = _rng(wl, STREAM_PAGES).permutation(total).astype(np.int32)
    maxp = int(npg.max())
    bt = np.zeros((wl.batch, maxp), dtype=np.int32)
    off = 0
    for b in range(wl.batch):
        bt[b, : npg[b]] = perm[off: off + npg[b]]
        off += int(npg[b])
    lens.setflags(write=False)
    bt.setflags(write=False)
    return Paging(lens, bt, total, maxp)


@functools.lru_cache(maxsize=4)
def _rope_tables(length: int, dim: int, base: float):
    half = dim // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / dim)
    ang = np.arange(length, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    c.setflags(write=False)
    s.setflags(write=False)
    return c, s


def apply_rope(x: np.ndarray, base: float) -> np.ndarray:
    """Rotate rows x[m] (float32 [L, D]) by position m; pairs are (d, d + D/2)."""
    L, D = x.shape
    c, s = _rope_tables(L, D, float(base))
    x1, x2 = x[:, : D // 2], x[:, D // 2:]
    out = np.empty_like(x)
    out[:, : D // 2] = x1 * c - x2 * s
    out[:, D // 2:] = x2 * c + x1 * s
    return out


def query(wl: Workload, layer: int) -> np.ndarray:
    """bf16 bits [B, Hq, D]."""
    x = _rng(wl, STREAM_Q, layer).standard_normal((wl.batch, wl.num_q_heads, wl.head_dim),
                                                  dtype=np.float32)
    return f32_to_bf16_bits(x)


def cluster_starts(wl: Workload, layer: int, b: int, length: int) -> np.ndarray:
    """Start positions of the planted clusters of sequence b at this layer."""
    n, cl, ns = wl.n_clusters, wl.cluster_len, wl.n_sinks
    span = (length - cl) - ns - (n - 1) * cl
    if span < n:
        raise ValueError("sequence too short for the planted clusters")
    draws = np.sort(_rng(wl, STREAM_CLUSTER, 0, b).choice(span, size=n, replace=False))
    p = ns + draws + cl * np.arange(n)            # non-overlapping at layer 0
    for lyr in range(1, layer + 1):
        sign = _rng(wl, STREAM_DRIFT, lyr, b).choice(np.array([-1, 1]), size=n)
        p = np.clip(p + wl.drift * sign, ns, length - cl)
    return p.astype(np.int64)


def kv_head(wl: Workload, layer: int, b: int, g: int, length: int, q_bits: np.ndarray):
    """K and V rows of one (sequence, kv head) at one layer: bf16 bits [length, D] each.

    q_bits: bf16 bits [B, Hq, D] of this layer (planted clusters align to it).
    """
    D = wl.head_dim
    k = _rng(wl, STREAM_K, layer, b, g).standard_normal((length, D), dtype=np.float32)
    k = apply_rope(k, wl.rope_base)
    if wl.planted:
        k[: wl.n_sinks] *= np.float32(wl.sink_scale)
        G = wl.group
        qf = bf16_bits_to_f32(q_bits[b]).astype(np.float64)
        cs = wl.cluster_cos
        sn = float(np.sqrt(1.0 - cs * cs))
        for c, p in enumerate(cluster_starts(wl, layer, b, length)):
            qh = qf[g * G + c % G]
            qh = qh / np.linalg.norm(qh)
            r = k[p: p + wl.cluster_len].astype(np.float64)
            norm = np.linalg.norm(r, axis=1, keepdims=True)
            u = r - (r @ qh)[:, None] * qh[None, :]
            u /= np.linalg.norm(u, axis=1, keepdims=True)
            k[p: p + wl.cluster_len] = (norm * (cs * qh[None, :] + sn * u)).astype(np.float32)
    v = _rng(wl, STREAM_V, layer, b, g).standard_normal((length, D), dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


@dataclass
class LayerInputs:
    layer: int
    q: np.ndarray        # uint16 [B, Hq, D]
    k_pages: np.ndarray  # uint16 [P, Hkv, S, D]
    v_pages: np.ndarray  # uint16 [P, Hkv, S, D]


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_inputs(wl: Workload, layer: int, threads: int | None = None,
                 pool: ThreadPoolExecutor | None = None) -> LayerInputs:
    pg = paging(wl)
    q = query(wl, layer)
    S, D, Hkv = wl.page_size, wl.head_dim, wl.num_kv_heads
    kp = np.zeros((pg.num_pages, Hkv, S, D), dtype=np.uint16)
    vp = np.zeros_like(kp)

    def job(bg):
        b, g = bg
        L = int(pg.seq_lens[b])
        k, v = kv_head(wl, layer, b, g, L, q)
        npg = (L + S - 1) // S
        pad = npg * S - L
        if pad:
            k = np.concatenate([k, np.zeros((pad, D), np.uint16)])
            v = np.concatenate([v, np.zeros((pad, D), np.uint16)])
        ids = pg.block_table[b, :npg]
        kp[ids, g] = k.reshape(npg, S, D)
        vp[ids, g] = v.reshape(npg, S, D)

    jobs = [(b, g) for b in range(wl.batch) for g in range(Hkv)]
    if pool is not None:
        list(pool.map(job, jobs))
    else:
        n = threads or default_threads()
        if n == 1:
            for j in jobs:
                job(j)
        else:
            with ThreadPoolExecutor(n) as ex:
                list(ex.map(job, jobs))
    return LayerInputs(layer, q, kp, vp)
