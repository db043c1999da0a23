"""Plain CPU reference ("oracle") for token-sparse GQA decode attention with
proposal-refined cross-layer index sharing, as "Prism Attention:
Proposal-Refined Index Sharing Mechanism for Efficient LLMs Inference"
(arXiv 2610.22985) describes it.

TEST INFRASTRUCTURE.  This module is slow on purpose and exists only to check
the GPU library.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library and imports nothing from it.

Everything is float64 numpy, except the INT2 quantizer, whose integer
decisions are taken in float32 (the precision the GPU takes them in).  bf16
inputs are widened exactly.  Readings taken where the paper is silent (all also
listed in the design notes):
  * scoring uses the bf16 keys themselves by default; with int2=True it uses
    the INT2 keys of Section 4.2 (Eqs. 7-9): groups of 32 dimensions, the
    scale and zero point stored as bf16, and the score taken against the
    dequantized key alpha * code + beta;
  * GQA: query head j belongs to KV head j // G (consecutive blocks);
  * TopK ties go to the lower token position; the selected set is returned as
    ascending positions (the paper treats it as a set);
  * refined layers use a positional window by default: the candidate pool is
    the union of [i - w, i + w], clipped to [0, L), over the anchor layer's
    top-kappa set; the paper's own pool, the anchor's top-(rho*kappa) tokens
    (Eq. 4), is the alternative (pool_rho >= 1);
  * a refined layer always expands the nearest preceding anchor's set;
  * SparseAttn is softmax attention with scale 1/sqrt(D) unless given.

Parity pins: every function below is pinned by tests (brute force on tiny
inputs, closed forms, invariants, a library routine for dense attention, and a
hand-worked example).  The chained multi-layer step is a composition of the
pinned parts and is otherwise "parity unpinned": the paper prints no numeric
end-to-end example.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# bf16 and the paged cache
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """A bf16 value is the upper 16 bits of a binary32 word; widening is exact."""
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def cache_rows(pages, block_table_row, kv_head: int, positions, page_size: int) -> np.ndarray:
    """Rows of the paged cache (the historical keys or values of Section 4.1)
    for one sequence and KV head, at the given token positions: float64 [n, D].

    pages: uint16 [num_pages, Hkv, page_size, D]; logical page p of the
    sequence lives at physical page block_table_row[p].
    """
    pos = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(block_table_row, dtype=np.int64)[pos // page_size]
    return bf16_to_f64(pages[phys, kv_head, pos % page_size, :])


def cache_row_bits(pages, block_table_row, kv_head: int, positions, page_size: int):
    """As cache_rows, the raw bf16 bit patterns: uint16 [n, D]."""
    pos = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(block_table_row, dtype=np.int64)[pos // page_size]
    return np.asarray(pages[phys, kv_head, pos % page_size, :], dtype=np.uint16)


# ---------------------------------------------------------------------------
# Section 4.2: INT2 proposal keys (Eqs. 7-8)
# ---------------------------------------------------------------------------

INT2_BITS = 2
INT2_GROUP = 32      # dimensions per quantization group (g); the paper leaves it open


def _round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quantize_int2(k_bits, group: int = INT2_GROUP):
    """Group-wise asymmetric b = 2 quantization of keys (Eqs. 7-8).  Each key
    row is split into D / group consecutive sub-vectors; a sub-vector's zero
    point beta is its minimum and its scale alpha is (max - min) / (2^b - 1),
    kept as a bf16 value; each element's code is (k - beta) / alpha rounded to
    the nearest integer (ties to even) and clipped to [0, 2^b - 1]; a constant
    sub-vector (alpha = 0) gets code 0.  The subtraction, division and rounding
    are float32 operations, the precision the GPU decides the codes in; -0 is
    read as +0.

    k_bits: uint16 bf16 bit patterns [n, D].  Returns (codes uint8 [n, D],
    alpha float64 [n, D / group], beta float64 [n, D / group]), the scales as
    the stored bf16 values."""
    bits = np.asarray(k_bits, dtype=np.uint16)
    n, D = bits.shape
    if D % group:
        raise ValueError("head dimension must be a multiple of the group size")
    k = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(n, D // group, group)
    k = k + np.float32(0.0)      # -0 reads as +0 (so a zero point is never -0)
    levels = np.float32(2 ** INT2_BITS - 1)
    mx, mn = k.max(axis=2), k.min(axis=2)
    alpha = _round_to_bf16((mx - mn) / levels)
    beta = mn
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        x = (k - beta[..., None]) / alpha[..., None]
        c = np.clip(np.rint(x), 0, levels)
    c = np.where(alpha[..., None] == 0, np.float32(0), c)
    return (c.astype(np.uint8).reshape(n, D), alpha.astype(np.float64), beta.astype(np.float64))


def dequantize_int2(codes, alpha, beta, group: int = INT2_GROUP) -> np.ndarray:
    """The key an INT2 code row stands for: alpha * code + beta per group
    (float64 [n, D])."""
    c = np.asarray(codes, dtype=np.float64)
    n, D = c.shape
    c = c.reshape(n, D // group, group)
    return (np.asarray(alpha)[..., None] * c + np.asarray(beta)[..., None]).reshape(n, D)


def proposal_rows(k_pages, block_table_row, kv_head, positions, page_size, int2=False):
    """The keys relevance is computed from: the cached bf16 rows, or with
    int2 the dequantized INT2 codes of those rows (Eq. 9 on the quantized
    keys)."""
    if not int2:
        return cache_rows(k_pages, block_table_row, kv_head, positions, page_size)
    bits = cache_row_bits(k_pages, block_table_row, kv_head, positions, page_size)
    return dequantize_int2(*quantize_int2(bits))


# ---------------------------------------------------------------------------
# Section 4.1 / 4.2: relevance, TopK, the candidate pool
# ---------------------------------------------------------------------------

def relevance(q_group: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Eq. 9 (used as phi in Eq. 1 and Eq. 5): the score of token i is the
    largest inner product <q_j, k_i> over the query heads j of the KV head's
    group.  q_group: [G, D]; keys: [n, D]; returns [n]."""
    dots = keys @ q_group.T          # [n, G]
    return dots.max(axis=1)


def top_kappa(scores: np.ndarray, kappa: int, positions: np.ndarray) -> np.ndarray:
    """Eq. 2 / Eq. 6: positions of the kappa largest scores.  A full stable sort
    on (-score, position): equal scores go to the lower position.  Returned
    ascending (set semantics)."""
    scores = np.asarray(scores, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    if not 1 <= kappa <= scores.shape[0]:
        raise ValueError("need 1 <= kappa <= number of candidates")
    order = np.lexsort((positions, -scores))
    return np.sort(positions[order[:kappa]])


def window_pool(anchor_positions, w: int, length: int) -> np.ndarray:
    """Candidate pool of a refined layer: every position within +-w of a token
    the anchor layer selected, clipped to [0, length), each position once.
    (The paper motivates refinement by salient tokens shifting to the
    neighbourhood of the previously selected ones; the positional window is
    this library's concrete pool rule.)  Returned ascending."""
    mask = np.zeros(length, dtype=bool)
    for i in np.asarray(anchor_positions, dtype=np.int64):
        lo = max(0, int(i) - w)
        hi = min(length - 1, int(i) + w)
        mask[lo: hi + 1] = True
    return np.flatnonzero(mask).astype(np.int64)


def rank_pool(anchor_scores, positions, rho: int, kappa: int) -> np.ndarray:
    """Eq. 4: the candidate pool a proposal (anchor) layer hands to the layers
    it serves is its own rho*kappa most relevant tokens, TopK of Eq. 2 with
    rho*kappa in place of kappa (every candidate when rho*kappa exceeds their
    number).  anchor_scores are the anchor layer's relevance over `positions`.
    Returned ascending."""
    if rho < 1:
        raise ValueError("rho must be >= 1")
    positions = np.asarray(positions, dtype=np.int64)
    return top_kappa(anchor_scores, min(rho * kappa, positions.shape[0]), positions)


# ---------------------------------------------------------------------------
# Algorithm 1, SparseAttn
# ---------------------------------------------------------------------------

def attention_weights(q_group: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """Softmax over the selected tokens of z_i = scale * <q_j, k_i>, per query
    head j: [G, n].  The largest logit is subtracted first (exact in real
    arithmetic, keeps exp in range)."""
    z = (q_group @ keys.T) * scale
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def sparse_attention(q_group: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     scale: float) -> np.ndarray:
    """SparseAttn of Algorithm 1: attention of each query head over the selected
    tokens only.  keys/values: [n, D] rows of the selected tokens; [G, D] out."""
    return attention_weights(q_group, keys, scale) @ values


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# One layer and one decode step over the paged cache
# ---------------------------------------------------------------------------

def anchor_select(q_group, k_pages, block_table_row, kv_head, length, kappa, page_size,
                  int2=False):
    """Proposal (anchor) layer of Algorithm 1: score every cached token (bf16
    keys, or INT2 keys with int2), keep the exact top-kappa.
    Returns (selected, scores)."""
    pos = np.arange(length, dtype=np.int64)
    s = relevance(q_group, proposal_rows(k_pages, block_table_row, kv_head, pos, page_size, int2))
    return top_kappa(s, kappa, pos), s


def refine_in_pool(q_group, k_pages, block_table_row, kv_head, pool, kappa, page_size,
                   int2=False):
    """Refined layer of Algorithm 1 (Eqs. 5-6) over a given candidate pool:
    re-score only the pool's tokens (with INT2 keys if int2, as Algorithm 1's
    refined layers do), keep the top-kappa there.
    Returns (selected, scores over the pool)."""
    pool = np.asarray(pool, dtype=np.int64)
    s = relevance(q_group, proposal_rows(k_pages, block_table_row, kv_head, pool, page_size,
                                         int2))
    return top_kappa(s, kappa, pool), s


def refined_select(q_group, k_pages, block_table_row, kv_head, length, kappa, page_size,
                   anchor_positions, w, int2=False):
    """Refined layer with the window pool built from the anchor's set.
    Returns (selected, pool, scores over the pool)."""
    pool = window_pool(anchor_positions, w, length)
    t, s = refine_in_pool(q_group, k_pages, block_table_row, kv_head, pool, kappa, page_size,
                          int2)
    return t, pool, s


def attend(q_group, k_pages, v_pages, block_table_row, kv_head, selected, page_size, scale):
    keys = cache_rows(k_pages, block_table_row, kv_head, selected, page_size)
    vals = cache_rows(v_pages, block_table_row, kv_head, selected, page_size)
    return sparse_attention(q_group, keys, vals, scale)


# ---------------------------------------------------------------------------
# Layer roles (Algorithm 1's partition into proposal and refined layers; the
# proposal / refined / shared hybrid of Appendix E, Table 9)
# ---------------------------------------------------------------------------

ROLES = ("F", "R", "S")


def layer_roles(pattern: str, *, table4: bool = False) -> list:
    """Roles of a layer-assignment pattern, one letter per layer.  F: proposal
    layer (scores the whole cache and exports the candidate pool); R: refined
    layer (re-selects within the pool of the nearest preceding F layer); S:
    shared layer (reuses the set of the nearest preceding F or R layer as it
    is).  These are Table 9's meanings; Table 4 writes its refined layers as S,
    which table4=True reads as R.  Layer 0 must be F."""
    letters = ("F", "S") if table4 else ROLES
    for c in pattern:
        if c not in letters:
            raise ValueError(f"pattern letter {c!r} is not one of {', '.join(letters)}")
    roles = [("R" if (table4 and c == "S") else c) for c in pattern]
    if not roles:
        raise ValueError("empty pattern")
    if roles[0] != "F":
        raise ValueError("the first layer of a pattern must be a proposal layer (F)")
    return roles


def stride_role(layer: int, anchor_stride: int) -> str:
    """Algorithm 1 with a fixed association: every anchor_stride-th layer,
    starting at layer 0, is a proposal layer; the others are refined."""
    return "F" if layer % anchor_stride == 0 else "R"


def dense_attend(q_group, k_pages, v_pages, block_table_row, kv_head, length, page_size, scale):
    """Dense decode attention: SparseAttn with every cached token [0, length)
    as the set (the full-attention baseline the paper's Tables 6-8 compare
    the sparse path against).  [G, D]."""
    return attend(q_group, k_pages, v_pages, block_table_row, kv_head,
                  np.arange(length, dtype=np.int64), page_size, scale)


def decode_layer(layer, q_bits, k_pages, v_pages, block_table, seq_lens, *, num_kv_heads,
                 kappa, anchor_stride, window, page_size, anchor_state=None, scale=None,
                 problems=None, pool_rho=0, pool_state=None, role=None, shared_state=None,
                 int2=False):
    """One layer of Algorithm 1 for every (sequence, KV head).

    q_bits: uint16 [B, Hq, D].  anchor_state: int64 [B, Hkv, kappa], the most
    recent anchor layer's sets (required for a refined layer).
    pool_rho: 0 for the window pool, rho >= 1 for the anchor's top rho*kappa
    tokens (Eq. 4); then pool_state, {(b, g): pool} from the most recent
    anchor layer, is required for a refined layer.
    role: 'F', 'R' or 'S' (see layer_roles); None derives F or R from the
    stride.  A shared layer attends over shared_state, the most recent F or R
    layer's sets, and scores nothing.
    int2: relevance from the INT2 keys (Section 4.2) at proposal and refined
    layers; attention always reads the bf16 keys and values.
    problems: optional list of (b, g) to restrict the work to (others are left
    as -1 / NaN).

    Returns dict(selected [B,Hkv,kappa] int64, out [B,Hq,D] float64,
    anchor_state, pool_state, shared_state, pools {(b,g): pool the layer
    selected from}, scores {(b,g): scores over that pool}).
    """
    B, Hq, D = q_bits.shape
    G = Hq // num_kv_heads
    if scale is None or scale == 0:
        scale = default_scale(D)
    q = bf16_to_f64(q_bits)
    if role is None:
        role = stride_role(layer, anchor_stride)
    if role not in ROLES:
        raise ValueError(f"unknown role {role!r}")
    is_anchor = role == "F"
    if role == "R" and anchor_state is None:
        raise ValueError("a refined layer needs the preceding anchor's sets")
    if role == "R" and pool_rho >= 1 and pool_state is None:
        raise ValueError("a refined layer needs the preceding anchor's pools")
    if role == "S" and shared_state is None:
        raise ValueError("a shared layer needs the preceding proposal or refined layer's sets")
    sel = np.full((B, num_kv_heads, kappa), -1, dtype=np.int64)
    out = np.full((B, Hq, D), np.nan)
    pools, scores = {}, {}
    new_pools = {} if is_anchor else pool_state
    todo = problems if problems is not None else [(b, g) for b in range(B)
                                                  for g in range(num_kv_heads)]
    for b, g in todo:
        qg = q[b, g * G:(g + 1) * G]
        L = int(seq_lens[b])
        if role == "S":
            t = np.asarray(shared_state[b, g], dtype=np.int64)
        elif is_anchor:
            t, s = anchor_select(qg, k_pages, block_table[b], g, L, kappa, page_size, int2)
            pools[(b, g)] = np.arange(L, dtype=np.int64)
            if pool_rho >= 1:
                new_pools[(b, g)] = rank_pool(s, pools[(b, g)], pool_rho, kappa)
        elif pool_rho >= 1:
            pool = pool_state[(b, g)]
            t, s = refine_in_pool(qg, k_pages, block_table[b], g, pool, kappa, page_size, int2)
            pools[(b, g)] = pool
        else:
            t, pool, s = refined_select(qg, k_pages, block_table[b], g, L, kappa, page_size,
                                        anchor_state[b, g], window, int2)
            pools[(b, g)] = pool
        if role != "S":
            scores[(b, g)] = s
        sel[b, g] = t
        out[b, g * G:(g + 1) * G] = attend(qg, k_pages, v_pages, block_table[b], g, t,
                                           page_size, scale)
    new_state = sel.copy() if is_anchor else anchor_state
    new_shared = sel.copy() if role != "S" else shared_state
    return dict(selected=sel, out=out, anchor_state=new_state, pool_state=new_pools,
                shared_state=new_shared, pools=pools, scores=scores)


def decode_step(layers, block_table, seq_lens, *, num_kv_heads, kappa, anchor_stride, window,
                page_size, scale=None, pool_rho=0, roles=None, int2=False):
    """Algorithm 1 over layers 0..N-1 in order; `layers` yields
    (q_bits, k_pages, v_pages) per layer.  roles: optional per-layer roles
    (layer_roles); without them layer l is F iff l mod anchor_stride == 0.
    Layer 0 must be a proposal layer."""
    state, pstate, shared = None, None, None
    results = []
    for l, (q_bits, kp, vp) in enumerate(layers):
        role = roles[l] if roles is not None else None
        r = decode_layer(l, q_bits, kp, vp, block_table, seq_lens, num_kv_heads=num_kv_heads,
                         kappa=kappa, anchor_stride=anchor_stride, window=window,
                         page_size=page_size, anchor_state=state, scale=scale,
                         pool_rho=pool_rho, pool_state=pstate, role=role,
                         shared_state=shared, int2=int2)
        state, pstate, shared = r["anchor_state"], r["pool_state"], r["shared_state"]
        results.append(r)
    return results
