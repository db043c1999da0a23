"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one: a pin set that a dropped term, a wrong sign or index
or a transposed operand slips through would not be pinning anything."""
import types

import numpy as np
import pytest

import oracle
from oracle import prism_oracle as po
from tests import pins


def _compose(ns, keep=()):
    """anchor/refined selection (and the rank pool, unless itself mutated)
    built from the namespace's own parts, so a mutated part shows through
    them."""
    def proposal_rows(kp, bt, g, pos, ps, int2=False):
        if not int2:
            return ns.cache_rows(kp, bt, g, pos, ps)
        return ns.dequantize_int2(*ns.quantize_int2(ns.cache_row_bits(kp, bt, g, pos, ps)))

    def anchor_select(q, kp, bt, g, L, kappa, ps, int2=False):
        pos = np.arange(L, dtype=np.int64)
        s = ns.relevance(q, ns.proposal_rows(kp, bt, g, pos, ps, int2))
        return ns.top_kappa(s, kappa, pos), s

    def refine_in_pool(q, kp, bt, g, pool, kappa, ps, int2=False):
        s = ns.relevance(q, ns.proposal_rows(kp, bt, g, pool, ps, int2))
        return ns.top_kappa(s, kappa, pool), s

    def refined_select(q, kp, bt, g, L, kappa, ps, A, w, int2=False):
        pool = ns.window_pool(A, w, L)
        t, s = ns.refine_in_pool(q, kp, bt, g, pool, kappa, ps, int2)
        return t, pool, s

    def rank_pool(s, pos, rho, kappa):
        return ns.top_kappa(s, min(rho * kappa, len(pos)), pos)

    ns.anchor_select, ns.refined_select = anchor_select, refined_select
    if "refine_in_pool" not in keep:
        ns.refine_in_pool = refine_in_pool
    if "rank_pool" not in keep:
        ns.rank_pool = rank_pool
    if "proposal_rows" not in keep:
        ns.proposal_rows = proposal_rows
    return ns


def _impl(**over):
    ns = types.SimpleNamespace(**{n: getattr(oracle, n) for n in oracle.__all__})
    for k, v in over.items():
        setattr(ns, k, v)
    return _compose(ns, keep=tuple(over))


def _topk_with(sort_keys):
    def f(scores, kappa, positions):
        scores, positions = np.asarray(scores, float), np.asarray(positions, np.int64)
        order = np.lexsort(sort_keys(scores, positions))
        return np.sort(positions[order[:kappa]])
    return f


def _pool_with(lo_fn, hi_fn, incl=1):
    def f(A, w, L):
        m = np.zeros(L, bool)
        for i in np.asarray(A, np.int64):
            m[max(0, lo_fn(int(i), w)): min(L - 1, hi_fn(int(i), w)) + incl] = True
        return np.flatnonzero(m)
    return f


def _attn_weights_with(transform):
    def f(q, k, scale):
        return transform(q, k, scale)
    return f


def _softmax_rows(z):
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def _attn_pair(weights):
    return dict(attention_weights=weights,
                sparse_attention=lambda q, k, v, s: weights(q, k, s) @ v)


def _quantize_with(levels=3, group=32, zero=lambda kg: kg.min(axis=2), rnd=np.rint,
                   bf16_scale=True, order=None):
    """The INT2 quantizer with one of its choices changed."""
    def q(bits, g_unused=32):
        bits = np.asarray(bits, np.uint16)
        n, D = bits.shape
        k = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
        perm = order(D) if order is not None else None
        if perm is not None:
            k = k[:, perm]
        kg = k.reshape(n, D // group, group)
        mn, mx = kg.min(axis=2), kg.max(axis=2)
        a = (mx - mn) / np.float32(levels)
        if bf16_scale:
            a = po._round_to_bf16(a)
        b = zero(kg)
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            c = np.clip(rnd((kg - b[..., None]) / a[..., None]), 0, 3)
        c = np.where(a[..., None] == 0, 0, c).astype(np.uint8).reshape(n, D)
        if perm is not None:
            c = c[:, np.argsort(perm)]
        reps = 32 // group if group < 32 else 1
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
        if group != 32:   # report per 32-dim block (first sub-block's values) for the shapes
            a64 = a64.reshape(n, -1, reps).max(axis=2) if group < 32 else np.repeat(a64, 2, axis=1)
            b64 = b64.reshape(n, -1, reps).min(axis=2) if group < 32 else np.repeat(b64, 2, axis=1)
        return c, a64, b64
    return q


def _step_with(fix):
    """decode_step whose per-layer (role, anchor_state, shared_state) pass
    through fix(role, anchor_state, shared_state) before each layer."""
    def step(layers, bt, lens, *, roles=None, anchor_stride=1, **kw):
        st = ps = sh = None
        out = []
        for l, (q, kp, vp) in enumerate(layers):
            role = roles[l] if roles is not None else po.stride_role(l, anchor_stride)
            role, a_state, s_state = fix(role, st, sh)
            r = po.decode_layer(l, q, kp, vp, bt, lens, anchor_stride=anchor_stride,
                                anchor_state=a_state, pool_state=ps, role=role,
                                shared_state=s_state, **kw)
            st, ps, sh = r["anchor_state"], r["pool_state"], r["shared_state"]
            out.append(r)
        return out
    return step


MUTANTS = {
    "bf16 widened by 15 bits": dict(
        bf16_to_f64=lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 15)
        .view(np.float32).astype(float)),
    "group mean instead of max": dict(relevance=lambda q, k: (k @ q.T).mean(axis=1)),
    "group sum instead of max": dict(relevance=lambda q, k: (k @ q.T).sum(axis=1)),
    "group min instead of max": dict(relevance=lambda q, k: (k @ q.T).min(axis=1)),
    "first head only": dict(relevance=lambda q, k: k @ q[0]),
    "negated score": dict(relevance=lambda q, k: -(k @ q.T).max(axis=1)),
    "ties to the higher position": dict(top_kappa=_topk_with(lambda s, p: (-p, -s))),
    "smallest instead of largest": dict(top_kappa=_topk_with(lambda s, p: (p, s))),
    "kappa-1 kept": dict(top_kappa=lambda s, k, p: oracle.top_kappa(s, k, p)[:-1]),
    "output in score order": dict(
        top_kappa=lambda s, k, p: np.asarray(p)[np.lexsort((np.asarray(p), -np.asarray(s)))[:k]]),
    "rank pool one short": dict(
        rank_pool=lambda s, p, r, k: oracle.rank_pool(s, p, r, k)[:-1]),
    "rank pool ignores rho": dict(rank_pool=lambda s, p, r, k: oracle.top_kappa(s, k, p)),
    "rank pool of the smallest": dict(
        rank_pool=lambda s, p, r, k: _topk_with(lambda a, b: (b, a))(s, min(r * k, len(p)), p)),
    "rank pool ties to the higher position": dict(
        rank_pool=lambda s, p, r, k: _topk_with(lambda a, b: (-b, -a))(s, min(r * k, len(p)), p)),
    "refinement keeps the pool's first kappa": dict(
        refine_in_pool=lambda q, kp, bt, g, pool, k, ps: (
            np.asarray(pool)[:k], oracle.relevance(q, oracle.cache_rows(kp, bt, g, pool, ps)))),
    "window w-1": dict(window_pool=_pool_with(lambda i, w: i - w + 1, lambda i, w: i + w - 1)),
    "window half open": dict(window_pool=_pool_with(lambda i, w: i - w, lambda i, w: i + w, 0)),
    "window left side only": dict(window_pool=_pool_with(lambda i, w: i - w, lambda i, w: i)),
    "window right side only": dict(window_pool=_pool_with(lambda i, w: i, lambda i, w: i + w)),
    "attention without scale": _attn_pair(lambda q, k, s: _softmax_rows(q @ k.T)),
    "attention scale squared": _attn_pair(lambda q, k, s: _softmax_rows(q @ k.T * s * s)),
    "softmax over heads": _attn_pair(lambda q, k, s: _softmax_rows((q @ k.T * s).T).T),
    "logits with a negated key": _attn_pair(lambda q, k, s: _softmax_rows(-(q @ k.T) * s)),
    "shared layers re-select": dict(
        layer_roles=lambda p, table4=False: ["R" if c == "S" else c
                                             for c in po.layer_roles(p, table4=table4)]),
    "table 4 refined letters read as shared": dict(
        layer_roles=lambda p, table4=False: po.layer_roles(p.replace("R", "X"), table4=False)),
    "shared layer takes the proposal layer's set": dict(
        decode_step=_step_with(lambda role, a, sh: (role, a, a if role == "S" else sh))),
    "refined layer expands the latest set": dict(
        decode_step=_step_with(lambda role, a, sh: (role, sh if role == "R" else a, sh))),
    "every layer a proposal layer": dict(
        decode_step=_step_with(lambda role, a, sh: ("F", a, sh))),
    "int2 scale over four levels": dict(quantize_int2=_quantize_with(levels=4)),
    "int2 zero point at the maximum": dict(
        quantize_int2=_quantize_with(zero=lambda kg: kg.max(axis=2))),
    "int2 codes truncated": dict(quantize_int2=_quantize_with(rnd=np.floor)),
    "int2 scale kept in float32": dict(quantize_int2=_quantize_with(bf16_scale=False)),
    "int2 groups of 16": dict(quantize_int2=_quantize_with(group=16)),
    "int2 groups of 64": dict(quantize_int2=_quantize_with(group=64)),
    "int2 groups interleaved": dict(
        quantize_int2=_quantize_with(
            order=lambda D: np.arange(D).reshape(32, D // 32).T.reshape(-1))),
    "int2 scores from the bare codes": dict(
        dequantize_int2=lambda c, a, b, group=32: np.asarray(c, dtype=np.float64)),
    "int2 dequantized without the zero point": dict(
        dequantize_int2=lambda c, a, b, group=32: po.dequantize_int2(c, a, np.zeros_like(b))),
    "dense decode drops the newest token": dict(
        dense_attend=lambda q, kp, vp, bt, g, L, ps, sc: po.attend(
            q, kp, vp, bt, g, np.arange(max(L - 1, 1)), ps, sc)),
    "dense decode without the scale": dict(
        dense_attend=lambda q, kp, vp, bt, g, L, ps, sc: po.attend(
            q, kp, vp, bt, g, np.arange(L), ps, 1.0)),
    "logical page ignores block table": dict(
        cache_rows=lambda pages, bt, g, pos, ps: po.bf16_to_f64(
            pages[np.asarray(pos) // ps, g, np.asarray(pos) % ps, :])),
    "row index off by one": dict(
        cache_rows=lambda pages, bt, g, pos, ps: po.bf16_to_f64(
            pages[np.asarray(bt)[np.asarray(pos) // ps], g, (np.asarray(pos) + 1) % ps, :])),
}


def test_unmutated_composition_passes():
    impl = _impl()
    for pin in pins.ALL_PINS:
        pin(impl)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    impl = _impl(**MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(impl)
        except Exception as e:   # an assertion or a crash both expose the mutant
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutant '{name}' passed every pin"
