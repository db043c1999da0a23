"""Checks that pin the CPU oracle to facts fixed independently of it: brute
force on tiny inputs, closed forms, invariants, a library routine for dense
attention and a hand-worked example (tests/golden/hand_example.json).

Each check takes the implementation under test as a namespace, so the same
checks run against the oracle (they must pass) and against deliberately broken
copies of it (each must be caught by at least one check).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

_GOLDEN_PATH = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")
with open(_GOLDEN_PATH) as _f:
    GOLDEN = json.load(_f)
_PATTERNS_PATH = os.path.join(os.path.dirname(__file__), "golden", "layer_patterns.json")
with open(_PATTERNS_PATH) as _f:
    PATTERNS = json.load(_f)


def _arr(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------- bf16
def pin_bf16_decode(impl):
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0, 0x3F00: 0.5, 0x0000: 0.0,
             0x7F7F: 3.3895313892515355e38, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x3FC0: 1.5, 0x3F81: 1.0 + 2.0 ** -7, 0x4248: 50.0}
    got = impl.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(cases.values()))), got
    neg0 = impl.bf16_to_f64(np.array([0x8000], dtype=np.uint16))
    assert neg0[0] == 0.0 and math.copysign(1.0, neg0[0]) < 0


# ---------------------------------------------------------------- relevance
def pin_relevance_bruteforce(impl, seed=11):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        G, D, n = int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.integers(1, 12))
        q = rng.integers(-9, 10, size=(G, D))
        k = rng.integers(-9, 10, size=(n, D))
        want = []
        for i in range(n):
            dots = [sum(int(q[j, t]) * int(k[i, t]) for t in range(D)) for j in range(G)]
            want.append(max(dots))
        got = impl.relevance(_arr(q), _arr(k))
        assert got.shape == (n,) and np.array_equal(got, _arr(want)), (got, want)
    for _ in range(20):   # real-valued: compare with exactly rounded sums
        G, D, n = int(rng.integers(1, 5)), 16, int(rng.integers(1, 8))
        q, k = rng.standard_normal((G, D)), rng.standard_normal((n, D))
        want = [max(math.fsum(q[j, t] * k[i, t] for t in range(D)) for j in range(G))
                for i in range(n)]
        np.testing.assert_allclose(impl.relevance(q, k), want, rtol=1e-12, atol=1e-12)


def pin_relevance_hand(impl):
    q = _arr(GOLDEN["q_group"])
    for part in ("anchor", "refined"):
        got = impl.relevance(q, _arr(GOLDEN[part]["keys"]))
        assert np.array_equal(got, _arr(GOLDEN[part]["scores"])), (part, got)


# --------------------------------------------------------------------- TopK
def _brute_topk(scores, kappa, pos):
    """Among all kappa-subsets, the largest score sum; among those, the
    lexicographically smallest ascending position tuple (= lower position wins
    ties at the threshold)."""
    best = None
    for comb in itertools.combinations(range(len(scores)), kappa):
        key = (-sum(scores[c] for c in comb), sorted(int(pos[c]) for c in comb))
        if best is None or key < best:
            best = key
    return best[1]


def pin_topk_exhaustive(impl, seed=12):
    rng = np.random.default_rng(seed)
    for _ in range(120):
        n = int(rng.integers(1, 9))
        scores = rng.integers(-2, 3, size=n)            # heavy ties
        pos = rng.permutation(40)[:n]                   # arbitrary distinct labels
        for kappa in range(1, n + 1):
            got = impl.top_kappa(_arr(scores), kappa, pos)
            assert list(map(int, got)) == _brute_topk(list(map(int, scores)), kappa, pos), \
                (scores, pos, kappa, got)


def pin_topk_invariants(impl, seed=13):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        n = int(rng.integers(2, 300))
        s = np.round(rng.standard_normal(n), 1)          # ties at 0.1 resolution
        pos = np.sort(rng.choice(10 * n, size=n, replace=False))
        kappa = int(rng.integers(1, n + 1))
        t = np.asarray(impl.top_kappa(s, kappa, pos))
        assert t.shape == (kappa,)
        assert np.all(np.diff(t) > 0), "ascending, no duplicates"
        assert np.isin(t, pos).all()
        sel = np.isin(pos, t)
        if kappa < n:
            lo, hi = s[sel].min(), s[~sel].max()
            assert lo >= hi
            if lo == hi:   # equal scores at the threshold: lower positions win
                assert pos[sel & (s == lo)].max() < pos[~sel & (s == hi)].min()


def pin_topk_hand(impl):
    s = _arr(GOLDEN["anchor"]["scores"])
    pos = np.arange(len(s))
    for k, want in GOLDEN["anchor"]["topk"].items():
        assert list(map(int, impl.top_kappa(s, int(k), pos))) == want, k


# --------------------------------------------------------------------- pool
def pin_pool_bruteforce(impl, seed=14):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        L = int(rng.integers(1, 50))
        kappa = int(rng.integers(1, L + 1))
        A = np.sort(rng.choice(L, size=kappa, replace=False))
        for w in (0, 1, 2, 3, 7, L - 1, L + 5):
            want = sorted({t for i in A for t in range(i - w, i + w + 1) if 0 <= t < L})
            got = impl.window_pool(A, w, L)
            assert list(map(int, got)) == want, (L, A, w)
            assert len(got) <= min(L, kappa * (2 * w + 1))
            assert np.isin(A, got).all()
            if w >= L - 1:
                assert list(map(int, got)) == list(range(L))
            if w == 0:
                assert list(map(int, got)) == list(map(int, A))


def pin_pool_hand(impl):
    A = GOLDEN["anchor"]["topk"]["3"]
    for w, want in GOLDEN["pool_of_anchor_top3"].items():
        if w == "derivation":
            continue
        assert list(map(int, impl.window_pool(np.array(A), int(w), 8))) == want, w


# --------------------------------------------------------------- refinement
def _tiny_paged(rows_per_layer, page_size=2, hkv=1, seed=0):
    """Pack per-layer key rows [L, D] (float, exactly bf16-representable) into a
    paged cache with a shuffled block table.  Returns (pages list, block_table)."""
    rng = np.random.default_rng(seed)
    L, D = np.asarray(rows_per_layer[0]).shape
    npg = (L + page_size - 1) // page_size
    perm = rng.permutation(npg + 3)[:npg]
    out = []
    for rows in rows_per_layer:
        bits = (np.asarray(rows, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        pages = np.zeros((npg + 3, hkv, page_size, D), dtype=np.uint16)
        for p in range(npg):
            chunk = bits[p * page_size:(p + 1) * page_size]
            pages[perm[p], 0, :len(chunk)] = chunk
        out.append(pages)
    return out, perm.astype(np.int32)


def pin_refine_hand(impl):
    q = _arr(GOLDEN["q_group"])
    (pa, pr), bt = _tiny_paged([GOLDEN["anchor"]["keys"], GOLDEN["refined"]["keys"]])
    A, s = impl.anchor_select(q, pa, bt, 0, 8, 3, 2)
    assert list(map(int, A)) == GOLDEN["anchor"]["topk"]["3"]
    assert np.array_equal(s, _arr(GOLDEN["anchor"]["scores"]))
    for w, want in GOLDEN["refined"]["refined_top3"].items():
        t, pool, _ = impl.refined_select(q, pr, bt, 0, 8, 3, 2, A, int(w))
        assert list(map(int, t)) == want, w
    ex, _ = impl.anchor_select(q, pr, bt, 0, 8, 3, 2)
    assert list(map(int, ex)) == GOLDEN["refined"]["exact_top3"]


def pin_refine_limits(impl, seed=15):
    """w >= L-1 makes refinement the exact TopK; w = 0 reproduces static reuse
    (Eq. 3) whenever the pool is exactly the anchor set."""
    rng = np.random.default_rng(seed)
    for _ in range(25):
        L, D, G = int(rng.integers(4, 60)), 4, int(rng.integers(1, 4))
        kappa = int(rng.integers(1, L + 1))
        ra = np.round(rng.standard_normal((L, D)) * 4) / 4
        rr = np.round(rng.standard_normal((L, D)) * 4) / 4
        (pa, pr), bt = _tiny_paged([ra, rr], page_size=4, seed=int(rng.integers(1000)))
        q = np.round(rng.standard_normal((G, D)) * 4) / 4
        A, _ = impl.anchor_select(q, pa, bt, 0, L, kappa, 4)
        exact, _ = impl.anchor_select(q, pr, bt, 0, L, kappa, 4)
        t_full, _, _ = impl.refined_select(q, pr, bt, 0, L, kappa, 4, A, L - 1)
        assert np.array_equal(t_full, exact)
        t0, pool0, _ = impl.refined_select(q, pr, bt, 0, L, kappa, 4, A, 0)
        assert np.array_equal(t0, A) and np.array_equal(pool0, A)


# ---------------------------------------------------------------- rank pool
def pin_rank_pool_exhaustive(impl, seed=19):
    """Eq. 4: the pool is the rho*kappa best of the anchor's scores (ties to the
    lower position), every candidate when rho*kappa exceeds their number;
    against the exhaustive subset search."""
    rng = np.random.default_rng(seed)
    for _ in range(60):
        n = int(rng.integers(1, 9))
        scores = rng.integers(-2, 3, size=n)            # heavy ties
        pos = rng.permutation(40)[:n]
        for kappa in range(1, n + 1):
            for rho in (1, 2, 3, 9):
                got = impl.rank_pool(_arr(scores), pos, rho, kappa)
                want = _brute_topk(list(map(int, scores)), min(rho * kappa, n), pos)
                assert list(map(int, got)) == want, (scores, pos, rho, kappa, got)


def pin_rank_pool_structure(impl, seed=20):
    """The anchor's own set lies inside its pool, and the pool grows with rho;
    every pool token outscores every other under the anchor's scores; rho = 1
    hands over the set itself, so a refined layer reuses it (Eq. 3); a pool
    covering the cache makes refinement the exact TopK of the refined layer."""
    rng = np.random.default_rng(seed)
    for _ in range(25):
        L, D, G = int(rng.integers(4, 60)), 4, int(rng.integers(1, 4))
        kappa = int(rng.integers(1, L + 1))
        ra = np.round(rng.standard_normal((L, D)) * 4) / 4
        rr = np.round(rng.standard_normal((L, D)) * 4) / 4
        (pa, pr), bt = _tiny_paged([ra, rr], page_size=4, seed=int(rng.integers(1000)))
        qa = np.round(rng.standard_normal((G, D)) * 4) / 4
        qr = np.round(rng.standard_normal((G, D)) * 4) / 4
        A, s = impl.anchor_select(qa, pa, bt, 0, L, kappa, 4)
        pos = np.arange(L)
        prev = None
        for rho in (1, 2, 3, L):
            C = np.asarray(impl.rank_pool(s, pos, rho, kappa))
            assert C.shape == (min(rho * kappa, L),)
            assert np.all(np.diff(C) > 0)
            assert np.isin(A, C).all()
            if prev is not None:
                assert np.isin(prev, C).all()
            prev = C
            rest = np.setdiff1d(pos, C)
            if rest.size:
                assert s[C].min() >= s[rest].max()
            t, _ = impl.refine_in_pool(qr, pr, bt, 0, C, kappa, 4)
            if rho == 1:
                assert np.array_equal(t, A)
            if rho * kappa >= L:
                exact, _ = impl.anchor_select(qr, pr, bt, 0, L, kappa, 4)
                assert np.array_equal(t, exact)


# ---------------------------------------------------------------- attention
def pin_attention_dense_library(impl, seed=16):
    """kappa = L: sparse attention over every token equals dense attention, here
    PyTorch's scaled_dot_product_attention in float64 on the CPU."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for _ in range(10):
        G, D, n = int(rng.integers(1, 9)), int(rng.choice([8, 64, 128])), int(rng.integers(1, 300))
        qg, k, v = (rng.standard_normal((G, D)), rng.standard_normal((n, D)),
                    rng.standard_normal((n, D)))
        scale = 1.0 / math.sqrt(D)
        tq = torch.tensor(qg)[None, :, None, :]
        tk = torch.tensor(k)[None, None].expand(1, G, n, D)
        tv = torch.tensor(v)[None, None].expand(1, G, n, D)
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0, :].numpy()
        np.testing.assert_allclose(impl.sparse_attention(qg, k, v, scale), ref,
                                   rtol=1e-10, atol=1e-12)


def pin_attention_closed_forms(impl, seed=17):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        G, D = int(rng.integers(1, 5)), int(rng.integers(1, 17))
        qg = rng.standard_normal((G, D)) * 3
        k1, v1 = rng.standard_normal((1, D)), rng.standard_normal((1, D))
        # one token: the output is that token's value row for every head
        assert np.allclose(impl.sparse_attention(qg, k1, v1, 0.3), np.repeat(v1, G, 0),
                           rtol=0, atol=1e-15)
        # two tokens: weights are the logistic function of the logit difference
        k2, v2 = rng.standard_normal((2, D)), rng.standard_normal((2, D))
        sc = float(rng.uniform(0.05, 1.0))
        dz = sc * (qg @ k2[0] - qg @ k2[1])
        w0 = 1.0 / (1.0 + np.exp(-dz))
        want = w0[:, None] * v2[0] + (1 - w0)[:, None] * v2[1]
        np.testing.assert_allclose(impl.sparse_attention(qg, k2, v2, sc), want, rtol=1e-12,
                                   atol=1e-13)
        # weights are a distribution; output does not depend on token order
        n = int(rng.integers(2, 50))
        k, v = rng.standard_normal((n, D)), rng.standard_normal((n, D))
        wts = impl.attention_weights(qg, k, sc)
        assert wts.shape == (G, n) and np.all(wts >= 0)
        np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        perm = rng.permutation(n)
        np.testing.assert_allclose(impl.sparse_attention(qg, k[perm], v[perm], sc),
                                   impl.sparse_attention(qg, k, v, sc), rtol=1e-12, atol=1e-13)


def pin_attention_hand(impl):
    a = GOLDEN["attention"]
    scale = math.log(3.0) / 2.0
    q, k, v = _arr(a["q_group"]), _arr(a["keys"]), _arr(a["values"])
    np.testing.assert_allclose(impl.attention_weights(q, k, scale), a["weights"], rtol=1e-14)
    np.testing.assert_allclose(impl.sparse_attention(q, k, v, scale), a["out"], rtol=1e-14)


# ------------------------------------------------------------- paged cache
def pin_cache_rows(impl):
    """The paged gather returns exactly the rows the generator produced for
    that (sequence, KV head) before paging."""
    import synth
    wl = synth.scaled(synth.BATCHED_16, name="paging-pin", wid=901, batch=3, num_q_heads=4,
                      num_kv_heads=2, len_range=(128, 640), num_layers=1)
    li = synth.layer_inputs(wl, 0, threads=1)
    pg = synth.paging(wl)
    rng = np.random.default_rng(18)
    for b in range(wl.batch):
        L = int(pg.seq_lens[b])
        for g in range(wl.num_kv_heads):
            kb, vb = synth.kv_head(wl, 0, b, g, L, li.q)
            pos = rng.choice(L, size=min(L, 50), replace=False)
            want_k = synth.bf16_bits_to_f32(kb[pos]).astype(np.float64)
            want_v = synth.bf16_bits_to_f32(vb[pos]).astype(np.float64)
            assert np.array_equal(impl.cache_rows(li.k_pages, pg.block_table[b], g, pos,
                                                  wl.page_size), want_k)
            assert np.array_equal(impl.cache_rows(li.v_pages, pg.block_table[b], g, pos,
                                                  wl.page_size), want_v)


# ------------------------------------------------------------ INT2 keys
def _bf16_round(x):
    """Nearest bf16 value of float64 x (through float32), as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
            .view(np.float32).astype(np.float64))


def pin_int2_exact_levels(impl, seed=22):
    """A 32-dimension group whose values lie exactly on beta + alpha * c,
    c in {0, 1, 2, 3}, with both end levels present and alpha a power of two,
    quantizes to exactly those codes, scale and zero point (Eq. 8), and
    dequantizes to itself; a constant group gets scale 0 and codes 0."""
    rng = np.random.default_rng(seed)
    for _ in range(40):
        n, M = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        c = rng.integers(0, 4, size=(n, M, 32))
        c[:, :, 0], c[:, :, 1] = 0, 3
        alpha = 2.0 ** rng.integers(-6, 5, size=(n, M))
        beta = alpha * rng.integers(-60, 61, size=(n, M))   # on alpha's grid: 7 bits suffice
        k = (alpha[..., None] * c + beta[..., None]).reshape(n, M * 32)
        assert np.array_equal(_bf16_round(k), k)
        codes, a, b = impl.quantize_int2(_bits(k))
        assert np.array_equal(codes, c.reshape(n, M * 32)), "codes"
        assert np.array_equal(a, alpha) and np.array_equal(b, beta)
        assert np.array_equal(impl.dequantize_int2(codes, a, b), k)
    k = np.zeros((1, 32))                     # -0 and +0 mixed: the zero point is +0
    k[0, ::3] = -0.0
    k[0, 5] = 3.0
    codes, a, b = impl.quantize_int2(_bits(k))
    assert b[0, 0] == 0.0 and math.copysign(1.0, b[0, 0]) > 0 and a[0, 0] == 1.0
    assert codes[0, 5] == 3 and codes[0].sum() == 3
    k = np.array([[0.0, 3.0, 0.5, 1.5, 2.5] + [0.0] * 27])   # exact midpoints go to even codes
    codes, a, b = impl.quantize_int2(_bits(k))
    assert list(codes[0, :5]) == [0, 3, 0, 2, 2] and a[0, 0] == 1.0
    k = np.repeat(np.array([[1.5, -2.0, 0.0, 3.25]]), 32, axis=1)   # four constant groups
    codes, a, b = impl.quantize_int2(_bits(k))
    assert not codes.any() and not a.any() and list(b[0]) == [1.5, -2.0, 0.0, 3.25]
    assert np.array_equal(impl.dequantize_int2(codes, a, b), k)


def pin_int2_nearest_level(impl, seed=23):
    """On random keys: beta is the group minimum; alpha is a bf16 value within
    half a bf16 step of (max - min) / 3; every code picks a nearest level of
    beta + alpha * {0, 1, 2, 3} (exact arithmetic, up to float32's decision
    tolerance); dequantization is within alpha / 2 of the key (plus the top
    level's shortfall when alpha rounds down); groups are the consecutive
    32-dimension blocks (a change in one block leaves the others alone)."""
    rng = np.random.default_rng(seed)
    for _ in range(30):
        n = int(rng.integers(1, 6))
        k = _bf16_round(rng.standard_normal((n, 128)) * float(rng.choice([0.01, 1.0, 30.0])))
        codes, a, b = impl.quantize_int2(_bits(k))
        assert codes.shape == (n, 128) and a.shape == b.shape == (n, 4)
        assert codes.max() <= 3
        kg = k.reshape(n, 4, 32)
        mn, mx = kg.min(axis=2), kg.max(axis=2)
        assert np.array_equal(b, mn)
        assert np.array_equal(_bf16_round(a), a)
        third = (mx - mn) / 3.0
        assert np.all(np.abs(a - third) <= third * 2.0 ** -8 * 1.0001)   # half a bf16 step
        lev = b[..., None, None] + a[..., None, None] * np.arange(4)        # [n, 4, 1, 4]
        dist = np.abs(kg[..., None] - lev)                                   # [n, 4, 32, 4]
        chosen = np.take_along_axis(dist, codes.reshape(n, 4, 32, 1).astype(np.int64), 3)[..., 0]
        assert np.all(chosen <= dist.min(axis=3) + a[..., None] * 2.0 ** -20)
        err = np.abs(impl.dequantize_int2(codes, a, b).reshape(n, 4, 32) - kg)
        bound = a / 2 + 3 * np.maximum(third - a, 0) + a * 2.0 ** -20
        assert np.all(err <= bound[..., None]), err.max()
        d = int(rng.integers(0, 128))
        k2 = k.copy()
        k2[0, d] = -k2[0, d] * 3 - 1
        k2 = _bf16_round(k2)
        c2, a2, b2 = impl.quantize_int2(_bits(k2))
        keep = [m for m in range(4) if m != d // 32]
        assert np.array_equal(a2[0, keep], a[0, keep]) and np.array_equal(b2[0, keep], b[0, keep])
        cols = [i for i in range(128) if i // 32 != d // 32]
        assert np.array_equal(c2[0, cols], codes[0, cols])


def pin_int2_relevance(impl, seed=24):
    """Relevance on INT2 keys (Eq. 9) is the group maximum of <q_j, k-hat_i>
    with k-hat = alpha * code + beta: brute-force loops over the quantizer's
    own output on tiny paged caches, the anchor set by exhaustive TopK, and the
    refined layer's pool scores likewise; keys already on their levels score
    exactly as the bf16 keys do."""
    rng = np.random.default_rng(seed)
    for trial in range(12):
        L, G, D = int(rng.integers(3, 8)), int(rng.integers(1, 3)), 64
        kappa = int(rng.integers(1, min(3, L) + 1))
        k = _bf16_round(rng.standard_normal((L, D)) * 2)
        q = _bf16_round(rng.standard_normal((G, D)))
        (kp,), bt = _tiny_paged([k], page_size=2, seed=trial)
        codes, a, b = impl.quantize_int2(_bits(k))
        want = [max(math.fsum(q[j, d] * (a[i, d // 32] * int(codes[i, d]) + b[i, d // 32])
                              for d in range(D)) for j in range(G)) for i in range(L)]
        sel, s = impl.anchor_select(q, kp, bt, 0, L, kappa, 2, int2=True)
        np.testing.assert_allclose(s, want, rtol=1e-12, atol=1e-12)
        assert list(map(int, sel)) == _brute_topk(want, kappa, list(range(L)))
        pool = np.sort(rng.choice(L, size=int(rng.integers(kappa, L + 1)), replace=False))
        t, sp = impl.refine_in_pool(q, kp, bt, 0, pool, kappa, 2, int2=True)
        np.testing.assert_allclose(sp, [want[i] for i in pool], rtol=1e-12, atol=1e-12)
        # on-level keys: alpha = 1/2, beta = -1, so quantization loses nothing
        c = rng.integers(0, 4, size=(L, 2, 32))
        c[:, :, 0], c[:, :, 1] = 0, 3
        kl = (0.5 * c - 1.0).reshape(L, D)
        (kpl,), btl = _tiny_paged([kl], page_size=2, seed=trial)
        s_int2 = impl.anchor_select(q, kpl, btl, 0, L, kappa, 2, int2=True)[1]
        s_bf16 = impl.anchor_select(q, kpl, btl, 0, L, kappa, 2)[1]
        np.testing.assert_allclose(s_int2, s_bf16, rtol=1e-12, atol=1e-12)


def pin_dense_attend_library(impl, seed=25):
    """Dense decode over a paged cache equals torch's scaled_dot_product_attention
    in float64 on the CPU over the sequence's rows in position order."""
    import torch
    rng = np.random.default_rng(seed)
    for trial in range(8):
        L, G, D = int(rng.integers(1, 40)), int(rng.integers(1, 4)), 8
        k = _bf16_round(rng.standard_normal((L, D)))
        v = _bf16_round(rng.standard_normal((L, D)))
        q = _bf16_round(rng.standard_normal((G, D)))
        (kp, vp), bt = _tiny_paged([k, v], page_size=4, seed=trial)
        scale = 1.0 / math.sqrt(D)
        got = impl.dense_attend(q, kp, vp, bt, 0, L, 4, scale)
        qt = torch.from_numpy(q)[:, None, :].double()                       # [G, 1, D]
        kt = torch.from_numpy(k)[None].double().expand(G, L, D)
        vt = torch.from_numpy(v)[None].double().expand(G, L, D)
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0]
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- layer roles
def pin_layer_patterns(impl):
    """The pages' printed patterns under their own letters: every Table 4
    pattern has one proposal layer per 'group' layers (Table 3's caption) and
    no shared layer once its S is read as refined; Table 9's configuration
    names give each role's count over GLM-5.2's 78 layers."""
    for name, e in PATTERNS["table4"]["patterns"].items():
        roles = impl.layer_roles(e["pattern"], table4=True)
        assert len(roles) == len(e["pattern"]) and set(roles) <= {"F", "R"}, name
        assert roles[0] == "F" and roles.count("F") * e["group"] == len(roles), (name, roles)
    for name, e in PATTERNS["table9"]["patterns"].items():
        roles = impl.layer_roles(e["pattern"])
        assert len(roles) == PATTERNS["table9"]["layers"], name
        assert {c: roles.count(c) for c in "FRS"} == {c: e[c] for c in "FRS"}, name
    for bad, t4 in (("", False), ("RFS", False), ("SF", False), ("FX", False), ("FR", True)):
        try:
            impl.layer_roles(bad, table4=t4)
        except ValueError:
            continue
        raise AssertionError(f"pattern {bad!r} accepted")
    assert [impl.stride_role(l, 3) for l in range(7)] == list("FRRFRRF")


def _bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _brute_step(pattern, qs, ks, vs, kappa, w, rho):
    """Sets and outputs of a layer-role pattern from its definition: F selects
    its own top-kappa over the whole cache; R re-selects within the pool of
    the nearest preceding F (the +-w windows of F's set, or F's top rho*kappa
    when rho >= 1); S reuses the set of the nearest preceding F or R layer.
    Brute-force scores, TopK and attention in plain Python."""
    L, D = len(ks[0]), len(ks[0][0])
    scale = 1.0 / math.sqrt(D)
    f_set = f_scores = last = None
    sets, outs = [], []
    for l, role in enumerate(pattern):
        q, k, v = qs[l], ks[l], vs[l]
        s = [max(math.fsum(q[j][d] * k[i][d] for d in range(D)) for j in range(len(q)))
             for i in range(L)]
        if role == "F":
            t = _brute_topk(s, kappa, list(range(L)))
            f_set, f_scores = t, s
        elif role == "R":
            if rho >= 1:
                pool = _brute_topk(f_scores, min(rho * kappa, L), list(range(L)))
            else:
                pool = sorted({p for a in f_set for p in range(max(0, a - w), min(L - 1, a + w) + 1)})
            t = _brute_topk([s[p] for p in pool], kappa, pool)
        else:
            t = list(last)
        if role != "S":
            last = t
        out = []
        for j in range(len(q)):
            z = [scale * math.fsum(q[j][d] * k[i][d] for d in range(D)) for i in t]
            m = max(z)
            e = [math.exp(x - m) for x in z]
            tot = math.fsum(e)
            out.append([math.fsum(e[n] * v[i][d] for n, i in enumerate(t)) / tot
                        for d in range(D)])
        sets.append(t)
        outs.append(out)
    return sets, outs


def pin_pattern_composition(impl, seed=21):
    """decode_step over random F/R/S patterns (and a stride) equals the
    brute-force reading of the roles on tiny caches, for the window pool and
    the rank-expanded pool."""
    rng = np.random.default_rng(seed)
    for trial in range(32):
        L, D, G = int(rng.integers(5, 14)), 4, int(rng.integers(1, 3))
        kappa = int(rng.integers(1, min(3, L) + 1))
        w, rho = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        stride = None
        if trial % 4 == 3:
            stride = int(rng.integers(2, 4))
            pattern = [impl.stride_role(l, stride) for l in range(6)]
        elif trial % 4 == 2:   # refined layers in a row: each expands the proposal's set
            w, rho, kappa = 1, 0, 2
            pattern = list("FRRSRS")
        else:
            pattern = ["F"] + list(rng.choice(list("FRS"), size=5, p=[0.2, 0.4, 0.4]))
        n = len(pattern)
        ks = [np.round(rng.standard_normal((L, D)) * 3) / 2 for _ in range(n)]
        vs = [np.round(rng.standard_normal((L, D)) * 4) / 4 for _ in range(n)]
        qs = [np.round(rng.standard_normal((G, D)) * 3) / 2 for _ in range(n)]
        pages, bt = _tiny_paged(ks + vs, page_size=2, seed=int(rng.integers(1000)))
        layers = [(_bits(qs[l])[None], pages[l], pages[n + l]) for l in range(n)]
        kw = dict(num_kv_heads=1, kappa=kappa, window=w, page_size=2, pool_rho=rho)
        if stride is None:
            res = impl.decode_step(layers, bt[None], np.array([L]), anchor_stride=1,
                                   roles=impl.layer_roles("".join(pattern)), **kw)
        else:
            res = impl.decode_step(layers, bt[None], np.array([L]), anchor_stride=stride, **kw)
        sets, outs = _brute_step(pattern, qs, ks, vs, kappa, w, rho)
        for l in range(n):
            got = list(map(int, res[l]["selected"][0, 0]))
            assert got == sets[l], (trial, "".join(pattern), l, got, sets[l])
            np.testing.assert_allclose(res[l]["out"][0], outs[l], rtol=1e-12, atol=1e-12)


ALL_PINS = [pin_bf16_decode, pin_relevance_bruteforce, pin_relevance_hand, pin_topk_exhaustive,
            pin_topk_invariants, pin_topk_hand, pin_pool_bruteforce, pin_pool_hand,
            pin_refine_hand, pin_refine_limits, pin_rank_pool_exhaustive,
            pin_rank_pool_structure, pin_attention_dense_library,
            pin_attention_closed_forms, pin_attention_hand, pin_cache_rows,
            pin_layer_patterns, pin_pattern_composition, pin_int2_exact_levels,
            pin_int2_nearest_level, pin_int2_relevance, pin_dense_attend_library]
