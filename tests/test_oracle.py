"""The CPU oracle against its pins (brute force, closed forms, invariants, a
library routine, a hand-worked example) and the layer/step composition."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _decode_case():
    """Two KV heads, G = 2 (query heads 0,1 -> KV head 0; 2,3 -> KV head 1).
    KV head 1 holds the negated anchor keys and its query heads are the negated
    ones of KV head 0, so with consecutive grouping both heads select the same
    set; interleaved grouping (j % Hkv) would not."""
    g = pins.GOLDEN
    ka, kr = np.array(g["anchor"]["keys"], float), np.array(g["refined"]["keys"], float)
    q = np.array([[1, 0], [0, 1], [-1, 0], [0, -1]], dtype=np.float32)
    q_bits = (q.view(np.uint32) >> 16).astype(np.uint16)[None]          # [1, 4, 2]
    layers_rows = [np.stack([ka, -ka]), np.stack([kr, -kr]), np.stack([kr, -kr])]
    ps, L = 2, 8
    bt = np.array([[3, 0, 2, 1]], dtype=np.int32)
    rng = np.random.default_rng(5)
    layers = []
    for rows in layers_rows:
        kp = np.zeros((4, 2, ps, 2), np.uint16)
        vp = np.zeros_like(kp)
        vals = np.round(rng.standard_normal((2, L, 2)) * 8) / 8
        for h in range(2):
            kb = (rows[h].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            vb = (vals[h].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for p in range(4):
                kp[bt[0, p], h] = kb[p * ps:(p + 1) * ps]
                vp[bt[0, p], h] = vb[p * ps:(p + 1) * ps]
        layers.append((q_bits, kp, vp))
    return layers, bt, np.array([L], np.int32)


def test_decode_step_roles_grouping_and_anchor_state():
    layers, bt, lens = _decode_case()
    res = oracle.decode_step(layers, bt, lens, num_kv_heads=2, kappa=3, anchor_stride=3,
                             window=1, page_size=2)
    want = [[0, 2, 5], [1, 3, 6], [1, 3, 6]]   # layer 2 expands layer 0's set, not layer 1's
    for l, r in enumerate(res):
        for h in range(2):
            assert list(r["selected"][0, h]) == want[l], (l, h)
    # chained from layer 1 instead, layer 2's pool would reach position 7 -> {1, 6, 7}
    assert list(res[2]["pools"][(0, 0)]) == list(range(7))


def test_decode_layer_output_is_attention_over_selected():
    layers, bt, lens = _decode_case()
    res = oracle.decode_step(layers, bt, lens, num_kv_heads=2, kappa=3, anchor_stride=3,
                             window=1, page_size=2)
    for l, (qb, kp, vp) in enumerate(layers):
        q = oracle.bf16_to_f64(qb)[0]
        for h in range(2):
            sel = res[l]["selected"][0, h]
            k = oracle.cache_rows(kp, bt[0], h, sel, 2)
            v = oracle.cache_rows(vp, bt[0], h, sel, 2)
            o = oracle.sparse_attention(q[2 * h:2 * h + 2], k, v, 1 / np.sqrt(2))
            np.testing.assert_allclose(res[l]["out"][0, 2 * h:2 * h + 2], o, rtol=1e-14)


def test_kappa_equals_length_is_dense_attention():
    import torch
    import torch.nn.functional as F
    layers, bt, lens = _decode_case()
    res = oracle.decode_layer(0, *layers[0], bt, lens, num_kv_heads=2, kappa=8,
                              anchor_stride=1, window=0, page_size=2)
    qb, kp, vp = layers[0]
    q = oracle.bf16_to_f64(qb)[0]
    for h in range(2):
        k = torch.tensor(oracle.cache_rows(kp, bt[0], h, np.arange(8), 2))
        v = torch.tensor(oracle.cache_rows(vp, bt[0], h, np.arange(8), 2))
        tq = torch.tensor(q[2 * h:2 * h + 2])[None, :, None, :]
        ref = F.scaled_dot_product_attention(tq, k[None, None].expand(1, 2, 8, 2),
                                             v[None, None].expand(1, 2, 8, 2),
                                             scale=1 / np.sqrt(2))[0, :, 0, :].numpy()
        np.testing.assert_allclose(res["out"][0, 2 * h:2 * h + 2], ref, rtol=1e-12)


def test_refined_layer_requires_anchor_state():
    layers, bt, lens = _decode_case()
    with pytest.raises(ValueError):
        oracle.decode_layer(1, *layers[1], bt, lens, num_kv_heads=2, kappa=3, anchor_stride=3,
                            window=1, page_size=2)


def test_decode_step_rank_pool():
    """pool_rho >= 1: the refined layers re-score the anchor layer's top
    rho*kappa tokens (Eq. 4).  In the hand example the anchor scores
    [3, 1, 4, -1, 2, 3, 0, 1] give the pool {0, 1, 2, 4, 5, 7} at rho = 2,
    kappa = 3 (1 and 7 tie at score 1 and both fit); the refined scores
    [0, 5, 1, 2, 0, 1, 6, 9] over that pool select {1, 2, 7}: position 6, the
    refined layer's second best, lies outside the pool, and 2 beats 5 on the
    tie at score 1."""
    layers, bt, lens = _decode_case()
    res = oracle.decode_step(layers, bt, lens, num_kv_heads=2, kappa=3, anchor_stride=3,
                             window=1, page_size=2, pool_rho=2)
    for h in range(2):
        assert list(res[0]["selected"][0, h]) == [0, 2, 5]
        for l in (1, 2):
            assert list(res[l]["pools"][(0, h)]) == [0, 1, 2, 4, 5, 7]
            assert list(res[l]["selected"][0, h]) == [1, 2, 7]
    with pytest.raises(ValueError):   # a refined layer needs the anchor's pools
        oracle.decode_layer(1, *layers[1], bt, lens, num_kv_heads=2, kappa=3, anchor_stride=3,
                            window=1, page_size=2, anchor_state=res[0]["anchor_state"],
                            pool_rho=2)


def test_decode_step_layer_roles_hand():
    """Explicit roles on the hand example (anchor scores [3, 1, 4, -1, 2, 3, 0,
    1], refined scores [0, 5, 1, 2, 0, 1, 6, 9], kappa = 3, w = 1).  FSR: the
    shared layer 1 attends over layer 0's set {0, 2, 5} with its own keys and
    values; the refined layer 2 still expands layer 0's set (pool 0..6) and
    keeps {1, 3, 6}.  FRS: layer 2 reuses layer 1's refined set {1, 3, 6}.
    FFS: layer 1 is a proposal layer over the whole cache ({1, 6, 7}) and
    layer 2 reuses that."""
    layers, bt, lens = _decode_case()
    kw = dict(num_kv_heads=2, kappa=3, anchor_stride=1, window=1, page_size=2)
    for pattern, want in (("FSR", [[0, 2, 5], [0, 2, 5], [1, 3, 6]]),
                          ("FRS", [[0, 2, 5], [1, 3, 6], [1, 3, 6]]),
                          ("FFS", [[0, 2, 5], [1, 6, 7], [1, 6, 7]])):
        res = oracle.decode_step(layers, bt, lens, roles=oracle.layer_roles(pattern), **kw)
        for l, r in enumerate(res):
            for h in range(2):
                assert list(r["selected"][0, h]) == want[l], (pattern, l, h)
        # the shared layer's output is attention over the reused set with its own K, V
        ls = pattern.index("S")
        qb, kp, vp = layers[ls]
        q = oracle.bf16_to_f64(qb)[0]
        o = oracle.attend(q[0:2], kp, vp, bt[0], 0, res[ls]["selected"][0, 0], 2,
                          oracle.default_scale(2))
        np.testing.assert_allclose(res[ls]["out"][0, 0:2], o, rtol=1e-14)
        assert not res[ls]["scores"]
    with pytest.raises(ValueError):   # a shared layer needs a preceding set
        oracle.decode_layer(1, *layers[1], bt, lens, role="S", **kw)
