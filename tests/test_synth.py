"""The input generator: determinism, shapes, paging, RoPE and the planted
structure of the 128K workloads."""
import numpy as np

import synth


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -9,
                  3.0, 1 + 2.0 ** -7], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, -1.0, 1.0, 3.0, 1 + 2.0 ** -7], dtype=np.float32)
    assert np.array_equal(got, want)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(0)
    L, D, base = 300, 128, 500000.0
    x = rng.standard_normal((L, D)).astype(np.float32)
    y = synth.apply_rope(x, base)
    m = np.arange(L)[:, None]
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]).astype(np.complex128) * np.exp(1j * m * theta)
    np.testing.assert_allclose(y[:, :D // 2], z.real, atol=2e-5)
    np.testing.assert_allclose(y[:, D // 2:], z.imag, atol=2e-5)
    assert np.array_equal(y[0], x[0])                      # position 0 is the identity
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)


def test_layer_is_deterministic_and_layers_differ():
    wl = synth.TINY_4K
    a, b = synth.layer_inputs(wl, 0), synth.layer_inputs(wl, 0, threads=1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_pages, b.k_pages)
    assert np.array_equal(a.v_pages, b.v_pages)
    c = synth.layer_inputs(wl, 1)
    assert not np.array_equal(a.k_pages, c.k_pages) and not np.array_equal(a.q, c.q)
    assert a.q.shape == (1, 8, 128) and a.q.dtype == np.uint16
    assert a.k_pages.shape == (4096 // 64, 2, 64, 128)


def test_values_are_standard_normal_in_bf16():
    wl = synth.TINY_4K
    li = synth.layer_inputs(wl, 0)
    v = synth.bf16_bits_to_f32(li.v_pages).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    k = synth.bf16_bits_to_f32(li.k_pages).astype(np.float64)
    assert abs(k.mean()) < 0.01 and abs(k.std() - 1) < 0.01  # rotation keeps N(0, I)


def test_paging_and_lengths():
    wl = synth.BATCHED_16
    pg = synth.paging(wl)
    assert pg.seq_lens.shape == (16,)
    assert np.all(pg.seq_lens % 64 == 0)
    assert pg.seq_lens.min() >= 8192 and pg.seq_lens.max() <= 65536
    assert len(set(pg.seq_lens.tolist())) > 8
    used = np.concatenate([pg.block_table[b, : pg.seq_lens[b] // 64] for b in range(16)])
    assert np.array_equal(np.sort(used), np.arange(pg.num_pages))   # a permutation
    assert np.array_equal(synth.seq_lens(wl), pg.seq_lens)


def test_planted_structure():
    wl = synth.scaled(synth.LLAMA_128K_PLANTED, name="planted-small", wid=903, context=16384,
                      n_clusters=16)
    pg = synth.paging(wl)
    L = int(pg.seq_lens[0])
    p0 = synth.cluster_starts(wl, 0, 0, L)
    assert np.all(np.diff(p0) >= wl.cluster_len) and p0.min() >= wl.n_sinks
    p1, p2 = synth.cluster_starts(wl, 1, 0, L), synth.cluster_starts(wl, 2, 0, L)
    assert set(np.abs(p1 - p0).tolist()) <= {0, 16} and set(np.abs(p2 - p1).tolist()) <= {0, 16}
    assert np.any(p1 != p0)
    li = synth.layer_inputs(wl, 2)
    q = synth.bf16_bits_to_f32(li.q[0]).astype(np.float64)
    G = wl.group
    for g in range(wl.num_kv_heads):
        k, _ = synth.kv_head(wl, 2, 0, g, L, li.q)
        kf = synth.bf16_bits_to_f32(k).astype(np.float64)
        for c, p in enumerate(p2):
            keep = np.ones(wl.cluster_len, bool)   # rows a later cluster overwrote are skipped
            for p_later in p2[c + 1:]:
                t = np.arange(p, p + wl.cluster_len)
                keep &= ~((t >= p_later) & (t < p_later + wl.cluster_len))
            qh = q[g * G + c % G] / np.linalg.norm(q[g * G + c % G])
            rows = kf[p: p + wl.cluster_len][keep]
            cos = rows @ qh / np.linalg.norm(rows, axis=1)
            np.testing.assert_allclose(cos, 0.6, atol=0.01)
        # sinks: 4x the RoPE-rotated raw key, so norm about 4 * sqrt(128)
        assert np.all(np.linalg.norm(kf[:4], axis=1) > 2.5 * np.sqrt(128))
