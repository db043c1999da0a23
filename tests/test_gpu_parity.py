"""HIP path against the CPU oracle, element by element, through the C ABI.

Small cases span several workgroup tiles and ragged tails; the full-size cases
run every workload at its real shape through prism_decode_layer (the launch
path the benchmark times) and check every (sequence, KV head) problem over a
whole anchor group."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
import token_sparse_attention_gqa_amd as tsa
from tests.conftest import record_summary
from tests.parity import Setup, check_attn, check_set, dev, unpack_int2_codes

pytestmark = pytest.mark.gpu
PAR_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tsa.lib()   # the HIP library must be built; no fallback exists
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _small(G, lengths, kappa, window=16, hkv=2, wid=100, planted=False, layers=2, stride=2,
           context=None):
    return synth.scaled(synth.TINY_4K, name=f"small-g{G}", wid=wid, batch=len(lengths),
                        num_q_heads=G * hkv, num_kv_heads=hkv, kappa=kappa, window=window,
                        context=context, lengths=None if context else tuple(lengths),
                        planted=planted, num_layers=layers, anchor_stride=stride)


def _anchor_gpu(st, l, scores=False):
    idx = st.idx_buf()
    sc = (torch.full((st.wl.batch, st.wl.num_kv_heads, st.kv[l].struct.max_seq_len), float("nan"),
                     device="cuda") if scores else None)
    tsa.prism_score_topk(st.kv[l], st.q[l], st.params, idx, sc, st.ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy() if scores else None)


# --------------------------------------------------------------------------- anchor
def test_anchor_scores_and_sets_tiny():
    st = Setup(synth.TINY_4K, [0])
    idx, sc = _anchor_gpu(st, 0, scores=True)
    for b in range(1):
        for g in range(2):
            want, s = st.oracle_anchor(0, b, g)
            np.testing.assert_allclose(sc[b, g, :4096], s, rtol=1e-5, atol=1e-3)
            assert check_set(idx[b, g], want, s, np.arange(4096), 256, f"b{b}g{g}") == "exact"


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("kappa", [1, 97, 130])
def test_anchor_ragged_groups(G, kappa):
    lengths = (1000, 4097, 130, 2113)
    st = Setup(_small(G, lengths, kappa, wid=110 + G), [0])
    idx, sc = _anchor_gpu(st, 0, scores=True)
    for b, L in enumerate(lengths):
        for g in range(2):
            want, s = st.oracle_anchor(0, b, g)
            np.testing.assert_allclose(sc[b, g, :L], s, rtol=1e-5, atol=1e-3)
            check_set(idx[b, g], want, s, np.arange(L), kappa, f"G{G} k{kappa} b{b} g{g}")


def _hand_cache(rows_by_head, lengths):
    """Identity-paged cache from explicit bf16 rows [Hkv][L][128] (same L per head)."""
    hkv = len(rows_by_head)
    L = max(lengths)
    npg = (L + 63) // 64
    B = len(lengths)
    kp = np.zeros((npg * B, hkv, 64, 128), np.uint16)
    for b in range(B):
        for h in range(hkv):
            r = np.zeros((npg * 64, 128), np.uint16)
            r[:L] = rows_by_head[h][:L]
            kp[b * npg:(b + 1) * npg, h] = r.reshape(npg, 64, 128)
    bt = np.arange(npg * B, dtype=np.int32).reshape(B, npg)
    return kp, bt


def test_exact_ties_go_to_lowest_position():
    """Equal scores in any precision (identical key rows): the lowest positions win."""
    rng = np.random.default_rng(7)
    L, kappa, G = 700, 50, 4
    base = synth.f32_to_bf16_bits(rng.standard_normal((L, 128)).astype(np.float32))
    tie = synth.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    rows0 = np.repeat(tie[None], L, 0)                    # head 0: every row equal
    rows1 = base.copy()                                   # head 1: 80 copies of one strong row
    q = synth.f32_to_bf16_bits(rng.standard_normal((1, 2 * G, 128)).astype(np.float32))
    qf = synth.bf16_bits_to_f32(q[0, G:2 * G]).astype(np.float64)
    strong = synth.f32_to_bf16_bits((3 * qf[0] / np.linalg.norm(qf[0]) * 11.3).astype(np.float32))
    dup_pos = np.sort(rng.choice(L, 80, replace=False))
    rows1[dup_pos] = strong
    kp, bt = _hand_cache([rows0, rows1], [L])
    kv = tsa.KVCache(dev(kp), dev(kp), dev(bt), dev(np.array([L], np.int32)), max_seq_len=L,
                     min_seq_len=L)
    p = tsa.params(2 * G, kappa)
    ws = torch.empty(tsa.prism_workspace_size(kv, p), dtype=torch.uint8, device="cuda")
    idx = torch.zeros((1, 2, kappa), dtype=torch.int32, device="cuda")
    tsa.prism_score_topk(kv, dev(q), p, idx, None, ws)
    got = idx.cpu().numpy()
    assert list(got[0, 0]) == list(range(kappa))
    assert list(got[0, 1]) == list(dup_pos[:kappa])


@pytest.mark.parametrize("L,kappa", [(3000, 100), (20000, 1000), (30000, 2000)])
def test_concentrated_scores_and_long_ties(L, kappa):
    """Head 0: every row equal (one score repeated L times).  Head 1: one key
    row scaled by 2^16, so every other score sits inside one 1/4096 slice of
    the score range.  Lists below and above 16384 entries, through the
    per-problem selection (prism_score_topk) and the fused anchor kernel
    (prism_decode_layer, which selects these contexts from keys in
    registers)."""
    rng = np.random.default_rng(8)
    G = 4
    base = rng.standard_normal((L, 128)).astype(np.float32)
    tie = synth.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    rows0 = np.repeat(tie[None], L, 0)
    base[L // 3] *= 65536.0
    rows1 = synth.f32_to_bf16_bits(base)
    q = synth.f32_to_bf16_bits(rng.standard_normal((1, 2 * G, 128)).astype(np.float32))
    kp, bt = _hand_cache([rows0, rows1], [L])
    kv = tsa.KVCache(dev(kp), dev(kp), dev(bt), dev(np.array([L], np.int32)), max_seq_len=L,
                     min_seq_len=L)
    p = tsa.params(2 * G, kappa)
    ws = torch.empty(tsa.prism_workspace_size(kv, p), dtype=torch.uint8, device="cuda")
    idx = torch.zeros((1, 2, kappa), dtype=torch.int32, device="cuda")
    tsa.prism_score_topk(kv, dev(q), p, idx, None, ws)
    got = idx.cpu().numpy()
    assert list(got[0, 0]) == list(range(kappa))
    qf = oracle.bf16_to_f64(q[0, G:2 * G])
    want, s = oracle.anchor_select(qf, kp, bt[0], 1, L, kappa, 64)
    check_set(got[0, 1], want, s, np.arange(L), kappa, f"outlier L{L}")
    anchor, sel = torch.zeros_like(idx), torch.zeros_like(idx)
    out = torch.zeros((1, 2 * G, 128), dtype=torch.float32, device="cuda")
    tsa.prism_decode_layer(0, kv, dev(q), p, anchor, sel, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), got), f"fused anchor kernel L{L}"


def test_wide_threshold_bin_with_ties():
    """A list longer than 16384 whose threshold bin (one coarse score bin)
    holds more candidates than LDS keeps: about 8000 of 40000 entries, each
    classify region within its own capacity.  Scores are exact (one query
    head, q = e_0 + e_1 / 256, keys with only those two dimensions), about 120
    of them equal at the kappa-th place: the selection ranks the stored
    candidates by their remaining key bits and gives the tie to the lowest
    positions, exactly as the oracle."""
    rng = np.random.default_rng(21)
    L = 40000
    k = np.zeros((L, 128), np.float32)
    u = rng.random(L)
    above, inbin = u < 0.05, (u >= 0.05) & (u < 0.25)
    below = ~(above | inbin)
    k[above, 0], k[above, 1] = 2.5, rng.standard_normal(int(above.sum()))
    k[inbin, 0], k[inbin, 1] = 1.0, rng.uniform(0.0, 24.0, int(inbin.sum()))  # scores in [1, 1.094)
    k[below, 0], k[below, 1] = 0.5, rng.standard_normal(int(below.sum()))
    k[np.sort(rng.choice(np.nonzero(inbin)[0], 100, replace=False)), 1] = 12.0
    rows = synth.f32_to_bf16_bits(k)
    q = np.zeros((1, 1, 128), np.float32)
    q[0, 0, 0], q[0, 0, 1] = 1.0, 1.0 / 256
    q = synth.f32_to_bf16_bits(q)
    kp, bt = _hand_cache([rows], [L])
    # kappa: every score above 1 + 12/256, then about half of those equal to it
    sc = oracle.relevance(oracle.bf16_to_f64(q[0]), oracle.bf16_to_f64(rows))
    thr = 1.0 + 12.0 / 256
    n_above, n_eq = int((sc > thr).sum()), int((sc == thr).sum())
    assert 4096 < int(((sc >= 1.0) & (sc < 1.125)).sum()) and 100 <= n_eq <= 256
    kappa = n_above + n_eq // 2
    kv = tsa.KVCache(dev(kp), dev(kp), dev(bt), dev(np.array([L], np.int32)), max_seq_len=L,
                     min_seq_len=L)
    p = tsa.params(1, kappa)
    ws = torch.empty(tsa.prism_workspace_size(kv, p), dtype=torch.uint8, device="cuda")
    idx = torch.zeros((1, 1, kappa), dtype=torch.int32, device="cuda")
    for rep in range(2):  # a fresh workspace takes the exact fallback once
        say(f"[wide-bin] kappa={kappa} n_eq={n_eq} rep={rep}")
        tsa.prism_score_topk(kv, dev(q), p, idx, None, ws)
        got = idx.cpu().numpy()[0, 0]
        want, _ = oracle.anchor_select(oracle.bf16_to_f64(q[0]), kp, bt[0], 0, L, kappa, 64)
        assert np.array_equal(np.sort(got), np.sort(want)), f"rep {rep}"


# --------------------------------------------------------------------------- refine
def test_refine_stage_isolated_tiny():
    st = Setup(synth.TINY_4K, [0, 1])
    A = np.stack([st.oracle_anchor(0, 0, g)[0] for g in range(2)])[None].astype(np.int32)
    P = 2
    idx, pool = st.idx_buf(), torch.full((1, 2, 4096), -5, dtype=torch.int32, device="cuda")
    plen = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    psc = torch.zeros((1, 2, 4096), dtype=torch.float32, device="cuda")
    tsa.prism_refine_topk(st.kv[1], st.q[1], st.params, dev(A), idx, pool, plen, psc, st.ws)
    idx, pool, plen, psc = (t.cpu().numpy() for t in (idx, pool, plen, psc))
    for g in range(P):
        want, wpool, s = st.oracle_refine(1, 0, g, A[0, g])
        n = int(plen[0, g])
        assert n == len(wpool) and np.array_equal(pool[0, g, :n], wpool)   # bit-exact pool
        np.testing.assert_allclose(psc[0, g, :n], s, rtol=1e-5, atol=1e-3)
        check_set(idx[0, g], want, s, wpool, 256, f"refine g{g}")


@pytest.mark.parametrize("window", [0, 1, 5, 33])
def test_refine_pools_and_sets_ragged(window):
    lengths = (1000, 4097, 300, 2113)
    wl = _small(4, lengths, 97, window=window, wid=130 + window)
    st = Setup(wl, [0, 1])
    A_gpu, _ = _anchor_gpu(st, 0)
    idx = st.idx_buf()
    pool = torch.full((4, 2, 4097), -5, dtype=torch.int32, device="cuda")
    plen = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    psc = torch.zeros((4, 2, 4097), dtype=torch.float32, device="cuda")
    tsa.prism_refine_topk(st.kv[1], st.q[1], st.params, dev(A_gpu), idx, pool, plen, psc, st.ws)
    idx, pool, plen, psc = (t.cpu().numpy() for t in (idx, pool, plen, psc))
    for b, L in enumerate(lengths):
        for g in range(2):
            want, wpool, s = st.oracle_refine(1, b, g, A_gpu[b, g])
            n = int(plen[b, g])
            assert n == len(wpool) and np.array_equal(pool[b, g, :n], wpool), (b, g)
            np.testing.assert_allclose(psc[b, g, :n], s, rtol=1e-5, atol=1e-3)
            check_set(idx[b, g], want, s, wpool, 97, f"w{window} b{b} g{g}")
            if window == 0:
                assert np.array_equal(idx[b, g], A_gpu[b, g])        # static reuse (Eq. 3)


def test_refine_full_window_is_exact_topk():
    lengths = (1000, 1500)
    wl = _small(4, lengths, 64, window=5000, wid=140)
    st = Setup(wl, [0, 1])
    A_gpu, _ = _anchor_gpu(st, 0)
    exact, _ = _anchor_gpu(st, 1)
    idx = st.idx_buf()
    tsa.prism_refine_topk(st.kv[1], st.q[1], st.params, dev(A_gpu), idx, workspace=st.ws)
    assert np.array_equal(idx.cpu().numpy(), exact)


# ------------------------------------------------------------------------ attention
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("kappa", [1, 100, 300])
def test_attention_on_identical_sets(G, kappa):
    lengths = (300, 1000, 4097)
    st = Setup(_small(G, lengths, kappa, wid=150 + G), [0])
    sets = np.zeros((3, 2, kappa), np.int32)
    for b in range(3):
        for g in range(2):
            sets[b, g] = st.oracle_anchor(0, b, g)[0]
    out = st.out_buf()
    tsa.prism_sparse_attn(st.kv[0], st.q[0], st.params, dev(sets), out, st.ws)
    out = out.cpu().numpy()
    for b in range(3):
        for g in range(2):
            check_attn(out[b, g * G:(g + 1) * G], st.oracle_attend(0, b, g, sets[b, g]),
                       f"G{G} k{kappa} b{b} g{g}")


def test_attention_dense_and_ignored_entries():
    """kappa = L is dense attention; negative entries of the set are skipped."""
    L = 300
    st = Setup(_small(4, (L, L), L, wid=160), [0])
    full = np.tile(np.arange(L, dtype=np.int32), (2, 2, 1))
    out = st.out_buf()
    tsa.prism_sparse_attn(st.kv[0], st.q[0], st.params, dev(full), out, st.ws)
    o = out.cpu().numpy()
    for b in range(2):
        for g in range(2):
            check_attn(o[b, 4 * g:4 * g + 4], st.oracle_attend(0, b, g, np.arange(L)), "dense")
    holes = full.copy()
    holes[:, :, ::3] = -1
    tsa.prism_sparse_attn(st.kv[0], st.q[0], st.params, dev(holes), out, st.ws)
    o = out.cpu().numpy()
    keep = np.array([i for i in range(L) if i % 3])
    for b in range(2):
        for g in range(2):
            check_attn(o[b, 4 * g:4 * g + 4], st.oracle_attend(0, b, g, keep), "holes")


# ---------------------------------------------------------------------- decode chain
def _par(fn, items):
    """fn over items on a thread pool (the oracle's numpy work releases the
    GIL), results in order; the first exception is raised."""
    items = list(items)
    if len(items) <= 2:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(min(len(items), PAR_WORKERS)) as ex:
        return list(ex.map(fn, items))


def _run_chain(st, layers, problems, label):
    """prism_decode_layer over `layers` in order; each layer checked against the
    oracle applied to the GPU's own anchor sets (chained) for the listed problems."""
    wl = st.wl
    anchor = st.idx_buf()
    layer_idx = st.idx_buf()
    out = st.out_buf()
    stats = {"exact": 0, "near-tie": 0}
    A_gpu = None
    for l in layers:
        say(f"[{label}] layer {l} ({'anchor' if wl.is_anchor(l) else 'refined'})")
        tsa.prism_decode_layer(l, st.kv[l], st.q[l], st.params, anchor, layer_idx, out, st.ws)
        torch.cuda.synchronize()
        sel = layer_idx.cpu().numpy()
        o = out.cpu().numpy()
        if wl.is_anchor(l):
            A_gpu = anchor.cpu().numpy()
            assert np.array_equal(A_gpu, sel)

        def check(bg, l=l, sel=sel, o=o, A_gpu=A_gpu):
            b, g = bg
            if wl.is_anchor(l):
                want, s = st.oracle_anchor(l, b, g)
                pool = np.arange(int(st.pg.seq_lens[b]))
            else:
                want, pool, s = st.oracle_refine(l, b, g, A_gpu[b, g])
            r = check_set(sel[b, g], want, s, pool, wl.kappa, f"{label} l{l} b{b} g{g}")
            G = wl.group
            check_attn(o[b, g * G:(g + 1) * G], st.oracle_attend(l, b, g, sel[b, g]),
                       f"{label} l{l} b{b} g{g}")
            return r

        for r in _par(check, problems):
            stats[r] += 1
    say(f"[{label}] sets: {stats}")
    return stats


def test_decode_chain_tiny():
    st = Setup(synth.TINY_4K, [0, 1])
    s = _run_chain(st, [0, 1], [(0, 0), (0, 1)], "tiny")
    assert s["exact"] == 4


def test_decode_chain_planted_small():
    wl = synth.scaled(synth.LLAMA_128K_PLANTED, name="planted-16k", wid=170, context=16384,
                      kappa=512, n_clusters=16, num_layers=8, anchor_stride=4)
    st = Setup(wl, range(8))
    _run_chain(st, range(8), [(0, g) for g in range(8)], "planted-16k")


def test_decode_chain_fused_128_token_splits():
    """16 (sequence, KV head) problems at kappa = 2048: 64-token splits of the
    fused refined kernel would need 512 workgroups, more than the device holds
    at once, so its refined layers take 128-token splits (256 workgroups);
    smaller grids take 64.  Both split sizes give the oracle's sets."""
    wl = synth.scaled(synth.TINY_4K, name="fused-128", wid=177, num_q_heads=32, num_kv_heads=8,
                      batch=2, context=None, lengths=(12000, 9000), kappa=2048, window=16,
                      num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3))
    _run_chain(st, range(3), [(b, g) for b in range(2) for g in (0, 3, 7)], "fused-128")


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_decode_chain_groups_mixed_pools(G):
    """Ragged batch whose refined pools fall on both sides of 16384 entries
    (the 20000-token sequence's pool exceeds it, the others stay below), for
    group sizes whose refined layers select inside the attention kernel
    (G <= 8) or in the selection kernel (G = 16)."""
    wl = synth.scaled(synth.TINY_4K, name=f"chain-g{G}", wid=180 + G, num_q_heads=2 * G,
                      num_kv_heads=2, batch=3, context=None, lengths=(4096, 1500, 20000),
                      kappa=300, window=100, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3))
    _run_chain(st, range(3), [(b, g) for b in range(3) for g in range(2)], f"chain-g{G}")


@pytest.mark.parametrize("fill", [0x00, 0xAB, 0xFF])
def test_decode_from_leftover_workspace(fill):
    """A workspace holding arbitrary bytes (as after other use): the counters in
    it are not trusted, results match the oracle, and a second decode step on
    the same workspace matches again."""
    wl = synth.scaled(synth.LLAMA_128K_PLANTED, name="leftover-ws", wid=190, context=40960,
                      kappa=512, n_clusters=16, num_layers=3, anchor_stride=2)
    st = Setup(wl, range(3))
    st.ws.fill_(fill)
    probs = [(0, g) for g in range(wl.num_kv_heads)]
    for rep in range(2):
        _run_chain(st, range(3), probs, f"leftover-ws {fill:#x} step {rep}")


@pytest.mark.parametrize("rho", [1, 4])
@pytest.mark.parametrize("fill", [0x00, 0xAB, 0xFF])
def test_rank_pool_from_leftover_workspace(fill, rho):
    """The rank-expanded pool from a workspace holding arbitrary bytes: both
    classifications (the anchor set's and the pool's) check their own counters,
    and two decode steps on the same workspace match the oracle.  At rho = 1
    the pool's classification is not made at all (it would equal the anchor
    set's), so its candidate counts are the workspace's bytes throughout."""
    wl = synth.scaled(synth.LLAMA_128K_PLANTED, name="leftover-rank", wid=191, context=40960,
                      kappa=512, n_clusters=16, num_layers=3, anchor_stride=2)
    st = Setup(wl, range(3), pool_rho=rho)
    st.ws.fill_(fill)
    probs = [(0, g) for g in range(wl.num_kv_heads)]
    for rep in range(2):
        _run_chain_rank(st, range(3), probs, f"leftover-rank rho={rho} {fill:#x} step {rep}")


@pytest.mark.parametrize("pool", ["window16", "rank4"])
@pytest.mark.parametrize("fill", [0xAB, 0xFF])
def test_multi_tile_from_leftover_workspace(fill, pool):
    """The multi-tile kernels from a workspace holding arbitrary bytes (48
    problems, G = 4, kappa = 1500): with the window pool the refined layers
    select from the pool's classification, with the rank pool the anchor layer
    from the list's; the selections check their own counters, and two decode
    steps on the same workspace match the oracle."""
    rho = 4 if pool == "rank4" else 0
    wl = synth.scaled(synth.TINY_4K, name=f"leftover-multi-{pool}", wid=540 + rho,
                      num_q_heads=32, num_kv_heads=8, batch=6, context=None,
                      lengths=(9024, 1500, 12000, 4096, 40000, 7001), kappa=1500,
                      window=16 if rho == 0 else 5, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=rho)
    st.ws.fill_(fill)
    probs = [(b, g) for b in range(wl.batch) for g in (0, 3, 7)]
    run = _run_chain_rank if rho else _run_chain
    for rep in range(2):
        run(st, range(3), probs, f"leftover-multi {pool} {fill:#x} step {rep}")


def test_decode_chain_per_problem_selection():
    """A grid the fused kernels do not use (32 problems x 9 splits of 128 > 256
    compute units): every layer selects once per problem (anchor lists and
    pools longer than 16384 entries are classified first), then attends.
    Ragged lengths; unstructured keys, so the pools cover most of the cache."""
    wl = synth.scaled(synth.BATCHED_16, name="per-problem", wid=193, batch=4, kappa=1100,
                      window=16, num_layers=3, anchor_stride=3, len_range=(17000, 40000))
    st = Setup(wl, range(3))
    probs = [(0, 0), (1, 3), (2, 5), (3, 7)]
    _run_chain(st, range(3), probs, "per-problem")


def _gpu_pool(st, l):
    """The pool the latest anchor selection left in the workspace, read through
    prism_refine_topk (rank-expanded pool: anchor_idx is not read), which also
    re-scores it with layer l's query and returns that selection."""
    wl = st.wl
    L_max = int(st.pg.seq_lens.max())
    sel = st.idx_buf()
    pool = torch.full((wl.batch, wl.num_kv_heads, L_max), -7, dtype=torch.int32, device="cuda")
    plen = torch.zeros((wl.batch, wl.num_kv_heads), dtype=torch.int32, device="cuda")
    tsa.prism_refine_topk(st.kv[l], st.q[l], st.params, None, sel, pool, plen, None, st.ws)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), plen.cpu().numpy(), sel.cpu().numpy()


def _run_chain_rank(st, layers, problems, label):
    """prism_decode_layer with the rank-expanded pool: each anchor layer's set
    and pool against the oracle (the pool by the same near-tie rule at its
    rho*kappa boundary), each refined layer against the oracle re-scoring the
    GPU's own pool, the attention on the GPU's sets."""
    wl = st.wl
    anchor, layer_idx, out = st.idx_buf(), st.idx_buf(), st.out_buf()
    stats = {"exact": 0, "near-tie": 0}
    pool_gpu = plen_gpu = None
    for l in layers:
        say(f"[{label}] layer {l} ({'anchor' if wl.is_anchor(l) else 'refined'})")
        tsa.prism_decode_layer(l, st.kv[l], st.q[l], st.params, anchor, layer_idx, out, st.ws)
        torch.cuda.synchronize()
        sel, o = layer_idx.cpu().numpy(), out.cpu().numpy()
        if wl.is_anchor(l):
            assert np.array_equal(anchor.cpu().numpy(), sel)
            pool_gpu, plen_gpu, _ = _gpu_pool(st, l)

        def check(bg, l=l, sel=sel, o=o, pool_gpu=pool_gpu, plen_gpu=plen_gpu):
            b, g = bg
            res = []
            L = int(st.pg.seq_lens[b])
            where = f"{label} l{l} b{b} g{g}"
            if wl.is_anchor(l):
                want, s = st.oracle_anchor(l, b, g)
                res.append(check_set(sel[b, g], want, s, np.arange(L), wl.kappa, where))
                m = min(st.pool_rho * wl.kappa, L)
                assert plen_gpu[b, g] == m, (where, plen_gpu[b, g], m)
                gp = pool_gpu[b, g, :m]
                wp = st.oracle_rank_pool(s, b)
                res.append(check_set(gp, wp, s, np.arange(L), m, where + " pool"))
                assert np.isin(sel[b, g], gp).all(), where + ": set outside its pool"
            else:
                gp = pool_gpu[b, g, :plen_gpu[b, g]]
                want, s = st.oracle_refine_in_pool(l, b, g, gp)
                res.append(check_set(sel[b, g], want, s, gp, wl.kappa, where))
            G = wl.group
            check_attn(o[b, g * G:(g + 1) * G], st.oracle_attend(l, b, g, sel[b, g]), where)
            return res

        for res in _par(check, problems):
            for r in res:
                stats[r] += 1
    say(f"[{label}] sets: {stats}")
    return stats


@pytest.mark.parametrize("rho", [1, 4, 16])
def test_decode_chain_rank_pool(rho):
    """Rank-expanded pool (Eq. 4) through prism_decode_layer on a ragged batch:
    lists selected in registers and after classification, and a sequence whose
    pool is its whole cache at rho = 16 (rho * kappa >= L)."""
    wl = synth.scaled(synth.TINY_4K, name=f"rank-pool-{rho}", wid=194, num_q_heads=32,
                      num_kv_heads=8, batch=3, context=None, lengths=(6016, 20032, 40000),
                      kappa=512, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=rho)
    probs = [(b, g) for b in range(wl.batch) for g in (0, 5)]
    _run_chain_rank(st, range(3), probs, f"rank-pool rho={rho}")


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_decode_chain_rank_pool_groups(G):
    """The rank-expanded pool for every group size: the fused anchor kernel's
    rank instantiation (G <= 8, pool written by its extra workgroups) and the
    per-problem rank kernel (G = 16), lengths on both sides of 16384."""
    wl = synth.scaled(synth.TINY_4K, name=f"rank-g{G}", wid=430 + G, num_q_heads=2 * G,
                      num_kv_heads=2, batch=3, context=None, lengths=(4096, 1500, 20000),
                      kappa=300, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=4)
    _run_chain_rank(st, range(3), [(b, g) for b in range(3) for g in range(2)], f"rank-g{G}")


def test_decode_chain_rank_pool_per_problem_selection():
    """Rank-expanded pool on a grid above the CU count (refined layers select
    once per problem, pools longer than 16384 entries classified first), G = 8."""
    wl = synth.scaled(synth.TINY_4K, name="rank-pool-pp", wid=195, num_q_heads=64,
                      num_kv_heads=8, batch=4, context=None, lengths=(20032, 36032, 24000, 30016),
                      kappa=1100, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=16)
    probs = [(0, 1), (1, 4), (2, 6), (3, 7)]
    _run_chain_rank(st, range(3), probs, "rank-pool per-problem")


# (G, kappa, pool): grids of 48 problems that the fused refined kernel's
# 128-token splits do not fit on 256 compute units, so refined layers take the
# multi-tile kernels: 256 ranks per workgroup at kappa = 700 (3 splits, the last
# ragged), 512 at kappa = 1500 (two tiles per wave, a ragged last split whose
# waves hold one or two tiles).  Windows of 3 and 5 keep every pool within
# 16384 entries (selected from registers); windows of 10 and 16 let the
# 40000-token sequence's pools exceed it (scored with coarse counts,
# classified, then selected from the classification).
MULTI_CASES = [(1, 1500, "rank4"), (2, 700, "window5"), (4, 1500, "window3"), (8, 1500, "rank4"),
               (8, 700, "window5"), (4, 1500, "window10"), (8, 700, "window16"),
               (1, 700, "window16")]


@pytest.mark.parametrize("G,kappa,pool", MULTI_CASES,
                         ids=[f"G{G}-k{k}-{pl}" for G, k, pl in MULTI_CASES])
def test_decode_chain_multi_tile_refined(G, kappa, pool):
    """Refined layers of grids above the device (48 problems) with pools of at
    most 16384 entries: every split's workgroup selects the pool's top-kappa
    itself and attends 256 or 512 of its ranks in 16-token tiles per wave.  A
    ragged batch with a sequence of 1500 tokens (at kappa = 1500 its pool is
    its whole cache and every token is selected) and one of 40000 (selected
    after classification), every problem checked on the anchor layer and both
    refined layers.  With the rank pool the anchor layer takes the multi-tile
    kernel too (two tiles per wave, and one more workgroup per problem that
    writes the pool)."""
    rho = 4 if pool == "rank4" else 0
    window = 5 if pool == "rank4" else int(pool[len("window"):])
    wl = synth.scaled(synth.TINY_4K, name=f"multi-{G}-{kappa}-{pool}", wid=520 + G + kappa % 7,
                      num_q_heads=8 * G, num_kv_heads=8, batch=6, context=None,
                      lengths=(9024, 1500, 12000, 4096, 40000, 7001), kappa=kappa,
                      window=window, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=rho)
    probs = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    if rho:
        _run_chain_rank(st, range(3), probs, f"multi G={G} kappa={kappa} {pool}")
    else:
        _run_chain(st, range(3), probs, f"multi G={G} kappa={kappa} {pool}")


def _run_pattern(st, pattern, problems, label, table4=False):
    """prism_decode_layer_role over a layer-role pattern: proposal layers
    against the oracle's exact TopK, refined layers against the oracle
    re-scoring the pool of the GPU's own nearest proposal layer, shared layers
    reusing the nearest proposal or refined layer's set bit for bit, and the
    attention of every layer on the GPU's set."""
    wl = st.wl
    set_idx, out = st.idx_buf(), st.out_buf()
    f_set = last = pool_gpu = plen_gpu = None
    stats = {"exact": 0, "near-tie": 0, "shared": 0}
    for l, c in enumerate(pattern):
        role = tsa.prism_pattern_role(pattern, l, table4=table4)
        kind = "FRS"[role]
        say(f"[{label}] layer {l} role {kind}")
        tsa.prism_decode_layer_role(role, st.kv[l], st.q[l], st.params, set_idx, out, st.ws)
        torch.cuda.synchronize()
        sel, o = set_idx.cpu().numpy(), out.cpu().numpy()
        if kind == "F":
            f_set = sel.copy()
            if st.pool_rho >= 1:
                pool_gpu, plen_gpu, _ = _gpu_pool(st, l)
        if kind == "S":
            assert np.array_equal(sel, last), f"{label} l{l}: shared layer changed the set"
            stats["shared"] += 1
        for b, g in problems:
            where = f"{label} l{l} b{b} g{g}"
            L = int(st.pg.seq_lens[b])
            if kind == "F":
                want, sc = st.oracle_anchor(l, b, g)
                stats[check_set(sel[b, g], want, sc, np.arange(L), wl.kappa, where)] += 1
            elif kind == "R":
                if st.pool_rho >= 1:
                    gp = pool_gpu[b, g, :plen_gpu[b, g]]
                    want, sc = st.oracle_refine_in_pool(l, b, g, gp)
                else:
                    want, gp, sc = st.oracle_refine(l, b, g, f_set[b, g])
                stats[check_set(sel[b, g], want, sc, gp, wl.kappa, where)] += 1
            G = wl.group
            check_attn(o[b, g * G:(g + 1) * G], st.oracle_attend(l, b, g, sel[b, g]), where)
        if kind != "S":
            last = sel.copy()
    say(f"[{label}] sets: {stats}")
    return stats


@pytest.mark.parametrize("rho", [0, 4])
def test_decode_layer_roles_hybrid_pattern(rho):
    """A proposal / refined / shared hybrid (Appendix E, Table 9's letters):
    refined layers after shared ones, shared layers after refined ones and a
    second proposal layer, with the window and the rank-expanded pool, on a
    ragged batch that spans the register and classified selection paths."""
    wl = synth.scaled(synth.TINY_4K, name=f"roles-{rho}", wid=196, num_q_heads=32,
                      num_kv_heads=8, batch=3, context=None, lengths=(6016, 20032, 40000),
                      kappa=512, num_layers=8, anchor_stride=8)
    st = Setup(wl, range(8), pool_rho=rho)
    probs = [(b, g) for b in range(wl.batch) for g in (1, 6)]
    s = _run_pattern(st, "FSRSRFSR", probs, f"roles rho={rho}")
    assert s["shared"] == 3


def test_decode_layer_roles_table4_pattern_per_problem_selection():
    """Layers 7-12 of Table 4's Qwen3-4B group-4 pattern (F proposal, S
    refined) on a grid above the CU count, G = 8: refined layers select once
    per problem."""
    wl = synth.scaled(synth.TINY_4K, name="roles-t4", wid=197, num_q_heads=64,
                      num_kv_heads=8, batch=4, context=None, lengths=(20032, 36032, 24000, 30016),
                      kappa=1100, num_layers=6, anchor_stride=6)
    st = Setup(wl, range(6), pool_rho=0)
    probs = [(0, 2), (1, 5), (2, 0), (3, 7)]
    s = _run_pattern(st, "FFSSSS", probs, "roles table-4", table4=True)
    assert s["shared"] == 0


# --------------------------------------------------------------------------- INT2 keys
def _plant_special_groups(kp, bt, L):
    """Key rows with edge cases, written into the cache of sequence 0, KV head 0:
    a constant group, -0 and +0 mixed, exact midpoints between levels, values
    near 1e30 and near 1e-30."""
    rows = {}
    vals = np.zeros((4, 128), np.float32)
    vals[0, :32] = 1.5                                    # constant group
    vals[0, 32:64] = np.where(np.arange(32) % 3 == 0, -0.0, 0.0)
    vals[0, 37] = 3.0                                     # -0 / +0 with one level above
    vals[1, :5] = [0.0, 3.0, 0.5, 1.5, 2.5]               # midpoints: ties to even
    vals[2, :32] = np.linspace(-1e30, 1e30, 32)
    vals[2, 32:64] = np.linspace(-3e-30, 5e-30, 32)
    vals[3] = np.random.default_rng(4).standard_normal(128)
    for i, pos in enumerate((5, 64, 65, L - 1)):
        bits = (vals[i].view(np.uint32) >> 16).astype(np.uint16)
        kp[bt[pos // 64], 0, pos % 64] = bits
        rows[pos] = bits
    return rows


def test_int2_quantize_bit_exact():
    """prism_quantize_keys against the oracle's quantizer, code for code and bit
    for bit in the scales, on a ragged batch with edge-case rows; rows of other
    positions stay untouched; num_new = 5 rewrites exactly the last 5
    positions of every sequence, num_new = 37 the last 37 (a kernel wave's 16
    positions then start unaligned and can span two pages)."""
    wl = synth.scaled(synth.TINY_4K, name="int2-quant", wid=198, num_q_heads=16,
                      num_kv_heads=4, batch=3, context=None, lengths=(6016, 777, 12000),
                      num_layers=1)
    pg = synth.paging(wl)
    li = synth.layer_inputs(wl, 0)
    kp = li.k_pages.copy()
    _plant_special_groups(kp, pg.block_table[0], int(pg.seq_lens[0]))
    bt, sl = dev(pg.block_table), dev(pg.seq_lens)
    kv = tsa.KVCache(dev(kp), dev(li.v_pages), bt, sl, max_seq_len=int(pg.seq_lens.max()),
                     min_seq_len=int(pg.seq_lens.min()))
    cs, ss = tsa.int2_shapes(kp.shape[0], wl.num_kv_heads)
    for num_new in (0, 5, 37):
        codes = torch.full(cs, 0xCD, dtype=torch.uint8, device="cuda")
        scales = torch.full(ss, 0x7BCD, dtype=torch.int16, device="cuda")
        say(f"[int2-quant] num_new={num_new}")
        tsa.prism_quantize_keys(kv, num_new, codes, scales)
        torch.cuda.synchronize()
        c = codes.cpu().numpy()
        sc = scales.cpu().numpy().view(np.uint16)
        touched = np.zeros(cs[:3], bool)
        for b in range(wl.batch):
            L = int(pg.seq_lens[b])
            pos = np.arange(L if num_new == 0 else min(num_new, L))
            if num_new:
                pos = L - 1 - pos[::-1]
            phys = pg.block_table[b][pos // 64]
            for g in range(wl.num_kv_heads):
                bits = kp[phys, g, pos % 64]
                wc, wa, wb = oracle.quantize_int2(bits)
                got_c = unpack_int2_codes(c[phys, g, pos % 64])
                assert np.array_equal(got_c, wc), f"codes b{b} g{g}"
                wa16 = (wa.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                wb16 = (wb.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                got_s = sc[phys, g, pos % 64]
                assert np.array_equal(got_s[..., 0], wa16), f"alpha b{b} g{g}"
                assert np.array_equal(got_s[..., 1], wb16), f"beta b{b} g{g}"
                touched[phys, g, pos % 64] = True
        assert np.all(c[~touched] == 0xCD) and np.all(sc[~touched] == 0x7BCD), "untouched rows"


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_int2_anchor_scores_and_sets(G):
    """INT2 relevance and anchor selection for every group size, ragged lengths
    on both sides of the register-selection limit: scores within fp32 rounding
    of the oracle's (dequantized keys in float64), sets by the index rule."""
    wl = _small(G, (3000, 17000, 700), kappa=130, wid=300 + G, layers=1, stride=1)
    st = Setup(wl, [0], int2=True)
    idx, sc = _anchor_gpu(st, 0, scores=True)
    stats = {"exact": 0, "near-tie": 0}
    for b in range(wl.batch):
        L = int(st.pg.seq_lens[b])
        for g in range(wl.num_kv_heads):
            want, s = st.oracle_anchor(0, b, g)
            np.testing.assert_allclose(sc[b, g, :L], s, rtol=1e-5, atol=1e-5 * np.abs(s).max())
            stats[check_set(idx[b, g], want, s, np.arange(L), wl.kappa, f"int2 G{G} b{b} g{g}")] += 1
    say(f"[int2 G={G}] sets: {stats}")


@pytest.mark.parametrize("rho", [0, 4])
def test_int2_decode_chain(rho):
    """INT2 scoring at anchor and refined layers through prism_decode_layer,
    window and rank-expanded pools, on a ragged batch (fused kernels)."""
    wl = synth.scaled(synth.TINY_4K, name=f"int2-chain-{rho}", wid=199, num_q_heads=32,
                      num_kv_heads=8, batch=3, context=None, lengths=(6016, 20032, 40000),
                      kappa=512, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), pool_rho=rho, int2=True)
    probs = [(b, g) for b in range(wl.batch) for g in (2, 7)]
    if rho:
        _run_chain_rank(st, range(3), probs, f"int2 rank rho={rho}")
    else:
        _run_chain(st, range(3), probs, "int2 window")


@pytest.mark.parametrize("G", [1, 16])
def test_int2_decode_chain_groups(G):
    """INT2 through the per-problem selection kernels (G = 16) and the
    smallest group, pools on both sides of 16384 entries."""
    wl = synth.scaled(synth.TINY_4K, name=f"int2-g{G}", wid=310 + G, num_q_heads=2 * G,
                      num_kv_heads=2, batch=3, context=None, lengths=(4096, 1500, 20000),
                      kappa=300, window=100, num_layers=3, anchor_stride=3)
    st = Setup(wl, range(3), int2=True)
    _run_chain(st, range(3), [(b, g) for b in range(3) for g in range(2)], f"int2-g{G}")


def _new_key_slots(st, nk):
    """(page, slot) of the last nk positions of every sequence."""
    pages, slots = [], []
    for b, L in enumerate(st.pg.seq_lens.tolist()):
        for pos in range(max(0, L - nk), L):
            pages.append(int(st.pg.block_table[b, pos // st.wl.page_size]))
            slots.append(pos % st.wl.page_size)
    return torch.tensor(pages, device="cuda"), torch.tensor(slots, device="cuda")


@pytest.mark.parametrize("mode,G", [("window", 4), ("rank", 4), ("roles", 4), ("standalone", 4),
                                    ("window", 1), ("window", 16), ("rank", 16),
                                    ("multi-window", 4), ("multi-rank", 4)])
@pytest.mark.parametrize("nk", [1, 5, 64])
def test_int2_new_keys_quantized_inside_the_call(mode, G, nk):
    """prism_kv_cache.new_keys: the codes and scales of every sequence's last
    nk positions hold garbage (0xFF codes, alpha and beta near 1.7e38), and
    the calls given new_keys = nk must write them exactly as
    prism_quantize_keys did before scoring them: every layer's sets, pool
    scores and outputs bit-identical to a step on correct codes, and afterwards
    every layer's codes and scales bit-identical to the standalone
    quantization.  Lengths 2050 (the new keys straddle two of the anchor
    kernel's 1024-token workgroups), 5000 and 4097; rho = 16 makes the first
    sequence's pool its whole cache, so its new keys are the pool's last
    entries and straddle a pool workgroup's 256 entries; the window pool may or may not
    hold them (the last pool workgroup writes those outside it); FRS puts a
    shared layer, which scores nothing, last.  G = 16 takes the per-problem
    selection and rank-pool kernels instead of the fused ones; the multi
    modes (16 KV heads, 48 problems, kappa = 700, the 5000-token sequence
    made 20000) the multi-tile kernels: refined layers classified first
    (window pools up to 20032 entries), or the rank pool's anchor kernel
    (selecting the 20000-token list from its classification) and refined
    kernel."""
    nl = 3
    multi = mode.startswith("multi")
    hkv = 16 if multi else 2
    wl = synth.scaled(synth.TINY_4K, name=f"new-keys-{mode}", wid=460, num_q_heads=hkv * G,
                      num_kv_heads=hkv, batch=3, context=None,
                      lengths=(2050, 20000 if multi else 5000, 4097),
                      kappa=700 if multi else 300, window=16, num_layers=nl, anchor_stride=nl)
    st = Setup(wl, range(nl), pool_rho=16 if mode.endswith("rank") else 0, int2=True)
    want_codes = [st.kv[l].tensors[4].clone() for l in range(nl)]
    want_scales = [st.kv[l].tensors[5].clone() for l in range(nl)]

    lens = st.pg.seq_lens.astype(np.int64)

    def step(kvs):
        anchor = st.idx_buf()
        res = []
        for l in range(nl):
            sel, out = st.idx_buf(), st.out_buf()
            sc = torch.full((wl.batch, wl.num_kv_heads, int(lens.max())), float("nan"),
                            device="cuda")
            valid = np.repeat(lens[:, None], wl.num_kv_heads, 1)  # scores rows' valid prefix
            if mode == "roles":
                tsa.prism_decode_layer_role("FRS"[l], kvs[l], st.q[l], st.params, anchor, out,
                                            st.ws)
                sel.copy_(anchor)
            elif mode == "standalone":
                if l == 0:
                    tsa.prism_score_topk(kvs[l], st.q[l], st.params, anchor, sc, st.ws)
                    sel.copy_(anchor)
                else:
                    plen = torch.zeros((wl.batch, wl.num_kv_heads), dtype=torch.int32,
                                       device="cuda")
                    tsa.prism_refine_topk(kvs[l], st.q[l], st.params, anchor, sel,
                                          pool_len_out=plen, pool_scores_out=sc, workspace=st.ws)
                    valid = plen.cpu().numpy()
            else:
                tsa.prism_decode_layer(l, kvs[l], st.q[l], st.params, anchor, sel, out, st.ws)
            torch.cuda.synchronize()
            scores = sc.cpu().numpy().view(np.uint32)
            scores = np.concatenate([scores[b, g, :valid[b, g]] for b in range(wl.batch)
                                     for g in range(wl.num_kv_heads)])
            res.append((sel.cpu().numpy(), out.cpu().numpy().view(np.uint32), scores))
        return res

    want = step([st.kv[l] for l in range(nl)])
    pages, slots = _new_key_slots(st, nk)
    for l in range(nl):
        st.kv[l].tensors[4][pages, :, slots] = 0xFF
        st.kv[l].tensors[5][pages, :, slots] = 0x7F00
        assert not torch.equal(st.kv[l].tensors[4], want_codes[l])
    say(f"[new-keys {mode} G={G} nk={nk}] fused step")
    got = step([st.kv[l].with_new_keys(nk) for l in range(nl)])
    for l in range(nl):
        for name, g_a, w_a in zip(("set", "output", "scores"), got[l], want[l]):
            assert np.array_equal(g_a, w_a), f"layer {l}: {name} differs"
        assert torch.equal(st.kv[l].tensors[4], want_codes[l]), f"layer {l}: codes"
        assert torch.equal(st.kv[l].tensors[5], want_scales[l]), f"layer {l}: scales"


# --------------------------------------------------------------------------- dense decode
def _dense_check(st, l, problems, label):
    out = st.out_buf()
    say(f"[{label}] dense layer {l}")
    tsa.prism_dense_attn(st.kv[l], st.q[l], st.params, out, st.ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    G, li = st.wl.group, st.host[l]
    for b, g in problems:
        want = oracle.dense_attend(st.q_group(l, b, g), li.k_pages, li.v_pages,
                                   st.pg.block_table[b], g, int(st.pg.seq_lens[b]),
                                   st.wl.page_size, oracle.default_scale(st.wl.head_dim))
        check_attn(o[b, g * G:(g + 1) * G], want, f"{label} l{l} b{b} g{g}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_dense_decode(G):
    """Dense decode against the oracle over ragged lengths (a sequence shorter
    than one chunk, one with a ragged last chunk, one of many chunks)."""
    wl = _small(G, (6016, 777, 40000), kappa=64, wid=400 + G, layers=1, stride=1)
    st = Setup(wl, [0])
    _dense_check(st, 0, [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)],
                 f"dense G={G}")


def test_dense_decode_full_size_planted_128k():
    """Dense decode at 128K (128 chunks of 1024 tokens), every problem."""
    wl = synth.LLAMA_128K_PLANTED
    st = Setup(wl, [0])
    _dense_check(st, 0, [(0, g) for g in range(wl.num_kv_heads)], "dense 128k")


def test_dense_call_keeps_the_sparse_pool():
    """A dense call between an anchor layer and its refined layer leaves the
    pool in the workspace: the refined layer's set and output are the same as
    without it."""
    wl = synth.scaled(synth.TINY_4K, name="dense-between", wid=410, num_q_heads=32,
                      num_kv_heads=8, batch=2, context=None, lengths=(6016, 20032), kappa=256,
                      num_layers=2, anchor_stride=2)
    st = Setup(wl, [0, 1])
    res = []
    for dense_between in (False, True):
        anchor, sel, out = st.idx_buf(), st.idx_buf(), st.out_buf()
        tsa.prism_decode_layer(0, st.kv[0], st.q[0], st.params, anchor, None, out, st.ws)
        if dense_between:
            tsa.prism_dense_attn(st.kv[0], st.q[0], st.params, st.out_buf(), st.ws)
        tsa.prism_decode_layer(1, st.kv[1], st.q[1], st.params, anchor, sel, out, st.ws)
        torch.cuda.synchronize()
        res.append((sel.cpu().numpy(), out.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


# --------------------------------------------------------------------------- maximum sizes
def _max_wl():
    return synth.scaled(synth.TINY_4K, name="max-size", wid=420, num_q_heads=8, num_kv_heads=2,
                        batch=1, context=262144, lengths=None, kappa=8192, window=2,
                        num_layers=2, anchor_stride=2)


@pytest.mark.parametrize("mode", ["window", "rank", "int2", "dense"])
def test_maximum_sizes(mode):
    """The largest supported shapes: a 262144-token context (the anchor layer
    selects in its own kernel), kappa = 8192, a window pool of about 40K
    entries (the refined layer's long-pool selection), a rank-expanded pool of
    rho * kappa = 32768 entries, INT2 keys over the whole context, and dense
    decode in 128 chunks of 2048 tokens."""
    wl = _max_wl()
    rho = 4 if mode == "rank" else 0
    st = Setup(wl, range(2), pool_rho=rho, int2=(mode == "int2"))
    probs = [(0, 0), (0, 1)]
    if mode == "dense":
        _dense_check(st, 0, probs, "max-size dense")
    elif mode == "rank":
        _run_chain_rank(st, range(2), probs, "max-size rank")
    else:
        _run_chain(st, range(2), probs, f"max-size {mode}")


def test_determinism():
    st = Setup(synth.TINY_4K, [0, 1])
    res = []
    for _ in range(2):
        anchor, li, out = st.idx_buf(), st.idx_buf(), st.out_buf()
        for l in (0, 1):
            tsa.prism_decode_layer(l, st.kv[l], st.q[l], st.params, anchor, li, out, st.ws)
        torch.cuda.synchronize()
        res.append((li.cpu().numpy(), out.cpu().numpy().view(np.uint32)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


# ---------------------------------------------------------------------- graph replay
@pytest.mark.parametrize("mode", ["window", "rank", "int2", "int2-new-keys", "roles", "dense",
                                  "multi-window", "multi-rank-int2"])
def test_graph_replay_matches_eager(mode):
    """The decode step captured once as a HIP graph (the launch the benchmark
    times) and replayed three times, with eager work and synchronisations
    between the replays: after an eager step, after the workspace was
    overwritten with 0xAB bytes, and after a standalone call into another
    output.  Outputs and sets are cleared before every replay, and each
    replay's must equal the eager step's bit for bit.  The INT2 cases quantize
    the newest key in a launch of its own or inside the layer's calls
    (new_keys = 1)."""
    nl, pattern = 4, "FRSR"
    # the multi modes: 48 problems at kappa = 1500, beyond the fused kernels'
    # grid (window pools classified per refined layer; the rank pool's
    # multi-tile anchor and refined kernels, with INT2 keys and new_keys = 1)
    multi = mode.startswith("multi")
    wl = synth.scaled(synth.LLAMA_128K_PLANTED, name=f"graph-{mode}", wid=450, context=20480,
                      batch=6 if multi else 1, kappa=1500 if multi else 512, n_clusters=16,
                      num_layers=nl, anchor_stride=2)
    st = Setup(wl, range(nl), pool_rho=4 if mode in ("rank", "multi-rank-int2") else 0,
               int2=mode.startswith("int2") or mode.endswith("int2"))
    if mode in ("int2-new-keys", "multi-rank-int2"):   # each layer's call quantizes its newest key
        for l in range(nl):
            st.kv[l] = st.kv[l].with_new_keys(1)
    anchor = st.idx_buf()
    sels = [st.idx_buf() for _ in range(nl)]
    outs = [st.out_buf() for _ in range(nl)]

    def step():
        for l in range(nl):
            kv, q = st.kv[l], st.q[l]
            if mode == "dense":
                tsa.prism_dense_attn(kv, q, st.params, outs[l], st.ws)
            elif mode == "roles":
                tsa.prism_decode_layer_role(pattern[l], kv, q, st.params, anchor, outs[l], st.ws)
            else:
                if mode == "int2":   # the newest position's key, as a decode step appends it
                    tsa.prism_quantize_keys(kv, 1, kv.tensors[4], kv.tensors[5])
                tsa.prism_decode_layer(l, kv, q, st.params, anchor, sels[l], outs[l], st.ws)

    def clear():
        for t in sels + [anchor]:
            t.fill_(-7)
        for t in outs:
            t.fill_(float("nan"))

    def snapshot():
        torch.cuda.synchronize()
        return ([t.cpu().numpy().copy() for t in sels + [anchor]],
                [t.cpu().numpy().view(np.uint32).copy() for t in outs])

    clear()
    step()
    want_sets, want_outs = snapshot()
    assert all(np.all(np.isfinite(o.view(np.float32))) for o in want_outs)
    if mode not in ("dense", "roles"):
        assert all((s >= 0).all() for s in want_sets)

    gr = torch.cuda.CUDAGraph()
    clear()
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        step()
    torch.cuda.synchronize()

    spare = st.out_buf()
    between = [
        lambda: step(),
        lambda: st.ws.fill_(0xAB),
        lambda: tsa.prism_decode_layer(0, st.kv[0], st.q[0], st.params, st.idx_buf(), None,
                                       spare, st.ws) if mode != "dense"
        else tsa.prism_dense_attn(st.kv[0], st.q[0], st.params, spare, st.ws),
    ]
    for r, eager_work in enumerate(between):
        eager_work()
        torch.cuda.synchronize()
        clear()
        say(f"[graph-{mode}] replay {r}")
        gr.replay()
        got_sets, got_outs = snapshot()
        for l in range(nl):
            assert np.array_equal(got_outs[l], want_outs[l]), f"replay {r}: layer {l} output"
        for i, (g_s, w_s) in enumerate(zip(got_sets, want_sets)):
            assert np.array_equal(g_s, w_s), f"replay {r}: index buffer {i}"
    del gr


# ---------------------------------------------------------------------- full sizes
# Every workload at its real shape, in the launch configuration the benchmark
# times (prism_decode_layer), over a whole anchor group (the anchor layer and
# every refined layer that re-selects from its set), every (sequence, KV head)
# problem against the oracle.  Variants: the window pool, the rank-expanded
# pool (rho = 4) and INT2 proposal keys with either pool.  A workload's host
# inputs are generated once (layer by layer, in parallel) and shared by its
# variants.
FULL_CASES = [
    (synth.LLAMA_32K, "window"), (synth.LLAMA_32K, "rank4"), (synth.LLAMA_32K, "int2-rank4"),
    (synth.LLAMA_128K_PLANTED, "window"), (synth.LLAMA_128K_PLANTED, "rank4"),
    (synth.LLAMA_128K_PLANTED, "int2-window"),
    (synth.BATCHED_16, "window"), (synth.BATCHED_16, "rank4"), (synth.BATCHED_16, "int2-rank4"),
    (synth.LONG_4x128K, "window"), (synth.LONG_4x128K, "rank4"),
    (synth.LONG_4x128K, "int2-rank4"),
]
_HOST_CACHE = {}


def _group_layers(wl):
    return list(range(min(wl.anchor_stride, wl.num_layers)))


def _host_layers(wl, layers):
    """Host inputs of `layers`, generated in parallel; only the latest
    workload's are kept."""
    if wl.name not in _HOST_CACHE:
        _HOST_CACHE.clear()
        with ThreadPoolExecutor(min(len(layers), PAR_WORKERS)) as ex:
            got = list(ex.map(lambda l: synth.layer_inputs(wl, l, 1), layers))
        _HOST_CACHE[wl.name] = dict(zip(layers, got))
    return _HOST_CACHE[wl.name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,variant", FULL_CASES, ids=[f"{w.name}-{v}" for w, v in FULL_CASES])
def test_full_size_every_problem(wl, variant):
    layers = _group_layers(wl)
    say(f"[full] {wl.name} {variant}: layers {layers[0]}-{layers[-1]}, "
        f"{wl.batch * wl.num_kv_heads} problems")
    host = _host_layers(wl, layers)
    rho = 4 if variant.endswith("rank4") else 0
    st = Setup(wl, layers, pool_rho=rho, int2=variant.startswith("int2"), host=host)
    probs = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    label = f"{wl.name} {variant}"
    stats = (_run_chain_rank if rho else _run_chain)(st, layers, probs, label)
    record_summary(f"full size {label}: layers {layers[0]}-{layers[-1]} x {len(probs)} problems, "
                   f"sets exact {stats['exact']}, near-tie {stats['near-tie']}")
    del st
