"""Helpers of the GPU parity tests: upload seeded inputs, call the HIP library
through its C ABI binding, and compare with the CPU oracle.

Every buffer a test hands to the library through Setup (index sets, outputs,
the workspace) sits between guard regions that check_guards() verifies after
each GPU test.

Comparison rules:
  * index sets: valid (kappa ascending distinct positions inside the pool) and
    identical to the oracle's whenever the oracle's kappa-th and (kappa+1)-th
    scores differ by more than 1e-3 relative; otherwise the overlap is at
    least 0.999.  In every case each element in which the sets differ must sit
    within 1e-4 (relative) of the oracle's threshold score: a difference is
    only allowed where fp32 accumulation can reorder a near-tie.
  * attention outputs: max-abs error <= 2e-3 and relative L2 error <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import token_sparse_attention_gqa_amd as tsa

GAP_RULE = 1e-3
OVERLAP_MIN = 0.999
ATTN_MAX_ABS = 2e-3
ATTN_REL_L2 = 1e-3
NEAR_TIE = 1e-4


# Output and workspace buffers handed to the library carry guard regions of a
# known byte pattern before and after them; check_guards() (run after every
# GPU test) asserts that no call wrote into them.
GUARD_BYTES = 4096
GUARD_BYTE = 0xA5
_GUARDED = []


def guarded_empty(shape, dtype, label=""):
    """An uninitialised device tensor inside a larger allocation whose
    GUARD_BYTES before and after it hold GUARD_BYTE."""
    itemsize = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape))
    base = torch.empty(n * itemsize + 2 * GUARD_BYTES, dtype=torch.uint8, device="cuda")
    base.fill_(GUARD_BYTE)
    body = base[GUARD_BYTES:GUARD_BYTES + n * itemsize].view(dtype).view(*shape)
    _GUARDED.append((base, label or f"{tuple(shape)} {dtype}"))
    return body


def check_guards():
    """Asserts that every guard region allocated since the last check still
    holds its pattern, then forgets them."""
    torch.cuda.synchronize()
    bad = []
    for base, label in _GUARDED:
        head = base[:GUARD_BYTES]
        tail = base[base.numel() - GUARD_BYTES:]
        if not (bool((head == GUARD_BYTE).all()) and bool((tail == GUARD_BYTE).all())):
            bad.append(label)
    _GUARDED.clear()
    assert not bad, f"a library call wrote outside its buffer: {bad}"


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


class Setup:
    """Seeded inputs of some layers of a workload, resident on the device."""

    def __init__(self, wl: synth.Workload, layers, pool_rho=0, int2=False, host=None):
        """int2: quantize every layer's keys on the GPU (prism_quantize_keys)
        and score from the INT2 codes; the oracle then scores its own
        quantization of the same keys.  host: already generated layer inputs
        ({layer: synth.layer_inputs(wl, layer)}) to use instead of generating."""
        self.wl = wl
        self.int2 = int2
        self.pg = synth.paging(wl)
        self.bt = dev(self.pg.block_table)
        self.sl = dev(self.pg.seq_lens)
        self.host = {}
        self.q, self.kv = {}, {}
        for l in layers:
            li = host[l] if host is not None else synth.layer_inputs(wl, l)
            self.host[l] = li
            self.q[l] = dev(li.q)
            self.kv[l] = tsa.KVCache(dev(li.k_pages), dev(li.v_pages), self.bt, self.sl,
                                     max_seq_len=int(self.pg.seq_lens.max()),
                                     min_seq_len=int(self.pg.seq_lens.min()))
            if int2:
                cs, ss = tsa.int2_shapes(li.k_pages.shape[0], wl.num_kv_heads, wl.page_size)
                codes = torch.zeros(cs, dtype=torch.uint8, device="cuda")
                scales = torch.zeros(ss, dtype=torch.int16, device="cuda")
                tsa.prism_quantize_keys(self.kv[l], 0, codes, scales)
                self.kv[l] = self.kv[l].with_int2(codes, scales)
        self.pool_rho = pool_rho
        self.params = tsa.params(wl.num_q_heads, wl.kappa, wl.anchor_stride, wl.window,
                                 pool_rho=pool_rho)
        first = next(iter(self.kv.values()))
        self.ws = guarded_empty((tsa.prism_workspace_size(first, self.params),), torch.uint8,
                                "workspace")

    @property
    def P(self):
        return self.wl.batch * self.wl.num_kv_heads

    def idx_buf(self):
        t = guarded_empty((self.wl.batch, self.wl.num_kv_heads, self.wl.kappa), torch.int32,
                          "index set")
        return t.fill_(-7)

    def out_buf(self):
        t = guarded_empty((self.wl.batch, self.wl.num_q_heads, self.wl.head_dim), torch.float32,
                          "attention output")
        return t.fill_(float("nan"))

    # --- oracle views -------------------------------------------------------
    def q_group(self, l, b, g):
        G = self.wl.group
        return oracle.bf16_to_f64(self.host[l].q[b, g * G:(g + 1) * G])

    def oracle_anchor(self, l, b, g):
        li = self.host[l]
        return oracle.anchor_select(self.q_group(l, b, g), li.k_pages, self.pg.block_table[b], g,
                                    int(self.pg.seq_lens[b]), self.wl.kappa, self.wl.page_size,
                                    int2=self.int2)

    def oracle_refine(self, l, b, g, anchor):
        li = self.host[l]
        return oracle.refined_select(self.q_group(l, b, g), li.k_pages, self.pg.block_table[b], g,
                                     int(self.pg.seq_lens[b]), self.wl.kappa, self.wl.page_size,
                                     np.asarray(anchor, np.int64), self.wl.window, int2=self.int2)

    def oracle_rank_pool(self, anchor_scores, b):
        """Eq. 4 on the anchor layer's oracle scores over the whole cache."""
        L = int(self.pg.seq_lens[b])
        return oracle.rank_pool(anchor_scores, np.arange(L), self.pool_rho, self.wl.kappa)

    def oracle_refine_in_pool(self, l, b, g, pool):
        li = self.host[l]
        return oracle.refine_in_pool(self.q_group(l, b, g), li.k_pages, self.pg.block_table[b], g,
                                     np.asarray(pool, np.int64), self.wl.kappa,
                                     self.wl.page_size, int2=self.int2)

    def oracle_attend(self, l, b, g, sel):
        li = self.host[l]
        return oracle.attend(self.q_group(l, b, g), li.k_pages, li.v_pages, self.pg.block_table[b],
                             g, np.asarray(sel, np.int64), self.wl.page_size,
                             oracle.default_scale(self.wl.head_dim))


def unpack_int2_codes(codes) -> np.ndarray:
    """uint8 [..., 32] rows of INT2 codes -> uint8 [..., 128] codes per
    dimension, by the layout include/prism.h documents (dimension d = 32 s +
    8 u + j: 32-bit word 2u + s/2, bit 2 (4 (s % 2) + j / 2) + 16 (j % 2))."""
    w = np.ascontiguousarray(codes).view("<u4")
    d = np.arange(128)
    s, u, j = d // 32, (d % 32) // 8, d % 8
    word = 2 * u + s // 2
    bit = 2 * (4 * (s % 2) + j // 2) + 16 * (j % 2)
    return ((w[..., word] >> bit.astype(np.uint32)) & 3).astype(np.uint8)


def check_set(gpu_sel, want, scores, pool, kappa, where=""):
    """Returns 'exact' or 'near-tie' (raises AssertionError otherwise)."""
    gpu_sel = np.asarray(gpu_sel, dtype=np.int64)
    want = np.asarray(want, dtype=np.int64)
    pool = np.asarray(pool, dtype=np.int64)
    assert gpu_sel.shape == (kappa,), f"{where}: shape {gpu_sel.shape}"
    assert np.all(np.diff(gpu_sel) > 0), f"{where}: not ascending/distinct"
    assert np.isin(gpu_sel, pool).all(), f"{where}: positions outside the pool"
    if np.array_equal(gpu_sel, want):
        return "exact"
    assert len(pool) > kappa, f"{where}: pool of size kappa must be selected whole"
    s = np.asarray(scores, dtype=np.float64)
    srt = np.sort(s)[::-1]
    sk, sk1 = srt[kappa - 1], srt[kappa]
    gap = (sk - sk1) / abs(sk) if sk != 0 else np.inf
    missing = np.setdiff1d(want, gpu_sel)
    extra = np.setdiff1d(gpu_sel, want)
    pos_score = dict(zip(pool.tolist(), s.tolist()))
    assert gap <= GAP_RULE, (f"{where}: sets differ ({len(missing)} missing) although the "
                             f"kappa-th gap is {gap:.3g} > {GAP_RULE}")
    overlap = 1.0 - len(missing) / kappa
    assert overlap >= OVERLAP_MIN, f"{where}: overlap {overlap:.5f} < {OVERLAP_MIN}"
    for e in np.concatenate([missing, extra]):
        assert abs(pos_score[int(e)] - sk) <= NEAR_TIE * max(abs(sk), 1e-30), \
            f"{where}: differing position {e} is not a near-tie ({pos_score[int(e)]} vs {sk})"
    return "near-tie"


def check_attn(gpu_out, want, where=""):
    gpu_out = np.asarray(gpu_out, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert np.all(np.isfinite(gpu_out)), f"{where}: non-finite output"
    err = np.abs(gpu_out - want).max()
    rel = np.linalg.norm(gpu_out - want) / max(np.linalg.norm(want), 1e-30)
    assert err <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, \
        f"{where}: max-abs {err:.3g} (<= {ATTN_MAX_ABS}), rel-L2 {rel:.3g} (<= {ATTN_REL_L2})"
    return err, rel
