"""prism_decode_layer_noalloc (the library's static per-GPU workspace) against
prism_decode_layer with a caller-owned workspace, through the C ABI: two
decode steps in a row on the static workspace, the second on smaller shapes
(fewer sequences, a shorter context, a smaller kappa).  Index sets must be
identical and outputs within the attention tolerance (the same kernels run
on the same inputs)."""
import numpy as np
import pytest
import torch

import synth
import token_sparse_attention_gqa_amd as tsa
from tests.parity import Setup, check_attn

pytestmark = pytest.mark.gpu


def _step(st, layers, call):
    anchor = st.idx_buf()
    sets, outs = [], []
    for l in layers:
        sel, out = st.idx_buf(), st.out_buf()
        call(l, anchor, sel, out)
        torch.cuda.synchronize()
        sets.append(sel.cpu().numpy())
        outs.append(out.cpu().numpy())
    return sets, outs


@pytest.mark.parametrize("rho", [0, 4])
def test_noalloc_matches_workspace_entry_point(rho):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    big = synth.scaled(synth.LLAMA_128K_PLANTED, name="noalloc-big", wid=470, batch=2,
                       context=20480, kappa=512, n_clusters=16, num_layers=4, anchor_stride=4)
    small = synth.scaled(synth.TINY_4K, name="noalloc-small", wid=471, batch=1,
                         num_q_heads=16, num_kv_heads=4, context=3000, kappa=200, window=8,
                         num_layers=3, anchor_stride=3)
    for wl in (big, small):
        layers = list(range(wl.num_layers))
        st = Setup(wl, layers, pool_rho=rho)
        assert tsa.prism_workspace_size(st.kv[0], st.params) <= tsa.PRISM_STATIC_WORKSPACE_BYTES
        want_sets, want_outs = _step(st, layers, lambda l, a, s, o: tsa.prism_decode_layer(
            l, st.kv[l], st.q[l], st.params, a, s, o, st.ws))
        got_sets, got_outs = _step(st, layers, lambda l, a, s, o: tsa.prism_decode_layer_noalloc(
            l, st.kv[l], st.q[l], st.params, a, s, o))
        G = wl.group
        for l in layers:
            assert np.array_equal(got_sets[l], want_sets[l]), f"{wl.name} layer {l}: sets differ"
            assert (got_sets[l] >= 0).all()
            for b in range(wl.batch):
                for g in range(wl.num_kv_heads):
                    check_attn(got_outs[l][b, g * G:(g + 1) * G], want_outs[l][b, g * G:(g + 1) * G],
                               f"{wl.name} layer {l} b{b} g{g}")
