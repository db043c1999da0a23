"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid calls on the host before touching any
device (fake, never dereferenced addresses are used)."""
import ctypes

import pytest

import token_sparse_attention_gqa_amd as tsa
from token_sparse_attention_gqa_amd import _lib as L

FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def _kv(**over):
    d = dict(k_pages=FAKE, v_pages=FAKE, block_table=FAKE, seq_lens=FAKE, batch=2,
             num_kv_heads=8, head_dim=128, page_size=64, num_pages=1024, max_pages_per_seq=512,
             max_seq_len=32768, min_seq_len=4096, k_codes=None, k_scales=None, new_keys=0)
    d.update(over)
    return L.KVCacheStruct(*[d[n] for n, _ in L.KVCacheStruct._fields_])


def _params(**over):
    d = dict(num_q_heads=32, kappa=2048, anchor_stride=8, window=32, softmax_scale=0.0,
             pool_rho=0)
    d.update(over)
    return L.ParamsStruct(*[d[n] for n, _ in L.ParamsStruct._fields_])


def _call(fn, kv, p, ws=FAKE, nbytes=1 << 40, **extra):
    lib = tsa.lib()
    kvp = ctypes.byref(kv) if kv is not None else None
    pp = ctypes.byref(p) if p is not None else None
    if fn == "score":
        return lib.prism_score_topk(kvp, FAKE, pp, FAKE, None, ws, nbytes, None)
    if fn == "refine":
        return lib.prism_refine_topk(kvp, FAKE, pp, FAKE, FAKE, None, None, None, ws, nbytes, None)
    if fn == "attn":
        return lib.prism_sparse_attn(kvp, FAKE, pp, FAKE, FAKE, ws, nbytes, None)
    if fn == "layer":
        return lib.prism_decode_layer(extra.get("layer", 0), kvp, FAKE, pp, FAKE, None, FAKE, ws,
                                      nbytes, None)
    if fn == "dense":
        return lib.prism_dense_attn(kvp, FAKE, pp, FAKE, ws, nbytes, None)
    if fn == "role":
        return lib.prism_decode_layer_role(extra.get("role", 0), kvp, FAKE, pp, FAKE, FAKE, ws,
                                           nbytes, None)
    raise ValueError(fn)


def test_library_exports_every_declared_function():
    declared = tsa.declared_functions()
    assert set(declared) == {"prism_workspace_size", "prism_score_topk", "prism_refine_topk",
                             "prism_sparse_attn", "prism_decode_layer", "prism_status_string",
                             "prism_last_error", "prism_abi_version", "prism_profile_events",
                             "prism_profile_launches", "prism_pattern_role",
                             "prism_decode_layer_role", "prism_quantize_keys",
                             "prism_dense_attn", "prism_decode_layer_noalloc"}
    lib = tsa.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    """The library, the header and the binding's structs agree on the ABI version."""
    import re
    with open(L.HEADER) as f:
        header = int(re.search(r"#define PRISM_ABI_VERSION (\d+)", f.read()).group(1))
    assert tsa.prism_abi_version() == header == L.ABI_VERSION == 7
    for s in (0, -1, -2, -3, -4):
        assert tsa.prism_status_string(s) and tsa.prism_status_string(s) != "unknown status"
    assert tsa.prism_status_string(-99) == "unknown status"


def test_workspace_size():
    lib = tsa.lib()
    n = lib.prism_workspace_size(ctypes.byref(_kv()), ctypes.byref(_params()))
    assert n > 2 * 16 * 32768 * 4            # scores + pool lists of 16 problems at least
    assert n % 256 == 0
    assert lib.prism_workspace_size(ctypes.byref(_kv()), ctypes.byref(_params(kappa=0))) == 0
    bigger = lib.prism_workspace_size(ctypes.byref(_kv(max_seq_len=65536, max_pages_per_seq=1024)),
                                      ctypes.byref(_params()))
    assert bigger > n


CASES = [
    ("null kv", dict(kv=None), L.PRISM_ERR_INVALID_ARG),
    ("null k_pages", dict(kv=_kv(k_pages=None)), L.PRISM_ERR_INVALID_ARG),
    ("null seq_lens", dict(kv=_kv(seq_lens=None)), L.PRISM_ERR_INVALID_ARG),
    ("batch 0", dict(kv=_kv(batch=0)), L.PRISM_ERR_INVALID_ARG),
    ("hq not multiple of hkv", dict(p=_params(num_q_heads=30)), L.PRISM_ERR_INVALID_ARG),
    ("group 3", dict(kv=_kv(num_kv_heads=2), p=_params(num_q_heads=6)), L.PRISM_ERR_UNSUPPORTED),
    ("group 32", dict(kv=_kv(num_kv_heads=1)), L.PRISM_ERR_UNSUPPORTED),
    ("head_dim 64", dict(kv=_kv(head_dim=64)), L.PRISM_ERR_UNSUPPORTED),
    ("page 32", dict(kv=_kv(page_size=32)), L.PRISM_ERR_UNSUPPORTED),
    ("no pages", dict(kv=_kv(num_pages=0)), L.PRISM_ERR_INVALID_ARG),
    ("min > max", dict(kv=_kv(min_seq_len=40000)), L.PRISM_ERR_INVALID_ARG),
    ("max beyond pages", dict(kv=_kv(max_pages_per_seq=100)), L.PRISM_ERR_INVALID_ARG),
    ("max_seq_len too big", dict(kv=_kv(max_seq_len=1 << 20, max_pages_per_seq=1 << 14)),
     L.PRISM_ERR_UNSUPPORTED),
    ("kappa 0", dict(p=_params(kappa=0)), L.PRISM_ERR_INVALID_ARG),
    ("kappa > min_seq_len", dict(p=_params(kappa=4097)), L.PRISM_ERR_INVALID_ARG),
    ("kappa above 8192", dict(kv=_kv(min_seq_len=20000), p=_params(kappa=9000)),
     L.PRISM_ERR_UNSUPPORTED),
    ("negative window", dict(p=_params(window=-1)), L.PRISM_ERR_INVALID_ARG),
    ("stride 0", dict(p=_params(anchor_stride=0)), L.PRISM_ERR_INVALID_ARG),
    ("nan scale", dict(p=_params(softmax_scale=float("nan"))), L.PRISM_ERR_INVALID_ARG),
    ("negative pool_rho", dict(p=_params(pool_rho=-1)), L.PRISM_ERR_INVALID_ARG),
    ("rank pool above 32768", dict(p=_params(pool_rho=17)), L.PRISM_ERR_UNSUPPORTED),
    ("misaligned k", dict(kv=_kv(k_pages=FAKE + 2)), L.PRISM_ERR_INVALID_ARG),
    ("negative new_keys", dict(kv=_kv(new_keys=-1)), L.PRISM_ERR_INVALID_ARG),
    ("new_keys above 64", dict(kv=_kv(k_codes=FAKE, k_scales=FAKE, new_keys=65)),
     L.PRISM_ERR_UNSUPPORTED),
    ("null workspace", dict(ws=None), L.PRISM_ERR_WORKSPACE),
    ("misaligned workspace", dict(ws=FAKE + 16), L.PRISM_ERR_WORKSPACE),
    ("small workspace", dict(nbytes=1024), L.PRISM_ERR_WORKSPACE),
]


@pytest.mark.parametrize("fn", ["score", "refine", "attn", "layer", "role", "dense"])
@pytest.mark.parametrize("name,args,want", CASES, ids=[c[0] for c in CASES])
def test_invalid_calls_rejected_on_host(fn, name, args, want):
    kv = args.get("kv", _kv()) if "kv" in args else _kv()
    p = args.get("p", _params())
    st = _call(fn, kv, p, ws=args.get("ws", FAKE), nbytes=args.get("nbytes", 1 << 40))
    assert st == want, (fn, name, st, tsa.prism_last_error())
    assert tsa.prism_last_error()


def test_negative_layer_rejected():
    assert _call("layer", _kv(), _params(), layer=-1) == L.PRISM_ERR_INVALID_ARG


def test_null_outputs_rejected():
    lib = tsa.lib()
    kv, p = _kv(), _params()
    assert lib.prism_score_topk(ctypes.byref(kv), FAKE, ctypes.byref(p), None, None, FAKE, 1 << 40,
                                None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_sparse_attn(ctypes.byref(kv), FAKE, ctypes.byref(p), FAKE, None, FAKE,
                                 1 << 40, None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_score_topk(ctypes.byref(kv), None, ctypes.byref(p), FAKE, None, FAKE, 1 << 40,
                                None) == L.PRISM_ERR_INVALID_ARG


def test_valid_call_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake addresses must not reach a kernel")
    for fn in ("score", "refine", "attn", "layer", "role", "dense"):
        st = _call(fn, _kv(), _params())
        assert st == L.PRISM_ERR_HIP, (fn, st)
        assert "device" in tsa.prism_last_error().lower()


def test_profile_hook_argument_checks():
    lib = tsa.lib()
    assert lib.prism_profile_events(99, None, None, 0) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_profile_events(0, None, None, -1) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_profile_events(0, None, None, 0) == L.PRISM_OK
    assert lib.prism_profile_launches(0) == 0
    assert lib.prism_profile_launches(42) == -1
    assert lib.prism_profile_launches(3) == 0


def test_refine_anchor_idx_needed_for_the_window_pool_only():
    """With the window pool the pool is built from anchor_idx (NULL rejected);
    with the rank-expanded pool the call re-scores the pool in the workspace
    and anchor_idx is not read (NULL accepted; without a GPU the call then
    fails on the device check)."""
    import torch
    lib = tsa.lib()
    kv = _kv()
    pw, pr = _params(), _params(pool_rho=4)
    assert lib.prism_refine_topk(ctypes.byref(kv), FAKE, ctypes.byref(pw), None, FAKE, None, None,
                                 None, FAKE, 1 << 40, None) == L.PRISM_ERR_INVALID_ARG
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake addresses must not reach a kernel")
    assert lib.prism_refine_topk(ctypes.byref(kv), FAKE, ctypes.byref(pr), None, FAKE, None, None,
                                 None, FAKE, 1 << 40, None) == L.PRISM_ERR_HIP


def test_pattern_roles_of_the_pages_patterns():
    """prism_pattern_role reads every letter of the pages' patterns (Table 4:
    F proposal, S refined; Table 9: F, R, S) and rejects malformed ones."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "layer_patterns.json")) as f:
        pats = json.load(f)
    for table4, key, letters in ((True, "table4", {"F": 0, "S": 1}),
                                 (False, "table9", {"F": 0, "R": 1, "S": 2})):
        for e in pats[key]["patterns"].values():
            pat = e["pattern"]
            got = [tsa.prism_pattern_role(pat, l, table4=table4) for l in range(len(pat))]
            assert got == [letters[c] for c in pat]
            assert tsa.prism_pattern_role(pat, len(pat), table4=table4) == -1
    for pat, layer, t4 in (("", 0, False), ("RFS", 1, False), ("SFF", 1, False),
                           ("FXS", 0, False), ("FRS", 0, True), ("FS", -1, False)):
        assert tsa.prism_pattern_role(pat, layer, table4=t4) == -1, (pat, layer, t4)
    assert tsa.lib().prism_pattern_role(None, 0, 0) == -1


def test_decode_layer_role_argument_checks():
    lib = tsa.lib()
    kv, p = _kv(), _params()
    for role in (-1, 3, 99):
        assert _call("role", kv, p, role=role) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_decode_layer_role(2, ctypes.byref(kv), FAKE, ctypes.byref(p), None, FAKE,
                                       FAKE, 1 << 40, None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_decode_layer_role(0, ctypes.byref(kv), FAKE, ctypes.byref(p), FAKE, None,
                                       FAKE, 1 << 40, None) == L.PRISM_ERR_INVALID_ARG
    with pytest.raises(tsa.PrismError):
        tsa.prism_decode_layer_role("X", _FakeKV(kv), FAKE, p, FAKE, FAKE, workspace=(FAKE, 1 << 40),
                                    stream=0)


class _FakeKV:
    def __init__(self, struct):
        self.struct = struct


def test_int2_cache_fields_checked_on_host():
    """k_codes and k_scales go together and are 16-byte aligned, in every call
    that reads the cache; prism_quantize_keys needs both outputs."""
    lib = tsa.lib()
    for fn in ("score", "refine", "attn", "layer", "role"):
        assert _call(fn, _kv(k_codes=FAKE), _params()) == L.PRISM_ERR_INVALID_ARG, fn
        assert _call(fn, _kv(k_scales=FAKE), _params()) == L.PRISM_ERR_INVALID_ARG, fn
        assert _call(fn, _kv(k_codes=FAKE + 8, k_scales=FAKE), _params()) == L.PRISM_ERR_INVALID_ARG
    kv = _kv()
    assert lib.prism_quantize_keys(None, 1, FAKE, FAKE, None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_quantize_keys(ctypes.byref(kv), 1, None, FAKE, None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_quantize_keys(ctypes.byref(kv), 1, FAKE, None, None) == L.PRISM_ERR_INVALID_ARG
    assert lib.prism_quantize_keys(ctypes.byref(kv), 1, FAKE + 4, FAKE, None) == \
        L.PRISM_ERR_INVALID_ARG
    bad = _kv(head_dim=64)
    assert lib.prism_quantize_keys(ctypes.byref(bad), 1, FAKE, FAKE, None) == L.PRISM_ERR_UNSUPPORTED
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake addresses must not reach a kernel")
    assert lib.prism_quantize_keys(ctypes.byref(kv), 1, FAKE, FAKE, None) == L.PRISM_ERR_HIP
    assert _call("score", _kv(k_codes=FAKE, k_scales=FAKE), _params()) == L.PRISM_ERR_HIP
    # new_keys: up to 64 accepted (ignored without codes); prism_quantize_keys does not read it
    for fn in ("score", "refine", "attn", "layer", "role", "dense"):
        assert _call(fn, _kv(k_codes=FAKE, k_scales=FAKE, new_keys=64), _params()) == \
            L.PRISM_ERR_HIP, fn
        assert _call(fn, _kv(new_keys=7), _params()) == L.PRISM_ERR_HIP, fn
    odd = _kv(new_keys=1000)
    assert lib.prism_quantize_keys(ctypes.byref(odd), 1, FAKE, FAKE, None) == L.PRISM_ERR_HIP
    # prism_quantize_keys reads neither kv->k_codes nor kv->k_scales: a half-set
    # or misaligned pair there is not an error for it
    for kvx in (_kv(k_codes=FAKE), _kv(k_scales=FAKE), _kv(k_codes=FAKE + 8, k_scales=FAKE)):
        assert lib.prism_quantize_keys(ctypes.byref(kvx), 1, FAKE, FAKE, None) == L.PRISM_ERR_HIP


def test_noalloc_entry_point_checks_on_host():
    """prism_decode_layer_noalloc validates like prism_decode_layer, rejects
    shapes whose workspace exceeds the static 64 MiB with PRISM_ERR_WORKSPACE
    before touching a device, and reports a missing GPU as PRISM_ERR_HIP."""
    lib = tsa.lib()
    assert tsa.PRISM_STATIC_WORKSPACE_BYTES == 64 << 20

    def call(kv, p, layer=0, anchor=FAKE, out=FAKE):
        return lib.prism_decode_layer_noalloc(layer, ctypes.byref(kv) if kv is not None else None,
                                              FAKE, ctypes.byref(p) if p is not None else None,
                                              anchor, None, out, None)
    assert call(None, _params()) == L.PRISM_ERR_INVALID_ARG
    assert call(_kv(), None) == L.PRISM_ERR_INVALID_ARG
    assert call(_kv(head_dim=64), _params()) == L.PRISM_ERR_UNSUPPORTED
    assert call(_kv(), _params(kappa=0)) == L.PRISM_ERR_INVALID_ARG
    assert call(_kv(), _params(), layer=-1) == L.PRISM_ERR_INVALID_ARG
    assert call(_kv(), _params(), anchor=None) == L.PRISM_ERR_INVALID_ARG
    assert call(_kv(), _params(), out=None) == L.PRISM_ERR_INVALID_ARG
    # 16 x 8 problems over 262144-token lists need far more than 64 MiB
    big = _kv(batch=16, num_pages=65536, max_pages_per_seq=4096, max_seq_len=262144,
              min_seq_len=8192)
    need = lib.prism_workspace_size(ctypes.byref(big), ctypes.byref(_params()))
    assert need > tsa.PRISM_STATIC_WORKSPACE_BYTES
    assert call(big, _params()) == L.PRISM_ERR_WORKSPACE
    assert b"static workspace" in lib.prism_last_error()
    small = _kv()
    assert lib.prism_workspace_size(ctypes.byref(small), ctypes.byref(_params())) <= \
        tsa.PRISM_STATIC_WORKSPACE_BYTES
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake addresses must not reach a kernel")
    assert call(small, _params()) == L.PRISM_ERR_HIP
