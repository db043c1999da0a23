#!/usr/bin/env python3
"""Decode-step benchmark of token-sparse GQA attention with proposal-refined
cross-layer index sharing on one MI355X.

A step is one decode step's attention path over every layer of the workload:
prism_decode_layer(l) for l = 0..N-1 (anchor layers: relevance of the whole
cache, exact top-kappa, SparseAttn; refined layers: window pool, re-score,
top-kappa, SparseAttn).  Inputs are seeded synthetic tensors of the workload's
shapes, resident in HBM before timing starts.

Two timed regions of K steps each, after W warm-up steps:
  1. the step captured once as a HIP graph and replayed K times: `value` and
     `ms_per_step` (with --eager, or if capture fails, region 2 is reported);
  2. the same steps launched eagerly from the host, each kernel's start and end
     recorded by its own dispatch (prism_profile_events): the per-kernel
     durations, the roofline of the dominant kernel and `eager_ms_per_step`.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor, as_completed

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SRC = os.path.join(ROOT, "token_sparse_attention_gqa_amd", "csrc", "prism_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the benchmark needs for raw events."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def layer_roles(wl, pattern=None):
    """One letter per layer: F (proposal / anchor), R (refined), S (shared)."""
    if pattern:
        return list(pattern)
    return ["F" if wl.is_anchor(l) else "R" for l in range(wl.num_layers)]


def launches_per_step(wl, cus, pool_rho=0, roles=None, dense=False):
    """Kernel launches of each kind in one decode step, mirroring the library's
    choice: layers select inside their attention kernel when G <= 8 and every
    attention workgroup of the layer fits the device at once (problems x
    ceil(kappa / 128) <= compute units; anchor layers also need contexts up to
    196608), else a selection kernel per layer precedes the attention, and a
    refined layer whose pool can exceed 16384 entries is classified first.
    Shared layers launch the attention and its merge only.  With INT2 keys
    the newest key of every layer is quantized inside the layer's scoring
    kernel (a shared layer's, which scores nothing, inside its attention
    launch)."""
    import synth
    if dense:   # every layer: the dense chunks and their merge
        return {"anchor_score": 0, "refine_score": 0, "select": 0, "attention": 0, "classify": 0,
                "merge": wl.num_layers, "quantize": 0, "dense": wl.num_layers}
    roles = roles or layer_roles(wl)
    na, nr = roles.count("F"), roles.count("R")
    L = int(synth.paging(wl).seq_lens.max())
    splits = -(-wl.kappa // 128)
    fused = wl.group <= 8 and wl.batch * wl.num_kv_heads * splits <= cus
    if pool_rho >= 1:   # rank pools: one more workgroup per problem writes the pool
        anchor_fused = (wl.group <= 8 and L <= 6144 * 32
                        and wl.batch * wl.num_kv_heads * (splits + 1) <= cus)
    else:
        anchor_fused = fused and L <= 6144 * 32
    n_cap = -(-L // 64) * 64
    pool_bound = min(n_cap, pool_rho * wl.kappa if pool_rho >= 1
                     else wl.kappa * (2 * wl.window + 1))
    pool_classify = not fused and pool_bound > 16384 and pool_bound > wl.kappa
    # the fused rank path classifies for kappa (and rho*kappa in the same pass)
    anchor_need = pool_rho * wl.kappa if (pool_rho >= 1 and not anchor_fused) else wl.kappa
    return {"anchor_score": na, "refine_score": nr,
            "select": (0 if anchor_fused else na) + (0 if fused else nr),
            "attention": wl.num_layers,
            "classify": (na if (L > 16384 and L > anchor_need) else 0)
                        + (nr if pool_classify else 0),
            "merge": wl.num_layers, "quantize": 0, "dense": 0}


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    e = t.get("kernels", {}).get(kernel)
    if not e or e.get("workload") != workload:
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(wl, host, seconds, pool_rho=0, roles=None, int2=False):
    """The CPU oracle, as it stands, on a bounded sample of the workload: one
    anchor layer and one refined layer (and the attention alone, for shared
    layers) for as many (sequence, KV head) problems as fit in about
    `seconds`, extrapolated to a whole decode step."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    pg = synth.paging(wl)
    G = wl.group
    la, lr = 0, 1
    qa, qr = oracle.bf16_to_f64(host[la].q), oracle.bf16_to_f64(host[lr].q)
    probs = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    ta, tr, ts, done = [], [], [], 0
    t_start = time.perf_counter()
    for b, g in probs:
        L = int(pg.seq_lens[b])
        t0 = time.perf_counter()
        A, sa = oracle.anchor_select(qa[b, g * G:(g + 1) * G], host[la].k_pages,
                                     pg.block_table[b], g, L, wl.kappa, wl.page_size, int2=int2)
        pool = oracle.rank_pool(sa, np.arange(L), pool_rho, wl.kappa) if pool_rho >= 1 else None
        oracle.attend(qa[b, g * G:(g + 1) * G], host[la].k_pages, host[la].v_pages,
                      pg.block_table[b], g, A, wl.page_size, oracle.default_scale(wl.head_dim))
        t1 = time.perf_counter()
        if pool is not None:
            T, _ = oracle.refine_in_pool(qr[b, g * G:(g + 1) * G], host[lr].k_pages,
                                         pg.block_table[b], g, pool, wl.kappa, wl.page_size,
                                         int2=int2)
        else:
            T, _, _ = oracle.refined_select(qr[b, g * G:(g + 1) * G], host[lr].k_pages,
                                            pg.block_table[b], g, L, wl.kappa, wl.page_size, A,
                                            wl.window, int2=int2)
        oracle.attend(qr[b, g * G:(g + 1) * G], host[lr].k_pages, host[lr].v_pages,
                      pg.block_table[b], g, T, wl.page_size, oracle.default_scale(wl.head_dim))
        t2 = time.perf_counter()
        if roles is not None and "S" in roles:   # a shared layer: attention over A only
            oracle.attend(qr[b, g * G:(g + 1) * G], host[lr].k_pages, host[lr].v_pages,
                          pg.block_table[b], g, A, wl.page_size,
                          oracle.default_scale(wl.head_dim))
        t3 = time.perf_counter()
        ta.append(t1 - t0)
        tr.append(t2 - t1)
        ts.append(t3 - t2)
        done += 1
        if time.perf_counter() - t_start > seconds:
            break
    roles = roles or [("F" if wl.is_anchor(l) else "R") for l in range(wl.num_layers)]
    n_anchor, n_ref, n_sh = roles.count("F"), roles.count("R"), roles.count("S")
    P = len(probs)
    step_s = P * (n_anchor * float(np.mean(ta)) + n_ref * float(np.mean(tr))
                  + n_sh * float(np.mean(ts)))
    return {"value": wl.batch / step_s, "unit": "tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"oracle (numpy float64"
                       + (", INT2 keys quantized from bf16 on the fly" if int2 else "")
                       + f") on layer {la} (anchor) and layer {lr} (refined) "
                       f"for {done} of {P} (sequence, KV head) problems "
                       f"({time.perf_counter() - t_start:.1f} s); per-problem times "
                       f"extrapolated to {n_anchor} anchor + {n_ref} refined"
                       + (f" + {n_sh} shared (attention only)" if n_sh else "")
                       + f" layers x {P} problems"),
            "ms_per_step": step_s * 1e3}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3-8b-128k-planted")
    ap.add_argument("--pool-rho", type=int, default=0, metavar="RHO",
                    help="refined layers re-score the anchor's top RHO*kappa tokens (Eq. 4) "
                         "instead of the +-w window pool (0, the default)")
    ap.add_argument("--pattern", default="", metavar="LETTERS",
                    help="layer roles, one letter per layer: F proposal (anchor), R refined, "
                         "S shared (reuses the nearest F or R layer's set); default: every "
                         "anchor_stride-th layer F, the others R")
    ap.add_argument("--int2", action="store_true",
                    help="score from INT2 proposal keys (Section 4.2): every layer's keys are "
                         "quantized before timing, and each timed layer quantizes its newest key "
                         "(inside its scoring kernel; a shared layer inside its attention launch)")
    ap.add_argument("--dense", action="store_true",
                    help="dense decode attention over every cached token at every layer (the "
                         "full-attention baseline of the sparse path); --cpu-seconds is ignored")
    ap.add_argument("--distinct-layers", type=int, default=0, metavar="N",
                    help="generate only N layers' inputs and give layer l those of layer l mod N "
                         "(for workloads whose full KV cache does not fit host memory for "
                         "generation; every layer still reads its own N-th of the data from HBM)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU-oracle baseline sample (0 skips it)")
    ap.add_argument("--eager", action="store_true",
                    help="report eager launches only (no HIP graph capture of the step)")
    ap.add_argument("--graph", action="store_true", help=argparse.SUPPRESS)  # the default
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times and "
                         "exit: the known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe > 0:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return

    import synth
    import token_sparse_attention_gqa_amd as tsa

    wl = synth.BY_NAME[args.workload]
    pg = synth.paging(wl)
    if args.pattern:
        bad = [l for l in range(len(args.pattern)) if tsa.prism_pattern_role(args.pattern, l) < 0]
        if bad or len(args.pattern) != wl.num_layers:
            print(f"--pattern must be {wl.num_layers} letters F/R/S starting with F",
                  file=sys.stderr, flush=True)
            sys.exit(2)
    roles = layer_roles(wl, args.pattern)
    dev = torch.device("cuda:0")
    tsa.lib()
    hip = Hip()

    # ---- inputs, resident in HBM ------------------------------------------------
    t0 = time.perf_counter()
    nd = min(args.distinct_layers, wl.num_layers) if args.distinct_layers > 0 else wl.num_layers
    log(f"[bench] generating {nd} of {wl.num_layers} layers of {wl.name} "
        f"(B={wl.batch}, L={int(pg.seq_lens.max())}, {wl.num_q_heads}q/{wl.num_kv_heads}kv)")
    bt = torch.from_numpy(pg.block_table).to(dev)
    sl = torch.from_numpy(pg.seq_lens).to(dev)
    L_max, L_min = int(pg.seq_lens.max()), int(pg.seq_lens.min())
    q_dev, kv_dev, host_keep = {}, {}, {}
    keep_host = {0, 1} if args.cpu_seconds > 0 else set()
    nthreads = synth.default_threads()
    with ThreadPoolExecutor(nthreads) as ex:
        futs = {ex.submit(synth.layer_inputs, wl, l, 1): l for l in range(nd)}
        for n_done, f in enumerate(as_completed(futs), 1):
            l = futs[f]
            li = f.result()
            q_dev[l] = torch.from_numpy(li.q.view(np.int16)).to(dev)
            k = torch.from_numpy(li.k_pages.view(np.int16)).to(dev)
            v = torch.from_numpy(li.v_pages.view(np.int16)).to(dev)
            kv_dev[l] = tsa.KVCache(k, v, bt, sl, max_seq_len=L_max, min_seq_len=L_min)
            if args.int2:   # the prefill's quantization, before timing
                cs, ss = tsa.int2_shapes(k.shape[0], wl.num_kv_heads, wl.page_size)
                codes = torch.zeros(cs, dtype=torch.uint8, device=dev)
                scales = torch.zeros(ss, dtype=torch.int16, device=dev)
                tsa.prism_quantize_keys(kv_dev[l], 0, codes, scales)
                # every step appends one key per layer: the layer's own call
                # quantizes it before scoring (new_keys = 1)
                kv_dev[l] = kv_dev[l].with_int2(codes, scales, new_keys=1)
            if l in keep_host:
                host_keep[l] = li
            del li
            log(f"[bench] layer {l} resident ({n_done}/{nd}, "
                f"{time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()

    p = tsa.params(wl.num_q_heads, wl.kappa, wl.anchor_stride, wl.window,
                   pool_rho=args.pool_rho)
    ws = torch.empty(tsa.prism_workspace_size(kv_dev[0], p), dtype=torch.uint8, device=dev)
    anchor = torch.zeros((wl.batch, wl.num_kv_heads, wl.kappa), dtype=torch.int32, device=dev)
    outs = torch.zeros((wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                       device=dev)
    stream = torch.cuda.current_stream()

    # raw addresses, resolved once: the per-layer call is then one C call
    ws_arg = (ws.data_ptr(), ws.numel())
    layer_args = [(kv_dev[l % nd], q_dev[l % nd].data_ptr(), outs[l].data_ptr())
                  for l in range(wl.num_layers)]
    anchor_ptr = anchor.data_ptr()

    role_ids = [tsa.ROLES[c] for c in roles]

    def step():
        s = torch.cuda.current_stream().cuda_stream  # the capture stream while recording
        if args.dense:
            for kv, qp, op in layer_args:
                tsa.prism_dense_attn(kv, qp, p, op, ws_arg, s)
            return
        for l, (kv, qp, op) in enumerate(layer_args):
            if args.pattern:
                tsa.prism_decode_layer_role(role_ids[l], kv, qp, p, anchor_ptr, op, ws_arg, s)
            else:
                tsa.prism_decode_layer(l, kv, qp, p, anchor_ptr, None, op, ws_arg, s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    rt = hip.rt
    rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    e_start, e_stop = hip.events(1)[0], hip.events(1)[0]

    # ---- timed region 1 (the reported value): the step captured once as a HIP
    #      graph, replayed K times ----------------------------------------------------
    graph_ms, graph_err = None, None
    if not args.eager:
        try:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step()
            for _ in range(max(1, args.warmup)):
                gr.replay()
            torch.cuda.synchronize()
            gs = torch.cuda.current_stream()
            wall0 = time.perf_counter()
            rt.hipEventRecord(e_start, ctypes.c_void_p(gs.cuda_stream))
            for _ in range(args.steps):
                gr.replay()
            rt.hipEventRecord(e_stop, ctypes.c_void_p(gs.cuda_stream))
            torch.cuda.synchronize()
            wall1 = time.perf_counter()
            graph_ms = hip.elapsed_ms(e_start, e_stop) / args.steps
            log(f"[bench] graph replay, {args.steps} steps: {graph_ms:.4f} ms/step "
                f"(wall {1e3 * (wall1 - wall0) / args.steps:.4f} ms/step)")
            del gr
        except Exception as exc:  # report it and fall back to eager launches
            graph_err = str(exc)[:200]
            log(f"[bench] graph capture failed ({graph_err}); reporting eager launches")
            torch.cuda.synchronize()

    # ---- timed region 2: eager launches, every kernel's start and end recorded
    #      by its dispatch (per-kernel durations and the roofline) -------------------
    per_step = launches_per_step(wl, torch.cuda.get_device_properties(dev).multi_processor_count,
                                 args.pool_rho, roles, args.dense)
    rings = {}
    for kind, n in per_step.items():
        cnt = n * args.steps
        rings[kind] = (hip.events(cnt), hip.events(cnt))
        tsa.prism_profile_events(kind, rings[kind][0], rings[kind][1])
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    rt.hipEventRecord(e_start, ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.steps):
        step()
    rt.hipEventRecord(e_stop, ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    eager_ms = hip.elapsed_ms(e_start, e_stop) / args.steps
    log(f"[bench] eager launches with per-kernel events, {args.steps} steps: {eager_ms:.4f} "
        f"ms/step (wall {1e3 * (wall1 - wall0) / args.steps:.4f} ms/step)")
    ms_per_step = graph_ms if graph_ms is not None else eager_ms

    kernels = {}
    for kind, (starts, stops) in rings.items():
        n = tsa.prism_profile_launches(kind)
        assert n == per_step[kind] * args.steps, (kind, n)
        durs = [hip.elapsed_ms(a, b) for a, b in zip(starts, stops)]
        kernels[kind] = {"launches_per_step": per_step[kind],
                         "avg_us": 1e3 * float(np.mean(durs)) if durs else 0.0,
                         "us_per_step": 1e3 * float(np.sum(durs)) / args.steps}
        tsa.prism_profile_events(kind, [], [])
        hip.destroy(starts + stops)

    # ---- algorithmic bytes ----------------------------------------------------------
    D2 = wl.head_dim * 2
    KB = 48 if args.int2 else D2   # key bytes scored per token: INT2 codes + scales, or bf16
    anchor_bytes = int(pg.seq_lens.astype(np.int64).sum()) * wl.num_kv_heads * KB
    attn_bytes = wl.batch * wl.num_kv_heads * wl.kappa * 2 * D2
    # pool sizes of the refined layers of this step (untimed pass, same inputs)
    pool_len = torch.zeros((wl.batch, wl.num_kv_heads), dtype=torch.int32, device=dev)
    tmp_idx = torch.zeros_like(anchor)
    pool_bytes = []
    for l in range(0 if args.dense else wl.num_layers):
        if roles[l] == "F":
            tsa.prism_score_topk(kv_dev[l % nd], q_dev[l % nd], p, anchor, None, ws)
        elif roles[l] == "R":
            tsa.prism_refine_topk(kv_dev[l % nd], q_dev[l % nd], p, anchor, tmp_idx, None, pool_len,
                                  None, ws)
            pool_bytes.append(int(pool_len.sum().item()) * KB)
    n_anchor = per_step["anchor_score"]
    quant_bytes = wl.batch * wl.num_kv_heads * (D2 + 48) if args.int2 else 0
    step_bytes = (n_anchor * anchor_bytes + sum(pool_bytes) + wl.num_layers * attn_bytes
                  + wl.num_layers * quant_bytes)
    dense_bytes = int(pg.seq_lens.astype(np.int64).sum()) * wl.num_kv_heads * 2 * D2
    if args.dense:
        step_bytes = wl.num_layers * dense_bytes
    algo = {"anchor_score": anchor_bytes,
            "refine_score": (sum(pool_bytes) / len(pool_bytes)) if pool_bytes else 0,
            "attention": attn_bytes, "dense": dense_bytes}
    for kind, k in kernels.items():
        if kind in algo and k["avg_us"] > 0:
            k["algorithmic_bytes_per_launch"] = algo[kind]
            k["GBps"] = algo[kind] / (k["avg_us"] * 1e-6) / 1e9

    dominant = max((k for k in kernels if k in algo), key=lambda k: kernels[k]["us_per_step"])
    dk = kernels[dominant]
    achieved = dk["GBps"]
    roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(dominant, wl.name),
                "algorithmic_bytes_per_launch": int(algo[dominant]),
                "avg_launch_us": round(dk["avg_us"], 3)}

    result = {
        "metric": "sparse decode-attn tokens/sec + % HBM roofline at 128K, kappa=2048 (1 GPU)",
        "value": round(wl.batch * 1e3 / ms_per_step, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; paged bf16 K/V with RoPE, planted sinks and drifting clusters)"
                if wl.planted else "synthetic (seeded; paged bf16 K/V with RoPE)",
        "config": {"workload": wl.name, "batch": wl.batch, "context": L_max,
                   "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "layers": wl.num_layers,
                   **({"layer_roles": args.pattern} if args.pattern
                      else {"anchor_stride": wl.anchor_stride}),
                   "kappa": wl.kappa, "window": wl.window,
                   "page_size": wl.page_size,
                   **({"distinct_layers": nd} if nd < wl.num_layers else {}),
                   **({"pool": "rank", "pool_rho": args.pool_rho} if args.pool_rho >= 1
                      else {"pool": "window"}),
                   "keys": "int2" if args.int2 else "bf16",
                   **({"attention": "dense"} if args.dense else {})},
        "roofline": roofline,
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
    }

    result["launch"] = "hip_graph_replay" if graph_ms is not None else "eager"
    result["eager_ms_per_step"] = round(eager_ms, 5)
    if graph_err:
        result["graph_error"] = graph_err

    if args.cpu_seconds > 0 and not args.dense:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cb = cpu_baseline(wl, host_keep, args.cpu_seconds, args.pool_rho, roles, args.int2)
        result["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                  for k, v in cb.items()}
    else:
        result["cpu_baseline"] = None
    hip.destroy([e_start, e_stop])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
