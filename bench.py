#!/usr/bin/env python3
"""Benchmark of the DCA + vertical-slash sparse prefill attention on one MI355X.

One step is one layer's prefill attention of one workload: for each prefill
chunk, the vertical-slash index build followed by the DCA attention
(key rotation, sparse plan, attention, LSE merge).  Inputs are seeded
synthetic tensors already resident in HBM; the timed region holds exactly
``--steps`` steps between two device synchronisations.

Prints one JSON line:  value = computed-block TFLOP/s of the whole step
(F_blocks / step time), ms_per_step = ms per layer, both from the median of
cold steps (a 512 MiB write evicts the caches before each).  F_attended (the
(row, key) pairs each row attends, times 4d) is reported beside F_blocks.
The roofline object reports the attention kernel alone (HIP events around it
on the stream it runs on); the cpu_baseline object times the fp64 oracle on a
bounded sample of the same workload on the host cores and extrapolates to the
full step.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "prefill attention TFLOP/s on computed blocks + ms/layer, 7B heads, 128K–1M"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through libamdhip64 (torch's events see only its current stream)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        t = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)


def kernel_source_hash() -> str:
    src = os.path.join(ROOT, "sparse_dual_chunk_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def traffic_from_profile(workload: str, exact: bool):
    """HBM bytes per attention launch from the committed counter summary, if it was taken
    on the current attention kernel source, for this workload and the block-cover
    semantics; else None."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if exact or not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("attn_source_sha256_16") != kernel_source_hash() or d.get("workload") != workload:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inputs, p0s, f_blocks_total: float, n_blocks_total: int):
    """Oracle timing on a bounded sample (about 10-15 s): index scores of three heads, attention of
    five query blocks of one head."""
    from oracle import dca_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    inp = inputs[-1]
    cfg = dict(h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local, rope_base=w.rope_base,
               yarn_s=w.yarn_s, vs_k_vertical=w.k_vertical, vs_k_slash=w.k_slash, vs_last_q=w.vs_last_q)
    t0 = time.perf_counter()
    v_idx = s_off = None
    t_index_head = 0.0
    if w.sparse:
        v_idx, s_off, _ = O.vs_index(inp["q"], inp["k"], inp["p0"], cfg, heads=[0, 1, 2])
        t_index_head = (time.perf_counter() - t0) / 3
    nb = (inp["n_q"] + 63) // 64
    blocks = sorted({nb - 1, (3 * nb) // 4, nb // 2, nb // 4, nb // 8}, reverse=True)
    t1 = time.perf_counter()
    fb_sample = 0
    for b in blocks:
        _, _, keys = O.attention_block(inp["q"], inp["k"], inp["v"], inp["p0"], 0, b, cfg, v_idx, s_off)
        rows = min(64, inp["n_q"] - 64 * b)
        fb_sample += 4 * 128 * rows * len(keys)
    t_att = time.perf_counter() - t1
    n_calls = len(p0s)
    # extrapolate: index per head x heads x calls, attention by the computed-block share
    t_step = t_index_head * w.h_q * n_calls + t_att * (f_blocks_total / max(fb_sample, 1))
    return {
        "value": f_blocks_total / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 oracle on the host: index scores of query heads 0-2 of the last chunk "
                   f"({t_index_head:.1f} s per head) and attention of query blocks {blocks} of head 0 "
                   f"({t_att:.1f} s, {fb_sample / 1e9:.1f} GFLOP); step time extrapolated to "
                   f"{w.h_q} heads x {n_calls} call(s) and to F_blocks"),
        "seconds_measured": round(time.perf_counter() - t0, 2),
        "ms_per_step_extrapolated": round(t_step * 1e3, 1),
    }


def decode_traffic_from_profile(n_tokens: int, page_keys: int):
    """HBM bytes per decode launch from the committed counter summary, if it was taken on
    the current decode kernel source and the same step (one token, contiguous cache); else None."""
    if n_tokens != 1 or page_keys:
        return None
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    src = os.path.join(ROOT, "sparse_dual_chunk_amd", "csrc", "decode.hip")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("decode_source_sha256_16") != hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]:
        return None
    return d.get("hbm_bytes_per_launch")


DECODE_METRIC = "decode-step attention over a 1M-key KV cache, 7B heads: cache GB/s (K + V read per step)"


def bench_decode(args) -> int:
    """One step = the attention of ``--decode-tokens`` new tokens over the whole 1,048,576-key
    cache of the 1M workload's layer (7B heads).  The rotated key cache is built before
    the timed region (its keys enter the cache once, at prefill time)."""
    import torch
    import sparse_dual_chunk_amd as S
    from oracle import dca_oracle as O

    w = W.C5_7B_1M
    n_k, n_t = w.n_k_total, args.decode_tokens
    log(f"decode: {n_t} token(s) over {n_k} cached keys, generating inputs (seed {args.seed})")
    k, v = W.make_keys_values(w, n_k, args.seed)
    q = W.make_queries(w, n_k - n_t, n_t, seed=args.seed + 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    cfg = S.Config(n_q=n_t, n_k=n_k, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                   rope_base=w.rope_base, yarn_s=w.yarn_s, split_k=args.split_k)
    K, V, Q = dev(k), dev(v), dev(q)
    if args.page_keys:
        # a pool of pages in a seeded random order (one spare page per 64)
        n_table = (n_k + args.page_keys - 1) // args.page_keys
        n_pages = n_table + n_table // 64 + 1
        table = np.random.default_rng([args.seed, 9]).permutation(n_pages)[:n_table]
        cache = S.PagedKV.allocate(n_pages, args.page_keys, w.h_kv, table)
        S.dca_paged_append(K, V, 0, cfg, cache)
        run = lambda **kw: S.dca_decode_paged(Q, cache, cfg, out, ws, **kw)
    else:
        cache = S.KeyCache.allocate(n_k, w.h_kv)
        S.dca_key_cache_append(K, 0, cfg, cache)
        run = lambda **kw: S.dca_decode(Q, cache, V, cfg, out, ws, **kw)
    del K
    out = torch.empty(Q.shape, dtype=torch.int16, device="cuda")
    ws = torch.empty(S.dca_decode_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    hev = HipEvents()
    n_ev = 2 * S.DCA_STAGE_COUNT
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [hev.create(n_ev) for _ in range(args.steps)]
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        run(stage_events=evs[st])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: float(np.mean([hev.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs]))
                for i, name in enumerate(S.STAGES)}
    attn_ms = stage_ms["attention"]
    # the same step captured once in a HIP graph and replayed (a serving loop's launch path)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
    # algorithmic bytes of the attention kernel: every K (rotated, hi) and V row once,
    # the query rows, and the parts' fp32 partials written
    ws_parts = S.dca_decode_workspace_size(cfg)
    kv_bytes = 2 * n_k * w.h_kv * w.head_dim * 2
    part_bytes = ws_parts - 2 * 3 * n_t * w.h_q * w.head_dim * 2
    algo_bytes = kv_bytes + 3 * n_t * w.h_q * w.head_dim * 2 + part_bytes
    achieved = algo_bytes / (attn_ms / 1e3) / 1e9
    result = {
        "metric": DECODE_METRIC,
        "value": round(kv_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7b_decode_1m_cache" + (f"_paged_{args.page_keys}" if args.page_keys else ""),
                   "n_tokens": n_t, "n_k": n_k, "h_q": w.h_q, "h_kv": w.h_kv,
                   "head_dim": w.head_dim, "dca_chunk": w.dca_chunk, "dca_local": w.dca_local,
                   "rope_base": w.rope_base, "yarn_s": w.yarn_s, "seed": args.seed},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": decode_traffic_from_profile(n_t, args.page_keys),
            "kernel": "dca_decode_kernel",
            "avg_launch_ms": round(attn_ms, 5),
            "algorithmic_bytes_per_launch": algo_bytes,
        },
        "tokens_per_s_per_layer": round(n_t / (ms_per_step / 1e3), 1),
        "graph_ms_per_step": round(graph_ms_per_step, 4),
        "stage_ms": {k2: round(v2, 5) for k2, v2 in stage_ms.items()},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle's decode of one query head")
        t1 = time.perf_counter()
        O.decode_attention(q, k, v, dict(h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                                         rope_base=w.rope_base, yarn_s=w.yarn_s), heads=[0])
        t_head = time.perf_counter() - t1
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count() or 1
        t_step = t_head * w.h_q
        result["cpu_baseline"] = {"value": round(kv_bytes / t_step / 1e9, 4), "unit": "GB/s", "cores": int(cores),
                                  "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"fp64 oracle decode of query head 0 over the whole cache "
                                            f"({t_head:.1f} s), extrapolated to {w.h_q} heads"}
    print(json.dumps(result), flush=True)
    return 0


SEQUENCE_METRIC = "whole-prompt chunked prefill ms per layer (index + attention of every chunk)"


def bench_sequence(args) -> int:
    """One step = the chunked prefill of a whole prompt (default: the 14B 256K prompt of 8
    chunks), every chunk's key append, index build and attention, through
    dca_prefill_sequence.  Compared: fixed 32K-row chunks against the equal-time schedule
    (the library's cost coefficients, the same number of chunks), each with the index
    builds in order on one stream and one chunk ahead on a second stream."""
    import torch
    import sparse_dual_chunk_amd as S

    w = W.WORKLOADS[args.workload] if args.workload != W.C5_7B_1M.name else W.C4_14B_256K
    n = w.n_k_total
    fixed = list(range(0, n, 32768)) + [n]
    log(f"sequence: {w.name}, {n} tokens, generating inputs (seed {args.seed})")
    k, v = W.make_keys_values(w, n, args.seed)
    q = np.concatenate([W.make_queries(w, a, b - a, args.seed) for a, b in zip(fixed[:-1], fixed[1:])])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    Q, K, V = dev(q), dev(k), dev(v)
    del q, k, v
    cfg = S.Config(n_q=n, n_k=n, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                   rope_base=w.rope_base, yarn_s=w.yarn_s, head_dim=w.head_dim, vs_last_q=w.vs_last_q,
                   vs_k_vertical=w.k_vertical, vs_k_slash=w.k_slash, split_k=args.split_k)
    sparse = w.sparse
    cost = S.dca_chunk_cost_default(cfg, sparse)
    equal, _ = S.dca_chunk_schedule(n, len(fixed) - 1, n, cost)
    schedules = {"fixed_32k": fixed, "equal_time": equal}
    fitted_cost = None
    cache = S.KeyCache.allocate(n, w.h_kv)
    out = torch.empty(Q.shape, dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    hev = HipEvents()
    results = {}
    def model_pairs(a, b, cap):
        e = np.arange(a, b, 64, dtype=np.float64)
        r = np.minimum(64, b - e)
        e = e + r
        if cap > 0:
            e = -e * np.expm1(-cap / e)
        return float((r * e).sum())

    def fit_cost(bounds, chunk_ms, index_ms):
        """Least-squares (non-negative) fit of the cost coefficients to measured chunk times (us)."""
        from scipy.optimize import nnls
        ab = list(zip(bounds[:-1], bounds[1:]))
        A = np.array([[1.0, b - a, model_pairs(a, b, cost.cover_cap)] for a, b in ab])
        x, _ = nnls(A, 1e3 * np.asarray(chunk_ms))
        ki = np.array([[1.0, b] for a, b in ab])
        y, _ = nnls(ki, 1e3 * np.asarray(index_ms))
        return S.chunk_cost(per_call=x[0] + y[0], per_row=x[1], per_index_key=y[1] if sparse else 0.0,
                            per_pair=x[2], cover_cap=cost.cover_cap)

    order = list(schedules)
    while order:
        name = order.pop(0)
        bounds = schedules[name]
        nc = len(bounds) - 1
        ws = torch.empty(max(S.dca_prefill_sequence_workspace_size(cfg, bounds, sparse, ov) for ov in (False, True)),
                         dtype=torch.uint8, device="cuda")
        pairs = torch.zeros(nc, dtype=torch.int64, device="cuda")
        for overlap in (False, True):
            tag = f"{name}{'_overlap' if overlap else ''}"
            istream = side.cuda_stream if overlap else None
            for _ in range(args.warmup):
                S.dca_prefill_sequence(Q, K, V, bounds, cfg, cache, out, ws, sparse=sparse, index_stream=istream)
            torch.cuda.synchronize()
            tot, ch, ix = [], [], []
            for _ in range(args.steps):
                ev = hev.create(2)
                cev = hev.create(2 * nc)
                iev = hev.create(2 * nc)
                st = torch.cuda.current_stream().cuda_stream
                hev.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
                hev.h.hipEventRecord(ctypes.c_void_p(ev[0]), ctypes.c_void_p(st))
                S.dca_prefill_sequence(Q, K, V, bounds, cfg, cache, out, ws, sparse=sparse, index_stream=istream,
                                       cover_pairs=pairs, chunk_events=cev, index_events=iev)
                hev.h.hipEventRecord(ctypes.c_void_p(ev[1]), ctypes.c_void_p(st))
                torch.cuda.synchronize()
                tot.append(hev.elapsed_ms(ev[0], ev[1]))
                ch.append([hev.elapsed_ms(cev[2 * c], cev[2 * c + 1]) for c in range(nc)])
                ix.append([hev.elapsed_ms(iev[2 * c], iev[2 * c + 1]) for c in range(nc)])
            chunk_ms = np.median(np.array(ch), axis=0)
            index_ms = np.median(np.array(ix), axis=0)
            f_blocks = 4 * w.head_dim * float(pairs.sum().item())
            results[tag] = {
                "bounds": bounds,
                "total_ms": round(float(np.median(tot)), 3),
                "chunk_attention_ms": [round(float(x), 3) for x in chunk_ms],
                "chunk_index_ms": [round(float(x), 3) for x in index_ms],
                "chunk_max_over_mean": round(float(chunk_ms.max() / chunk_ms.mean()), 4),
                "attention_tflops_on_computed_blocks": round(f_blocks / (float(chunk_ms.sum()) / 1e3) / 1e12, 1),
            }
            log(f"{tag}: total {results[tag]['total_ms']} ms, chunk max/mean {results[tag]['chunk_max_over_mean']}")
            if name == "fixed_32k" and not overlap:
                # the cost model refitted to this GPU's measured chunk times, then scheduled again
                fitted_cost = fit_cost(bounds, chunk_ms, index_ms)
                schedules["equal_time_fitted"], _ = S.dca_chunk_schedule(n, nc, n, fitted_cost)
                order.append("equal_time_fitted")
        del ws
    best = min(results, key=lambda t: results[t]["total_ms"])
    result = {
        "metric": SEQUENCE_METRIC,
        "value": results[best]["total_ms"],
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": results[best]["total_ms"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_whole_prompt", "n_tokens": n, "h_q": w.h_q, "h_kv": w.h_kv,
                   "k_vertical": w.k_vertical, "k_slash": w.k_slash, "best": best,
                   "cost_model": {"per_call": cost.per_call, "per_row": cost.per_row,
                                  "per_index_key": cost.per_index_key, "per_pair": cost.per_pair,
                                  "cover_cap": int(cost.cover_cap)},
                   "fitted_cost_model": None if fitted_cost is None else
                   {"per_call": fitted_cost.per_call, "per_row": fitted_cost.per_row,
                    "per_index_key": fitted_cost.per_index_key, "per_pair": fitted_cost.per_pair}},
        "runs": results,
    }
    print(json.dumps(result), flush=True)
    return 0


MOE_METRIC = "fused MoE layer memory bandwidth (routed experts' weights + activations / layer time)"


def bench_moe(args) -> int:
    """One step = one fused MoE layer (64 experts, top-8, d_model 3584, d_ff 2560) over a
    generation batch of --moe-tokens tokens: slot sort, gate/up product + SwiGLU, down
    product, weighted sum.  Weights resident in HBM before the timed region."""
    import torch
    import sparse_dual_chunk_amd as S
    from oracle import moe_oracle as M
    from workloads import moe as WM

    w = WM.MOE_DECODE_64.scaled(n_tokens=args.moe_tokens)
    log(f"moe: {w.n_tokens} tokens, {w.n_experts} experts top-{w.top_k}, {w.d_model} x {w.d_ff}; generating")
    w13, w2 = WM.make_weights(w, args.seed)
    x, ids, wts = WM.make_tokens(w, args.seed)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                     else np.ascontiguousarray(a)).cuda()
    X, IDS, WTS = dev(x), dev(ids), dev(wts)
    cfg = S.MoeConfig(n_tokens=w.n_tokens, n_experts=w.n_experts, top_k=w.top_k, d_model=w.d_model, d_ff=w.d_ff)
    # the weights enter HBM once, in the packed layout the layer streams
    U13, U2 = dev(w13), dev(w2)
    W13, W2 = torch.empty_like(U13), torch.empty_like(U2)
    S.moe_pack_weights(U13, U2, cfg, W13, W2)
    torch.cuda.synchronize()
    del U13, U2
    out = torch.empty((w.n_tokens, w.d_model), dtype=torch.int16, device="cuda")
    ws = torch.empty(S.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    hev = HipEvents()
    n_ev = 2 * S.MOE_STAGE_COUNT
    for _ in range(args.warmup):
        S.moe_forward(X, IDS, WTS, W13, W2, cfg, out, ws)
    torch.cuda.synchronize()
    evs = [hev.create(n_ev) for _ in range(args.steps)]
    log(f"timing {args.steps} step(s)")
    t0 = time.perf_counter()
    for st in range(args.steps):
        S.moe_forward(X, IDS, WTS, W13, W2, cfg, out, ws, stage_events=evs[st])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: float(np.median([hev.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs]))
                for i, name in enumerate(S.MOE_STAGES)}
    layer_ms = float(np.median([hev.elapsed_ms(e[0], e[-1]) for e in evs]))
    # the layer captured once in a HIP graph and replayed
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.moe_forward(X, IDS, WTS, W13, W2, cfg, out, ws)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
    active = len(set(int(i) for i in ids.ravel() if 0 <= i < w.n_experts))
    N = int(((ids >= 0) & (ids < w.n_experts)).sum())
    d, dff = w.d_model, w.d_ff
    # algorithmic bytes: each routed expert's weights once, each token row once,
    # activations written and read once, weighted outputs written and read once
    gate_up_bytes = active * 2 * dff * d * 2 + w.n_tokens * d * 2 + N * dff * 2
    down_bytes = active * d * dff * 2 + N * dff * 2 + N * d * 4
    sum_bytes = N * d * 4 + w.n_tokens * d * 2
    layer_bytes = gate_up_bytes + down_bytes + sum_bytes
    achieved = gate_up_bytes / (stage_ms["gate_up"] / 1e3) / 1e9
    result = {
        "metric": MOE_METRIC,
        "value": round(layer_bytes / (layer_ms / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": w.n_tokens, "n_experts": w.n_experts, "top_k": w.top_k,
                   "d_model": d, "d_ff": dff, "routed_experts": active, "seed": args.seed},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": moe_traffic_from_profile(args.moe_tokens),
            "kernel": "moe_mma_kernel<true> (gate/up + SwiGLU)",
            "avg_launch_ms": round(stage_ms["gate_up"], 5),
            "algorithmic_bytes_per_launch": gate_up_bytes,
        },
        "layer_ms": round(layer_ms, 5),
        "graph_ms_per_step": round(graph_ms_per_step, 5),
        "stage_ms": {k2: round(v2, 5) for k2, v2 in stage_ms.items()},
        "down_GBps": round(down_bytes / (stage_ms["down"] / 1e3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        sample = list(range(min(8, w.n_tokens)))
        log(f"cpu baseline: the oracle on tokens {sample[0]}..{sample[-1]}")
        t1 = time.perf_counter()
        M.moe_forward(x, ids, wts, w13, w2, tokens=sample)
        t_s = time.perf_counter() - t1
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count() or 1
        e_s = len(set(int(i) for t in sample for i in ids[t] if 0 <= i < w.n_experts))
        s_bytes = e_s * 3 * d * dff * 2 + len(sample) * d * 2
        result["cpu_baseline"] = {"value": round(s_bytes / t_s / 1e9, 3), "unit": "GB/s", "cores": int(cores),
                                  "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"fp64 oracle on tokens 0..{len(sample) - 1} ({e_s} routed experts, "
                                            f"{t_s:.1f} s): their experts' weight bytes over the time"}
    print(json.dumps(result), flush=True)
    return 0


def moe_traffic_from_profile(n_tokens: int):
    """HBM bytes per gate/up launch from the committed FETCH_SIZE / WRITE_SIZE summary, if it
    was taken on the current kernel source for the same token count (64)."""
    if n_tokens != 64:
        return None
    path = os.path.join(ROOT, "profiles", "moe_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src = os.path.join(ROOT, "sparse_dual_chunk_amd", "csrc", "moe.hip")
        if rec.get("source_sha256_16") != hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]:
            return None
        return rec.get("gate_up_bytes_per_launch")
    except Exception:
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=W.C5_7B_1M.name, choices=sorted(W.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-k", type=int, default=0,
                    help="key-range split of each (block, head) unit (0: the library's heuristic)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (3 launches), "
                         "the reference for scaling the HBM byte counters")
    ap.add_argument("--slash-exact", action="store_true",
                    help="sparse calls with the exact-diagonal semantics instead of the 64-row block cover")
    ap.add_argument("--decode", action="store_true",
                    help="measure the generation-step attention over the 1M-key cache instead of the prefill")
    ap.add_argument("--decode-tokens", type=int, default=1)
    ap.add_argument("--page-keys", type=int, default=0,
                    help="decode over a paged cache with pages of this many keys (0: contiguous cache)")
    ap.add_argument("--moe", action="store_true",
                    help="measure the fused MoE layer (64 experts, top-8, 3584 x 2560) instead of the prefill")
    ap.add_argument("--moe-tokens", type=int, default=64)
    ap.add_argument("--sequence", action="store_true",
                    help="measure the whole-prompt chunked prefill (default prompt: the 14B 256K one), "
                         "fixed 32K chunks against the equal-time schedule, index builds in order or overlapped")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the path is measured on one MI355X; --gpus {args.gpus} "
              "is not supported: the library has no collectives or sharding)", file=sys.stderr)
        return 2

    if args.decode:
        return bench_decode(args)
    if args.sequence:
        return bench_sequence(args)
    if args.moe:
        return bench_moe(args)

    import torch
    import sparse_dual_chunk_amd as S

    w = W.WORKLOADS[args.workload]
    log(f"workload {w.name}: generating inputs (seed {args.seed})")
    kv = W.make_keys_values(w, w.n_k_total, args.seed)
    calls = []
    for c in range(len(w.chunks)):
        inp = W.make(w, c, seed=args.seed, kv=kv)
        cfg = S.config_for(w, c, **({"split_k": args.split_k} if args.split_k else {}),
                           **({"slash_exact": 1} if args.slash_exact else {}))
        calls.append((inp, cfg))
    log("uploading to HBM")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    K = dev(kv[0])
    V = dev(kv[1])
    ws_bytes = max(S.dca_workspace_size(cfg) for _, cfg in calls)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    gpu_calls = []
    for inp, cfg in calls:
        n_k = inp["n_k"]
        q = dev(inp["q"])
        out = torch.empty(q.shape, dtype=torch.int16, device="cuda")
        vi = torch.empty((w.h_q, max(w.k_vertical, 1)), dtype=torch.int32, device="cuda")
        so = torch.empty((w.h_q, max(w.k_slash, 1)), dtype=torch.int32, device="cuda")
        pairs = torch.zeros(1, dtype=torch.int64, device="cuda")
        pos = torch.from_numpy(np.ascontiguousarray(inp["positions"], dtype=np.int32)).cuda()
        gpu_calls.append(dict(q=q, k=K[:n_k], v=V[:n_k], out=out, vi=vi, so=so, pairs=pairs,
                              pos=pos, cfg=cfg))
    torch.cuda.synchronize()

    hev = HipEvents()
    n_stage_ev = 2 * S.DCA_STAGE_COUNT

    def step(stage_events=None, index_events=None, attended=None):
        for ci, g in enumerate(gpu_calls):
            if w.sparse:
                if index_events is not None:
                    index_events[ci][0].record()
                S.vs_index_build(g["q"], g["k"], g["pos"], g["cfg"], g["vi"], g["so"], ws)
                if index_events is not None:
                    index_events[ci][1].record()
            S.dca_sparse_prefill(g["q"], g["k"], g["v"], g["pos"], g["cfg"], g["out"], ws,
                                 v_idx=g["vi"] if w.sparse else None, s_off=g["so"] if w.sparse else None,
                                 cover_pairs=g["pairs"],
                                 stage_events=None if stage_events is None else stage_events[ci],
                                 attended_pairs=None if attended is None else attended[ci])

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stage_ev = [[hev.create(n_stage_ev) for _ in gpu_calls] for _ in range(args.steps)]
    index_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in gpu_calls] for _ in range(args.steps)]
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(stage_ev[s], index_ev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # per-stage times (ms per step, summed over the chunk calls)
    stage_ms = {name: 0.0 for name in S.STAGES}
    attn_launch_ms = []
    index_ms = 0.0
    for s in range(args.steps):
        for ci in range(len(gpu_calls)):
            ev = stage_ev[s][ci]
            for si, name in enumerate(S.STAGES):
                stage_ms[name] += hev.elapsed_ms(ev[2 * si], ev[2 * si + 1]) / args.steps
            attn_launch_ms.append(hev.elapsed_ms(ev[4], ev[5]))
            if w.sparse:
                a, b = index_ev[s][ci]
                index_ms += a.elapsed_time(b) / args.steps

    # cold steps: before each, a 512 MiB write evicts the L2s and the 256 MB
    # Infinity Cache; each step alone is timed with HIP events on the stream
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    hev.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    cold_ms = []
    for s in range(args.steps):
        flush.fill_(s & 0xFF)
        ev = hev.create(2)
        st = torch.cuda.current_stream().cuda_stream
        hev.h.hipEventRecord(ctypes.c_void_p(ev[0]), ctypes.c_void_p(st))
        step()
        hev.h.hipEventRecord(ctypes.c_void_p(ev[1]), ctypes.c_void_p(st))
        torch.cuda.synchronize()
        cold_ms.append(hev.elapsed_ms(ev[0], ev[1]))
    del flush
    cold_ms_step = float(np.median(cold_ms))
    # attended pairs (F_attended / 4d), from one more step outside the timed regions: the
    # exact-diagonal count is a pass of its own
    attended = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in gpu_calls]
    step(attended=attended)
    torch.cuda.synchronize()
    f_attended = 4 * 128 * sum(int(a.item()) for a in attended)

    pairs_per_call = [int(g["pairs"].item()) for g in gpu_calls]
    f_blocks = 4 * 128 * sum(pairs_per_call)
    # headline: the median of cold steps (caches flushed before each); the back-to-back
    # mean is reported beside it
    value = f_blocks / (cold_ms_step / 1e3) / 1e12
    value_warm = f_blocks / (ms_per_step / 1e3) / 1e12
    # dominant kernel: the attention launch; algorithmic flops per launch = 4 d * cover pairs of that call
    attn_avg_ms = float(np.mean(attn_launch_ms))
    f_per_launch = f_blocks / len(gpu_calls)
    achieved = f_per_launch / (attn_avg_ms / 1e3) / 1e12
    traffic = traffic_from_profile(w.name, args.slash_exact)
    dense_pairs = sum(
        sum(min(64, inp["n_q"] - 64 * b) * (inp["p0"] + 64 * b + min(64, inp["n_q"] - 64 * b))
            for b in range((inp["n_q"] + 63) // 64)) * w.h_q for inp, _ in calls)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "prefill_calls": [[p0, nq] for p0, nq in w.chunks],
            "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.head_dim,
            "dca_chunk": w.dca_chunk, "dca_local": w.dca_local, "rope_base": w.rope_base, "yarn_s": w.yarn_s,
            "k_vertical": w.k_vertical, "k_slash": w.k_slash, "seed": args.seed,
            **({"slash_semantics": "exact diagonals"} if args.slash_exact else {}),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            # sparse calls: the stage is two launches, the second serving KV heads with more
            # than 1024 high-norm keys (none in these workloads: its workgroups return at once)
            "kernel": (("dca_attn_exact_kernel + dca_attn_exact_hn_kernel" if args.slash_exact
                        else "dca_attn_kernel + dca_attn_hn_kernel") if w.sparse
                       else ("dca_attn_dense4_kernel" if w.dca_chunk % 128 == 0 and all(p0 % 128 == 0 for p0, _ in w.chunks)
                             else "dca_attn_dense_kernel")),
            "avg_launch_ms": round(attn_avg_ms, 4),
            "algorithmic_flops_per_launch": f_per_launch,
        },
        "f_blocks": f_blocks,
        "f_attended": f_attended,
        "cover_fraction_of_dense": round(sum(pairs_per_call) / dense_pairs, 4),
        "attended_fraction_of_blocks": round(f_attended / f_blocks, 4),
        "stage_ms": {"index_build": round(index_ms, 3), **{k: round(v, 3) for k, v in stage_ms.items()}},
        "attention_tflops": round(achieved, 2),
        "attention_tflops_attended": round(f_attended / len(gpu_calls) / (attn_avg_ms / 1e3) / 1e12, 2),
        "step_tflops_attended": round(f_attended / (cold_ms_step / 1e3) / 1e12, 2),
        "timing": "value and ms_per_step: median of steps each after a 512 MiB write that evicts L2 and "
                  "Infinity Cache, timed alone with HIP events; warm: mean of back-to-back steps",
        "warm": {"ms_per_step": round(ms_per_step, 3), "value": round(value_warm, 2)},
    }
    if w.sparse and not args.slash_exact:
        result["exact_diagonals"] = exact_reading(args, w, calls, gpu_calls, hev, f_blocks)
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w, [c[0] for c in calls], [p0 for p0, _ in w.chunks],
                                              f_blocks, 0)
    print(json.dumps(result), flush=True)
    return 0


def exact_reading(args, w, calls, gpu_calls, hev, f_blocks):
    """The same calls with exact-diagonal slashes, on the index the timed steps built:
    the prefill's stages timed with HIP events over back-to-back calls, and the pairs
    the rows attend (F_attended) next to the computed blocks (F_blocks, unchanged)."""
    import torch
    import sparse_dual_chunk_amd as S
    cfgs = [S.config_for(w, c, **({"split_k": args.split_k} if args.split_k else {}), slash_exact=1)
            for c in range(len(calls))]
    ws = torch.empty(max(S.dca_workspace_size(c) for c in cfgs), dtype=torch.uint8, device="cuda")
    n_stage_ev = 2 * S.DCA_STAGE_COUNT

    def run(stage_events=None, attended=None):
        for ci, g in enumerate(gpu_calls):
            S.dca_sparse_prefill(g["q"], g["k"], g["v"], g["pos"], cfgs[ci], g["out"], ws, v_idx=g["vi"],
                                 s_off=g["so"], stage_events=None if stage_events is None else stage_events[ci],
                                 attended_pairs=None if attended is None else attended[ci])

    log("exact-diagonal slashes on the same index")
    run()
    torch.cuda.synchronize()
    n = max(1, min(args.steps, 3))
    evs = [[hev.create(n_stage_ev) for _ in gpu_calls] for _ in range(n)]
    for s in range(n):
        run(evs[s])
    torch.cuda.synchronize()
    stage_ms = {name: 0.0 for name in S.STAGES}
    attn = []
    for s in range(n):
        for ci in range(len(gpu_calls)):
            ev = evs[s][ci]
            for si, name in enumerate(S.STAGES):
                stage_ms[name] += hev.elapsed_ms(ev[2 * si], ev[2 * si + 1]) / n
            attn.append(hev.elapsed_ms(ev[4], ev[5]))
    attended = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in gpu_calls]
    run(attended=attended)
    torch.cuda.synchronize()
    f_att = 4 * 128 * sum(int(a.item()) for a in attended)
    t_attn = float(np.mean(attn)) * len(gpu_calls) / 1e3   # seconds of attention per step
    del ws
    torch.cuda.empty_cache()
    return {
        "kernel": "dca_attn_exact_kernel + dca_attn_exact_hn_kernel",
        "steps": n,
        "stage_ms": {k: round(v, 3) for k, v in stage_ms.items()},
        "attention_tflops": round(f_blocks / t_attn / 1e12, 2),
        "f_attended": f_att,
        "attended_fraction_of_blocks": round(f_att / f_blocks, 4),
        "attention_tflops_attended": round(f_att / t_attn / 1e12, 2),
    }


if __name__ == "__main__":
    sys.exit(main())
