"""Parity at the full sizes of the benchmark workloads, in the launch configuration
bench.py times (default split, default high-norm threshold).

The oracle cannot finish a whole call at these sizes, so each check uses outputs the
oracle computes one by one:
  * the vertical-slash index of sampled query heads, bit-exact;
  * the exact F_blocks cover count of every head from the GPU's own index;
  * the attention rows of sampled (head, query block) pairs (blocks 0, 1, middle,
    last and two seeded random ones), within the bf16 output tolerance, plus lse
    (for the 128K chunk also with the exact-diagonal semantics);
  * properties that hold at any size on all rows (finite outputs, |o| <= max |v|).
"""
from __future__ import annotations

import gc
import sys

import numpy as np
import pytest

import workloads as W
from oracle import dca_oracle as O

from gpu_helpers import MAX_ABS, MEAN_ABS, bf16_f64, oracle_cfg

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-2
CASES = [
    ("7b_dense_32k", 0, 0),
    ("7b_chunk_at_98304_of_128k", 0, 0),
    ("7b_chunk_at_98304_of_128k", 0, 1),
    ("14b_256k_in_8_chunks", 7, 0),
    ("7b_last_chunk_of_1m", 0, 0),
]
_cache: dict = {}


def log(msg: str) -> None:
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


def gpu_call(name: str, chunk: int, exact: int = 0) -> dict:
    """Run index build + prefill of one call on the GPU once per (workload, chunk, semantics)."""
    key = (name, chunk, exact)
    if key in _cache:
        return _cache[key]
    _cache.clear()
    gc.collect()
    import torch
    import sparse_dual_chunk_amd as S
    from gpu_helpers import dev, host_u16
    w = W.WORKLOADS[name]
    log(f"{name} chunk {chunk}: generating inputs")
    inp = W.make(w, chunk, seed=0)
    cfg = S.config_for(w, chunk, slash_exact=exact)
    log(f"{name} chunk {chunk}: GPU index + prefill (n_q {cfg.n_q}, n_k {cfg.n_k})")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    out = torch.empty(q.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((cfg.h_q, cfg.n_q), dtype=torch.float32, device="cuda")
    pairs = torch.zeros(1, dtype=torch.int64, device="cuda")
    vi = so = None
    if w.sparse:
        vi = torch.empty((w.h_q, w.k_vertical), dtype=torch.int32, device="cuda")
        so = torch.empty((w.h_q, w.k_slash), dtype=torch.int32, device="cuda")
        S.vs_index_build(q, k, inp["positions"], cfg, vi, so, ws)
    S.dca_sparse_prefill(q, k, v, inp["positions"], cfg, out, ws, v_idx=vi, s_off=so, lse_out=lse,
                         cover_pairs=pairs)
    torch.cuda.synchronize()
    res = dict(w=w, inp=inp, cfg=cfg, exact=bool(exact), out=host_u16(out), lse=lse.cpu().numpy(), pairs=int(pairs.item()),
               v_idx=None if vi is None else vi.cpu().numpy(), s_off=None if so is None else so.cpu().numpy())
    del q, k, v, ws, out, lse, pairs, vi, so
    torch.cuda.empty_cache()
    _cache[key] = res
    return res


def sampled_heads(h_q: int):
    return [0, h_q - 1]


def check_index(r):
    heads = sampled_heads(r["w"].h_q)
    log(f"oracle index of heads {heads}")
    v_ref, s_ref, _ = O.vs_index(r["inp"]["q"], r["inp"]["k"], r["inp"]["p0"], oracle_cfg(r["cfg"]), heads=heads)
    for h in heads:
        assert np.array_equal(r["v_idx"][h], v_ref[h]), f"vertical index of head {h} differs"
        assert np.array_equal(r["s_off"][h], s_ref[h]), f"slash index of head {h} differs"


def check_cover_pairs(r):
    cfg = r["cfg"]
    log("oracle cover counts of every head")
    fb, _ = O.flop_counts(cfg.n_q, cfg.h_q, 128, r["inp"]["p0"], cfg.n_k, r["v_idx"], r["s_off"])
    assert 4 * 128 * r["pairs"] == fb, f"F_blocks {4 * 128 * r['pairs']} != oracle {fb}"


def check_sampled_blocks(r):
    w, inp, cfg = r["w"], r["inp"], r["cfg"]
    heads = sampled_heads(w.h_q)
    pairs = [(h, b) for (h, b) in W.sample_blocks(cfg.n_q, w.h_q, seed=0) if h in heads]
    log(f"oracle attention of {len(pairs)} (head, block) pairs")
    ocfg = oracle_cfg(cfg)
    worst, tot, cnt = 0.0, 0.0, 0
    for h, b in pairs:
        ref, lse_ref, _ = O.attention_block(inp["q"], inp["k"], inp["v"], inp["p0"], h, b, ocfg,
                                            r["v_idx"], r["s_off"], exact=r["exact"])
        r0 = 64 * b
        got = bf16_f64(r["out"][r0:r0 + ref.shape[0], h])
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        tot += float(err.sum())
        cnt += err.size
        lse_got = r["lse"][h, r0:r0 + ref.shape[0]].astype(np.float64)
        assert np.max(np.abs(lse_got - lse_ref)) <= LSE_TOL, f"lse of head {h} block {b}"
    assert worst <= MAX_ABS, f"max abs error {worst:.3e}"
    assert tot / cnt <= MEAN_ABS, f"mean abs error {tot / cnt:.3e}"


def check_all_rows_bounded(r):
    """Every output is finite and no larger than the largest |v| of its KV head (a convex
    combination, up to bf16 rounding); every lse is finite (no row is empty)."""
    w, inp = r["w"], r["inp"]
    G = w.h_q // w.h_kv
    for g in range(w.h_kv):
        vmax_bits = int((inp["v"][:, g] & np.uint16(0x7FFF)).max())      # |x| orders like its bits
        vmax = float(bf16_f64(np.array([vmax_bits], dtype=np.uint16))[0])
        for h in range(g * G, (g + 1) * G):
            o = bf16_f64(r["out"][:, h])
            assert np.all(np.isfinite(o)), f"non-finite output in head {h}"
            assert np.abs(o).max() <= vmax * (1 + 2 ** -7), f"head {h} exceeds max |v|"
    assert np.all(np.isfinite(r["lse"]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk,exact", CASES)
def test_fullsize(name, chunk, exact):
    r = gpu_call(name, chunk, exact)
    if r["w"].sparse:
        check_index(r)
    check_cover_pairs(r)
    check_sampled_blocks(r)
    check_all_rows_bounded(r)
