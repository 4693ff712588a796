"""GPU parity of the generation-step (decode) attention through the C ABI against the fp64 oracle.

The newest n_t tokens (positions n_k - n_t .. n_k - 1) attend the whole key
cache with DCA positions.  Cases span several DCA chunks (all three modes),
tokens on both sides of a chunk boundary, GQA groups of 2 and 7 query heads,
one and two blocks of 32 query columns, sinks and periodic high-norm keys (the
split-precision tiles), explicit and default key-part counts, a cache built by
several appends, and the 7B shape against a million-key cache.
Tolerance as for the prefill: max-abs <= 2e-2, mean-abs <= 2e-3 on the bf16
output; natural-log LSE within 1e-2.
"""
import sys

import numpy as np
import pytest

from oracle import dca_oracle as O
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_dual_chunk_amd as S  # noqa: E402
from tests.gpu_helpers import check_close, dev, host_u16, oracle_cfg  # noqa: E402

LSE_TOL = 1e-2


def log(msg):
    print(f"[decode] {msg}", file=sys.stderr, flush=True)


def _inputs(seed, n_k, n_t, h_q, h_kv, sinks=True, periodic=97):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((n_t, h_q, 128)).astype(np.float32))
    kf = rng.standard_normal((n_k, h_kv, 128)).astype(np.float32)
    if sinks:
        kf[:4] *= 8
    if periodic:
        kf[periodic::periodic] *= 4
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    return q, k, v


def _cfg(n_k, n_t, h_q, h_kv, S_, W, base=1e6, s=4.0, split=0):
    return S.Config(n_q=n_t, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=S_, dca_local=W, rope_base=base, yarn_s=s,
                    split_k=split)


def run_decode(q, k, v, cfg, appends=None, capacity=None):
    """Append the keys (in the given pieces), decode, return (out bits, lse)."""
    n_k = k.shape[0]
    cap = capacity or n_k
    cache = S.KeyCache.allocate(cap, cfg.h_kv)
    kd, vd = dev(k), dev(v)
    if cap > n_k:
        vd = torch.cat([vd, torch.zeros((cap - n_k,) + tuple(vd.shape[1:]), dtype=vd.dtype, device="cuda")])
    cuts = [0] + list(appends or []) + [n_k]
    for a, b in zip(cuts[:-1], cuts[1:]):
        S.dca_key_cache_append(kd[a:b], a, cfg, cache)
    qd = dev(q)
    out = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((cfg.h_q, cfg.n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(S.dca_decode_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    S.dca_decode(qd, cache, vd, cfg, out, ws, lse_out=lse)
    torch.cuda.synchronize()
    return host_u16(out), lse.cpu().numpy()


def _check(q, k, v, cfg, what, **kw):
    out, lse = run_decode(q, k, v, cfg, **kw)
    ref, ref_lse = O.decode_attention(q, k, v, oracle_cfg(cfg))
    check_close(out, ref, what)
    assert np.abs(lse - ref_lse).max() <= LSE_TOL, what
    return out


@pytest.mark.parametrize("n_k,n_t,split", [(700, 1, 0), (700, 3, 0), (700, 3, 5), (64, 1, 0), (33, 2, 0),
                                            (900, 64, 0), (900, 64, 3)])   # 64 tokens: the most one call takes
def test_decode_multichunk(n_k, n_t, split):
    """S = 256: keys in up to three chunks before the tokens' one."""
    q, k, v = _inputs(n_k + n_t, n_k, n_t, 4, 2)
    _check(q, k, v, _cfg(n_k, n_t, 4, 2, 256, 64, split=split), f"n_k {n_k} n_t {n_t} split {split}")


@pytest.mark.parametrize("h_q,h_kv,n_t", [(6, 3, 2), (16, 16, 1), (10, 5, 3)])
def test_decode_head_counts(h_q, h_kv, n_t):
    """KV-head counts that do not divide the 8 dies, and one query head per KV head."""
    n_k = 900
    q, k, v = _inputs(40 + h_kv, n_k, n_t, h_q, h_kv)
    _check(q, k, v, _cfg(n_k, n_t, h_q, h_kv, 256, 64), f"h_q {h_q} h_kv {h_kv}")


def test_decode_tokens_straddle_a_chunk_boundary():
    """Tokens at 510 .. 513 with S = 256: two token chunks, so tiles carry two modes."""
    n_k, n_t = 514, 4
    q, k, v = _inputs(7, n_k, n_t, 4, 2)
    _check(q, k, v, _cfg(n_k, n_t, 4, 2, 256, 64), "straddle")


@pytest.mark.parametrize("n_t", [1, 4, 5])
def test_decode_gqa_seven_heads(n_t):
    """7B grouping (7 query heads per KV head): 7, 28 and 35 columns (two blocks)."""
    n_k = 1500
    q, k, v = _inputs(20 + n_t, n_k, n_t, 28, 4)
    _check(q, k, v, _cfg(n_k, n_t, 28, 4, 512, 128, base=1e7), f"gqa n_t {n_t}")


def test_decode_cache_built_by_appends_is_identical():
    n_k, n_t = 900, 2
    q, k, v = _inputs(30, n_k, n_t, 4, 2)
    cfg = _cfg(n_k, n_t, 4, 2, 256, 64)
    one, _ = run_decode(q, k, v, cfg)
    pieces, _ = run_decode(q, k, v, cfg, appends=[5, 37, 500, 899], capacity=1000)
    assert np.array_equal(one, pieces)


def test_decode_deterministic():
    n_k, n_t = 800, 3
    q, k, v = _inputs(31, n_k, n_t, 4, 2)
    cfg = _cfg(n_k, n_t, 4, 2, 256, 64)
    a, la = run_decode(q, k, v, cfg)
    b, lb = run_decode(q, k, v, cfg)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_t", [1, 4])
def test_decode_7b_million_key_cache(n_t):
    """7B heads (28 / 4), S = 262144, W = 4096, a 1,048,576-key cache with sinks and
    periodic high-norm keys (the benchmark workload's generator); heads 0 and 27
    against the oracle, every head finite and bounded by max |v|."""
    import workloads as W
    w = W.WORKLOADS["7b_last_chunk_of_1m"]
    n_k = w.n_k_total
    log(f"generating a {n_k}-key cache")
    k, v = W.make_keys_values(w, n_k, seed=0)
    q = W.make_queries(w, n_k - n_t, n_t, seed=1)
    cfg = _cfg(n_k, n_t, w.h_q, w.h_kv, w.dca_chunk, w.dca_local, base=w.rope_base, s=w.yarn_s)
    log("GPU decode")
    out, lse = run_decode(q, k, v, cfg)
    heads = [0, w.h_q - 1]
    log(f"oracle heads {heads}")
    ref, ref_lse = O.decode_attention(q, k, v, oracle_cfg(cfg), heads=heads)
    for h in heads:
        check_close(out[:, h], ref[:, h], f"head {h}")
        assert np.abs(lse[h] - ref_lse[h]).max() <= LSE_TOL
    o = (out.astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    vmax = float(np.abs((v.astype(np.uint32) << 16).view(np.float32)).max())
    assert np.abs(o).max() <= vmax * (1 + 2 ** -7)
