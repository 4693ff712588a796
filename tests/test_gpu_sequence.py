"""GPU tests of the whole-prompt chunked prefill (dca_prefill_sequence).

The driver runs, chunk after chunk, the key append, the chunk's index build
(on a second stream one chunk ahead, or in order on one stream) and the
attention from the rotated key cache.  It must equal the same per-chunk calls
made one by one bit for bit (outputs, LSE columns, cover pairs), with and
without the second stream, sparse and dense, with a chunk small enough to run
dense inside a sparse prompt, and over bounds from the equal-time schedule;
the whole output is also checked against the oracle chunk by chunk (its own
index, then its attention).
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


def log(msg):
    print(f"[sequence] {msg}", file=sys.stderr, flush=True)


def _prompt(seed, n, h_q, h_kv):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((n, h_q, 128)).astype(np.float32))
    kf = rng.standard_normal((n, h_kv, 128)).astype(np.float32)
    kf[:4] *= 8
    kf[97::97] *= 4
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(rng.standard_normal((n, h_kv, 128)).astype(np.float32))
    return q, k, v


def _cfg(n_q, n_k, h_q, h_kv, **kw):
    return S.Config(n_q=n_q, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=256, dca_local=64, rope_base=1e6, yarn_s=4.0,
                    **kw)


def _per_chunk(qd, kd, vd, bounds, cfg, sparse):
    """The same chunked prefill made of individual calls on one stream."""
    n, h_q = cfg.n_k, cfg.h_q
    cache = S.KeyCache.allocate(n, cfg.h_kv)
    out = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((h_q, n), dtype=torch.float32, device="cuda")
    pairs = torch.zeros(len(bounds) - 1, dtype=torch.int64, device="cuda")
    for c, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        cc = S.Config(**{**cfg.__dict__, "n_q": b - a, "n_k": b})
        ws = torch.empty(S.dca_workspace_size(cc), dtype=torch.uint8, device="cuda")
        pos = np.arange(a, b, dtype=np.int32)
        vi = so = None
        if sparse and b > cfg.vs_k_slash:
            vi = torch.empty((h_q, cfg.vs_k_vertical), dtype=torch.int32, device="cuda")
            so = torch.empty((h_q, cfg.vs_k_slash), dtype=torch.int32, device="cuda")
            S.vs_index_build(qd[a:b], kd[:b], pos, cc, vi, so, ws)
        S.dca_key_cache_append(kd[a:b], a, cc, cache)
        lc = torch.empty((h_q, b - a), dtype=torch.float32, device="cuda")
        S.dca_sparse_prefill_cached(qd[a:b], cache, vd, pos, cc, out[a:b], ws, v_idx=vi, s_off=so, lse_out=lc,
                                    cover_pairs=pairs[c:c + 1])
        lse[:, a:b] = lc
    torch.cuda.synchronize()
    return out, lse, pairs


def _sequence(qd, kd, vd, bounds, cfg, sparse, overlap):
    n, h_q = cfg.n_k, cfg.h_q
    cache = S.KeyCache.allocate(n, cfg.h_kv)
    out = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((h_q, n), dtype=torch.float32, device="cuda")
    pairs = torch.zeros(len(bounds) - 1, dtype=torch.int64, device="cuda")
    ws = torch.empty(S.dca_prefill_sequence_workspace_size(cfg, bounds, sparse, overlap), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream() if overlap else None
    S.dca_prefill_sequence(qd, kd, vd, bounds, cfg, cache, out, ws, sparse=sparse,
                           index_stream=side.cuda_stream if side is not None else None, lse_out=lse,
                           cover_pairs=pairs)
    torch.cuda.synchronize()
    return out, lse, pairs


def _sequence_paged(qd, kd, vd, bounds, cfg, sparse, overlap, page_keys=64, seed=0):
    """The driver over a paged pool: pages of page_keys keys placed by a seeded permutation."""
    n, h_q = cfg.n_k, cfg.h_q
    n_table = (n + page_keys - 1) // page_keys
    table = np.random.default_rng(seed).permutation(n_table + 2)[:n_table].astype(np.int32)
    pool = S.PagedKV.allocate(n_table + 2, page_keys, cfg.h_kv, table)
    out = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((h_q, n), dtype=torch.float32, device="cuda")
    pairs = torch.zeros(len(bounds) - 1, dtype=torch.int64, device="cuda")
    ws = torch.empty(S.dca_prefill_sequence_paged_workspace_size(cfg, bounds, sparse, overlap), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream() if overlap else None
    S.dca_prefill_sequence_paged(qd, kd, vd, bounds, cfg, pool, out, ws, sparse=sparse,
                                 index_stream=side.cuda_stream if side is not None else None, lse_out=lse,
                                 cover_pairs=pairs)
    torch.cuda.synchronize()
    return out, lse, pairs


CASES = [
    # (n, bounds, sparse, k_v, k_s)
    (960, [0, 320, 704, 960], True, 24, 40),
    (960, [0, 320, 704, 960], False, 0, 0),
    (1000, [0, 256, 512, 768, 1000], True, 16, 300),   # the first chunk (256 keys <= 300) runs dense
    (1000, [0, 1000], True, 16, 64),                   # one chunk
]


@pytest.mark.parametrize("n,bounds,sparse,kv,ks", CASES)
@pytest.mark.parametrize("overlap", [False, True])
def test_sequence_equals_per_chunk_calls(n, bounds, sparse, kv, ks, overlap):
    h_q, h_kv = 4, 2
    log(f"n {n} bounds {bounds} sparse {sparse} overlap {overlap}")
    q, k, v = _prompt(n + ks, n, h_q, h_kv)
    qd, kd, vd = dev(q), dev(k), dev(v)
    cfg = _cfg(n, n, h_q, h_kv, vs_k_vertical=kv, vs_k_slash=ks)
    a, la, pa = _sequence(qd, kd, vd, bounds, cfg, sparse, overlap)
    b, lb, pb = _per_chunk(qd, kd, vd, bounds, cfg, sparse)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(pa, pb)


@pytest.mark.parametrize("n,bounds,sparse,kv,ks", CASES)
def test_paged_driver_equals_the_contiguous_driver(n, bounds, sparse, kv, ks):
    """The driver over scattered pages of 64 keys equals the contiguous-cache driver bit for bit."""
    h_q, h_kv = 4, 2
    q, k, v = _prompt(n + ks + 1, n, h_q, h_kv)
    qd, kd, vd = dev(q), dev(k), dev(v)
    cfg = _cfg(n, n, h_q, h_kv, vs_k_vertical=kv, vs_k_slash=ks)
    a, la, pa = _sequence_paged(qd, kd, vd, bounds, cfg, sparse, overlap=True, seed=n)
    b, lb, pb = _sequence(qd, kd, vd, bounds, cfg, sparse, overlap=True)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(pa, pb)


@pytest.mark.parametrize("sparse", [True, False])
def test_sequence_against_the_oracle(sparse):
    h_q, h_kv, n = 4, 2, 960
    bounds = [0, 320, 704, 960]
    q, k, v = _prompt(77, n, h_q, h_kv)
    cfg = _cfg(n, n, h_q, h_kv, vs_k_vertical=24 if sparse else 0, vs_k_slash=40 if sparse else 0)
    out, lse, _ = _sequence(dev(q), dev(k), dev(v), bounds, cfg, sparse, overlap=True)
    got = host_u16(out)
    got_lse = lse.cpu().numpy()
    for a, b in zip(bounds[:-1], bounds[1:]):
        ocfg = oracle_cfg(S.Config(**{**cfg.__dict__, "n_q": b - a, "n_k": b}))
        if sparse:
            v_ref, s_ref, _ = O.vs_index(q[a:b], k[:b], a, ocfg)
            ref, ref_lse = O.attention(q[a:b], k[:b], v[:b], a, ocfg, v_idx=v_ref, s_off=s_ref)
        else:
            ref, ref_lse = O.attention(q[a:b], k[:b], v[:b], a, ocfg)
        check_close(got[a:b], ref, f"chunk {a}..{b}")
        assert np.abs(got_lse[:, a:b] - ref_lse).max() <= 1e-2


def test_sequence_over_the_equal_time_schedule():
    """Bounds from dca_chunk_schedule (the library's own cost coefficients) feed the driver."""
    h_q, h_kv, n = 8, 2, 2496
    cfg = _cfg(n, n, h_q, h_kv, vs_k_vertical=32, vs_k_slash=96)
    bounds, _ = S.dca_chunk_schedule(n, 5, n, S.dca_chunk_cost_default(cfg, True))
    log(f"schedule {bounds}")
    assert len(bounds) == 6
    q, k, v = _prompt(3, n, h_q, h_kv)
    qd, kd, vd = dev(q), dev(k), dev(v)
    a, la, pa = _sequence(qd, kd, vd, bounds, cfg, True, overlap=True)
    b, lb, pb = _per_chunk(qd, kd, vd, bounds, cfg, True)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(pa, pb)


@pytest.mark.timeout(900)
def test_sequence_14b_256k_prompt_equals_per_chunk_calls():
    """The 14B prompt of 262,144 tokens (40 / 8 heads, S = 65536, W = 2048, k_v 2048,
    k_s 8192) in the eight 32K chunks of the benchmark and in the equal-time chunks of the
    library's cost model: the driver with the index stream equals the per-chunk calls bit
    for bit, and every output is finite and bounded by max |v|."""
    import workloads as W
    w = W.C4_14B_256K
    n = w.n_k_total
    log("generating the 256K prompt")
    k, v = W.make_keys_values(w, n, seed=0)
    fixed = list(range(0, n, 32768)) + [n]
    q = np.concatenate([W.make_queries(w, a, b - a, seed=0) for a, b in zip(fixed[:-1], fixed[1:])])
    qd, kd, vd = dev(q), dev(k), dev(v)
    cfg = S.Config(n_q=n, n_k=n, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                   rope_base=w.rope_base, yarn_s=w.yarn_s, vs_k_vertical=w.k_vertical, vs_k_slash=w.k_slash)
    equal, _ = S.dca_chunk_schedule(n, 8, n, S.dca_chunk_cost_default(cfg, True))
    vmax = float(np.abs((v.astype(np.uint32) << 16).view(np.float32)).max())
    for bounds in (fixed, equal):
        log(f"bounds {bounds}")
        a, la, pa = _sequence(qd, kd, vd, bounds, cfg, True, overlap=True)
        b, lb, pb = _per_chunk(qd, kd, vd, bounds, cfg, True)
        assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(pa, pb)
        o = (host_u16(a).astype(np.uint32) << 16).view(np.float32)
        assert np.isfinite(o).all() and np.abs(o).max() <= vmax * (1 + 2 ** -7)
        del a, b, la, lb
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_sequence_14b_256k_prompt_through_the_paged_driver():
    """The 14B prompt of 262,144 tokens in the benchmark's eight 32K chunks, its keys and
    values appended into scattered pages of 256 keys: the paged driver equals the
    contiguous-cache driver bit for bit."""
    import workloads as W
    w = W.C4_14B_256K
    n = w.n_k_total
    log("generating the 256K prompt")
    k, v = W.make_keys_values(w, n, seed=0)
    fixed = list(range(0, n, 32768)) + [n]
    q = np.concatenate([W.make_queries(w, a, b - a, seed=0) for a, b in zip(fixed[:-1], fixed[1:])])
    qd, kd, vd = dev(q), dev(k), dev(v)
    cfg = S.Config(n_q=n, n_k=n, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                   rope_base=w.rope_base, yarn_s=w.yarn_s, vs_k_vertical=w.k_vertical, vs_k_slash=w.k_slash)
    log("paged driver")
    a, la, pa = _sequence_paged(qd, kd, vd, fixed, cfg, True, overlap=True, page_keys=256, seed=5)
    log("contiguous driver")
    b, lb, pb = _sequence(qd, kd, vd, fixed, cfg, True, overlap=True)
    assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(pa, pb)
