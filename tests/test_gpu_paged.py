"""GPU tests of the paged key / value cache (dca_paged_append, dca_decode_paged).

A pool larger than the sequence needs, with the sequence's pages scattered by
a seeded permutation, filled by appends that cross page boundaries.  Checked:
every pool page holds bit for bit, head-major, the rows (rotated K hi / lo, V)
and flag bits of the contiguous cache for its logical page; the paged decode equals
the contiguous decode bit for bit (output and LSE) for pages of 32, 64 and 256
keys, several DCA chunks, GQA groups of 2 and 7 and 1-5 tokens; and one case
against the fp64 oracle.
"""
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


def _inputs(seed, n_k, n_t, h_q, h_kv):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((n_t, h_q, 128)).astype(np.float32))
    kf = rng.standard_normal((n_k, h_kv, 128)).astype(np.float32)
    kf[:4] *= 8
    kf[97::97] *= 4
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    return q, k, v


def _cfg(n_k, n_t, h_q, h_kv, S_=256, W=64):
    return S.Config(n_q=n_t, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=S_, dca_local=W, rope_base=1e6, yarn_s=4.0)


def _build(k, v, cfg, page_keys, seed, cuts):
    n_k, h_kv = k.shape[0], k.shape[1]
    n_table = (n_k + page_keys - 1) // page_keys
    n_pages = n_table + 3
    table = np.random.default_rng(seed).permutation(n_pages)[:n_table].astype(np.int32)
    paged = S.PagedKV.allocate(n_pages, page_keys, h_kv, table)
    flat = S.KeyCache.allocate(n_k, h_kv)
    kd, vd = dev(k), dev(v)
    S.dca_key_cache_append(kd, 0, cfg, flat)
    b = [0] + sorted(c for c in cuts if 0 < c < n_k) + [n_k]
    for a, c in zip(b[:-1], b[1:]):
        S.dca_paged_append(kd[a:c], vd[a:c], a, cfg, paged)
    torch.cuda.synchronize()
    return paged, flat, vd, table


def _decode_both(q, paged, flat, vd, cfg):
    qd = dev(q)
    ws = torch.empty(S.dca_decode_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    outs = []
    for kind in ("paged", "flat"):
        out = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
        lse = torch.empty((cfg.h_q, cfg.n_q), dtype=torch.float32, device="cuda")
        if kind == "paged":
            S.dca_decode_paged(qd, paged, cfg, out, ws, lse_out=lse)
        else:
            S.dca_decode(qd, flat, vd, cfg, out, ws, lse_out=lse)
        torch.cuda.synchronize()
        outs.append((host_u16(out), lse.cpu().numpy()))
    return outs


def test_pool_pages_hold_the_contiguous_rows():
    n_k, h_kv, P = 700, 2, 64
    q, k, v = _inputs(1, n_k, 1, 4, h_kv)
    cfg = _cfg(n_k, 1, 4, h_kv)
    paged, flat, vd, table = _build(k, v, cfg, P, 5, cuts=[3, 64, 100, 511])
    khi, klo = host_u16(flat.k_hi), host_u16(flat.k_lo)
    pk, pl, pv = host_u16(paged.k_hi), host_u16(paged.k_lo), host_u16(paged.v)
    flags = flat.k_flags.cpu().numpy().view(np.uint32)
    pflags = paged.k_flags.cpu().numpy().view(np.uint32)
    for p, pg in enumerate(table):
        a, b = p * P, min(n_k, (p + 1) * P)
        for g in range(h_kv):
            assert np.array_equal(pk[pg, g, : b - a], khi[a:b, g]), (p, g)
            assert np.array_equal(pl[pg, g, : b - a], klo[a:b, g]), (p, g)
            assert np.array_equal(pv[pg, g, : b - a], v[a:b, g]), (p, g)
        for g in range(h_kv):
            for w in range((b - a + 31) // 32):
                want = flags[g, a // 32 + w]
                if b - a < 32 * (w + 1):
                    want &= (1 << ((b - a) % 32)) - 1
                assert pflags[pg, g, w] == want, (p, g, w)
    assert flags.any()


@pytest.mark.parametrize("n_k,n_t,h_q,h_kv,P,S_,W", [(700, 1, 4, 2, 32, 256, 64), (700, 3, 4, 2, 64, 256, 64),
                                                     (1500, 5, 28, 4, 256, 512, 128), (96, 2, 4, 2, 256, 256, 64),
                                                     (1030, 4, 14, 2, 64, 256, 64), (800, 2, 6, 3, 64, 256, 64),
                                                     (500, 1, 16, 16, 32, 256, 64)])
def test_paged_decode_equals_contiguous(n_k, n_t, h_q, h_kv, P, S_, W):
    q, k, v = _inputs(n_k + P, n_k, n_t, h_q, h_kv)
    cfg = _cfg(n_k, n_t, h_q, h_kv, S_, W)
    paged, flat, vd, _ = _build(k, v, cfg, P, n_k, cuts=[P - 1, 2 * P + 5])
    (a, la), (b, lb) = _decode_both(q, paged, flat, vd, cfg)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_paged_decode_against_the_oracle():
    n_k, n_t, h_q, h_kv = 900, 3, 8, 2
    q, k, v = _inputs(44, n_k, n_t, h_q, h_kv)
    cfg = _cfg(n_k, n_t, h_q, h_kv)
    paged, flat, vd, _ = _build(k, v, cfg, 128, 9, cuts=[300])
    (a, la), _ = _decode_both(q, paged, flat, vd, cfg)
    ref, ref_lse = O.decode_attention(q, k, v, oracle_cfg(cfg))
    check_close(a, ref, "paged decode")
    assert np.abs(la - ref_lse).max() <= 1e-2


@pytest.mark.timeout(600)
def test_paged_decode_million_key_cache_equals_contiguous():
    """7B heads, a 1,048,576-key cache of the benchmark's generator in pages of 256 keys
    placed by a seeded permutation: 1 and 4 tokens, paged output and LSE equal the
    contiguous decode bit for bit."""
    import workloads as W
    w = W.WORKLOADS["7b_last_chunk_of_1m"]
    n_k = w.n_k_total
    k, v = W.make_keys_values(w, n_k, seed=0)
    cfg = S.Config(n_q=1, n_k=n_k, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                   rope_base=w.rope_base, yarn_s=w.yarn_s)
    paged, flat, vd, _ = _build(k, v, cfg, 256, 3, cuts=[])
    for n_t in (1, 4):
        q = W.make_queries(w, n_k - n_t, n_t, seed=1)
        c = S.Config(**{**cfg.__dict__, "n_q": n_t})
        (a, la), (b, lb) = _decode_both(q, paged, flat, vd, c)
        assert np.array_equal(a, b) and np.array_equal(la, lb), n_t


# ------------------------------------------------------------------ prefill from the paged pool
def _prefill_both(q, k, p0, paged, flat, vd, cfg, v_idx=None, s_off=None):
    """(out, lse) of dca_sparse_prefill_cached over the contiguous cache and of
    dca_sparse_prefill_paged over the pool, for the chunk [p0, n_k)."""
    qd, pos = dev(q), dev(np.arange(p0, cfg.n_k, dtype=np.int32))
    vi = dev(np.asarray(v_idx, dtype=np.int32)) if v_idx is not None else None
    so = dev(np.asarray(s_off, dtype=np.int32)) if s_off is not None else None
    res = []
    for kind in ("flat", "paged"):
        out = torch.full(qd.shape, -1, dtype=torch.int16, device="cuda")
        lse = torch.empty((cfg.h_q, cfg.n_q), dtype=torch.float32, device="cuda")
        if kind == "flat":
            ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
            S.dca_sparse_prefill_cached(qd, flat, vd, pos, cfg, out, ws, v_idx=vi, s_off=so, lse_out=lse)
        else:
            ws = torch.empty(S.dca_paged_prefill_workspace_size(cfg), dtype=torch.uint8, device="cuda")
            S.dca_sparse_prefill_paged(qd, paged, pos, cfg, out, ws, v_idx=vi, s_off=so, lse_out=lse)
        torch.cuda.synchronize()
        res.append((host_u16(out), lse.cpu().numpy()))
    return res


def _prefill_cfg(n_k, n_q, h_q, h_kv, sparse, split):
    return S.Config(n_q=n_q, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=256, dca_local=64, rope_base=1e6, yarn_s=4.0,
                    vs_last_q=64, vs_k_vertical=24 if sparse else 0, vs_k_slash=40 if sparse else 0, split_k=split)


def _index(q, k, p0, cfg):
    from tests.gpu_helpers import run_index
    inp = dict(q=q, k=k, positions=np.arange(p0, cfg.n_k, dtype=np.int32))
    return run_index(inp, cfg)


@pytest.mark.parametrize("P,sparse,split,h_q,h_kv", [(64, True, 0, 4, 2), (256, True, 2, 4, 2), (32, False, 0, 4, 2),
                                                     (64, False, 3, 14, 2), (128, True, 0, 6, 3)])
def test_paged_prefill_equals_cached(P, sparse, split, h_q, h_kv):
    """The chunk [640, 960) of a prompt whose keys sit in scattered pages (appends that
    cross page boundaries): output and LSE equal the contiguous-cache prefill bit for bit."""
    p0, n_k = 640, 960
    q, k, v = _inputs(P + h_q, n_k, n_k - p0, h_q, h_kv)
    cfg = _prefill_cfg(n_k, n_k - p0, h_q, h_kv, sparse, split)
    paged, flat, vd, _ = _build(k, v, cfg, P, P + 7, cuts=[P - 1, 333, 2 * P + 5, 700])
    vi = so = None
    if sparse:
        vi, so = _index(q, k, p0, cfg)
    (a, la), (b, lb) = _prefill_both(q, k, p0, paged, flat, vd, cfg, vi, so)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_paged_prefill_against_the_oracle():
    p0, n_k, h_q, h_kv = 512, 896, 4, 2
    q, k, v = _inputs(71, n_k, n_k - p0, h_q, h_kv)
    cfg = _prefill_cfg(n_k, n_k - p0, h_q, h_kv, True, 0)
    paged, flat, vd, _ = _build(k, v, cfg, 64, 13, cuts=[200, 640])
    vi, so = _index(q, k, p0, cfg)
    (a, la), _ = _prefill_both(q, k, p0, paged, flat, vd, cfg, vi, so)
    ref, ref_lse = O.attention(q, k, v, p0, oracle_cfg(cfg), v_idx=vi, s_off=so)
    check_close(a, ref, "paged prefill")
    assert np.abs(la - ref_lse).max() <= 1e-2
