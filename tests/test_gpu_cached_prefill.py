"""GPU tests of the prefill fed from a rotated key cache (dca_sparse_prefill_cached).

A chunked prefill appends each chunk's keys to the cache and runs the chunk's
attention from it, so every key is rotated once.  With the same keys the
cached prefill must equal dca_sparse_prefill bit for bit (the same rotated
keys, flags and kernels), chunk after chunk; the last chunk is also checked
against the oracle, and a generation step then runs on the same cache.
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


def _seq(seed, n, h_q, h_kv):
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


def _index(q, k, pos, cfg, ws):
    vi = torch.empty((cfg.h_q, cfg.vs_k_vertical), dtype=torch.int32, device="cuda")
    so = torch.empty((cfg.h_q, cfg.vs_k_slash), dtype=torch.int32, device="cuda")
    S.vs_index_build(q, k, pos, cfg, vi, so, ws)
    return vi, so


@pytest.mark.parametrize("sparse,split", [(False, 0), (True, 0), (True, 3)])
def test_chunked_prefill_from_cache_equals_uncached(sparse, split):
    h_q, h_kv, n = 4, 2, 960
    chunks = [(0, 320), (320, 384), (704, 256)]          # p0 multiples of 64, ragged last chunk
    q, k, v = _seq(5 + split, n, h_q, h_kv)
    kd, vd = dev(k), dev(v)
    cache = S.KeyCache.allocate(n, h_kv)
    kw = dict(vs_k_vertical=24, vs_k_slash=40) if sparse else {}
    for p0, n_q in chunks:
        n_k = p0 + n_q
        cfg = _cfg(n_q, n_k, h_q, h_kv, split_k=split, **kw)
        pos = np.arange(p0, n_k, dtype=np.int32)
        ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
        qd = dev(q[p0:n_k])
        S.dca_key_cache_append(kd[p0:n_k], p0, cfg, cache)
        vi = so = None
        if sparse:
            vi, so = _index(qd, kd[:n_k], pos, cfg, ws)
        a = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
        b = torch.empty(qd.shape, dtype=torch.int16, device="cuda")
        la = torch.empty((h_q, n_q), dtype=torch.float32, device="cuda")
        lb = torch.empty((h_q, n_q), dtype=torch.float32, device="cuda")
        S.dca_sparse_prefill_cached(qd, cache, vd[:n_k], pos, cfg, a, ws, v_idx=vi, s_off=so, lse_out=la)
        S.dca_sparse_prefill(qd, kd[:n_k], vd[:n_k], pos, cfg, b, ws, v_idx=vi, s_off=so, lse_out=lb)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb), f"chunk at {p0}"
    # the last chunk against the oracle
    p0, n_q = chunks[-1]
    ocfg = oracle_cfg(cfg)
    if sparse:
        v_ref, s_ref, _ = O.vs_index(q[p0:], k, p0, ocfg)
        assert np.array_equal(vi.cpu().numpy(), v_ref) and np.array_equal(so.cpu().numpy(), s_ref)
        ref, _ = O.attention(q[p0:], k, v, p0, ocfg, v_idx=v_ref, s_off=s_ref)
    else:
        ref, _ = O.attention(q[p0:], k, v, p0, ocfg)
    check_close(host_u16(a), ref, "last chunk")


def test_generation_after_a_cached_prefill():
    """Prefill 2 chunks through the cache, append 3 generated tokens' keys, decode them."""
    h_q, h_kv = 8, 2
    q, k, v = _seq(9, 515, h_q, h_kv)
    kd, vd = dev(k), dev(v)
    cache = S.KeyCache.allocate(600, h_kv)
    vpad = torch.cat([vd, torch.zeros((85, h_kv, 128), dtype=vd.dtype, device="cuda")])
    for p0, n_q in [(0, 256), (256, 256)]:
        cfg = _cfg(n_q, p0 + n_q, h_q, h_kv)
        ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
        S.dca_key_cache_append(kd[p0:p0 + n_q], p0, cfg, cache)
        out = torch.empty((n_q, h_q, 128), dtype=torch.int16, device="cuda")
        S.dca_sparse_prefill_cached(dev(q[p0:p0 + n_q]), cache, vpad, np.arange(p0, p0 + n_q, dtype=np.int32), cfg,
                                    out, ws)
    dcfg = _cfg(3, 515, h_q, h_kv)
    S.dca_key_cache_append(kd[512:515], 512, dcfg, cache)
    out = torch.empty((3, h_q, 128), dtype=torch.int16, device="cuda")
    ws = torch.empty(S.dca_decode_workspace_size(dcfg), dtype=torch.uint8, device="cuda")
    S.dca_decode(dev(q[512:515]), cache, vpad, dcfg, out, ws)
    torch.cuda.synchronize()
    ref, _ = O.decode_attention(q[512:515], k, v, oracle_cfg(dcfg))
    check_close(host_u16(out), ref, "decode after cached prefill")
