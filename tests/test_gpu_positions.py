"""Device positions and the pair counts, through the C ABI.

* positions is a device int32 array checked by the call's first kernel: a call
  whose positions are not p0 + i writes none of its outputs and reports
  DCA_EINVAL in the status word; a good call reports DCA_OK.
* attended_pairs (F_attended / (4 d)) and cover_pairs (F_blocks / (4 d)) against
  the oracle's flop_counts, for dense, block-cover and exact-diagonal calls.
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
from tests.gpu_helpers import dev  # noqa: E402


def _inputs(seed, p0, n_q, h_q, h_kv):
    rng = np.random.default_rng(seed)
    n_k = p0 + n_q
    q = f32_to_bf16_bits(rng.standard_normal((n_q, h_q, 128)).astype(np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    return q, k, v


def _pattern(seed, h_q, n_k, kv, ks):
    rng = np.random.default_rng(seed)
    vi = np.sort(rng.choice(n_k, size=(h_q, kv)), axis=1).astype(np.int32)
    so = np.sort(rng.choice(n_k, size=(h_q, ks)), axis=1).astype(np.int32)
    return vi, so


@pytest.mark.parametrize("which", ["prefill", "cached", "index"])
def test_bad_positions_write_nothing_and_report(which):
    p0, n_q, h_q, h_kv = 128, 200, 4, 2
    n_k = p0 + n_q
    q, k, v = _inputs(1, p0, n_q, h_q, h_kv)
    cfg = S.Config(n_q=n_q, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=128, dca_local=32, rope_base=1e6, yarn_s=4.0,
                   vs_k_vertical=8, vs_k_slash=16)
    vi_h, so_h = _pattern(2, h_q, n_k, 8, 16)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    good = torch.arange(p0, n_k, dtype=torch.int32, device="cuda")
    for bad_at in (0, 77, n_q - 1):
        bad = good.clone()
        bad[bad_at] += 1
        for positions, want in ((bad, S.DCA_EINVAL), (good, S.DCA_OK)):
            status = torch.full((1,), 123, dtype=torch.int32, device="cuda")
            out = torch.full((n_q, h_q, 128), 0x1234, dtype=torch.int16, device="cuda")
            lse = torch.full((h_q, n_q), 7.0, dtype=torch.float32, device="cuda")
            cover = torch.full((1,), -5, dtype=torch.int64, device="cuda")
            att = torch.full((1,), -6, dtype=torch.int64, device="cuda")
            vi = torch.full((h_q, 8), -7, dtype=torch.int32, device="cuda")
            so = torch.full((h_q, 16), -7, dtype=torch.int32, device="cuda")
            if which == "index":
                S.vs_index_build(qd, kd, positions, cfg, vi, so, ws, status=status)
            elif which == "prefill":
                S.dca_sparse_prefill(qd, kd, vd, positions, cfg, out, ws, v_idx=dev(vi_h), s_off=dev(so_h),
                                     lse_out=lse, cover_pairs=cover, attended_pairs=att, status=status)
            else:
                cache = S.KeyCache.allocate(n_k, h_kv)
                S.dca_key_cache_append(kd, 0, cfg, cache)
                S.dca_sparse_prefill_cached(qd, cache, vd, positions, cfg, out, ws, v_idx=dev(vi_h),
                                            s_off=dev(so_h), lse_out=lse, cover_pairs=cover, attended_pairs=att,
                                            status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == want, (which, bad_at, positions is good)
            if which == "index":
                untouched = bool((vi == -7).all()) and bool((so == -7).all())
            else:
                untouched = (bool((out == 0x1234).all()) and bool((lse == 7.0).all())
                             and int(cover.item()) == -5 and int(att.item()) == -6)
            assert untouched == (want == S.DCA_EINVAL), (which, bad_at)


@pytest.mark.parametrize("kind", ["dense", "block", "exact"])
@pytest.mark.parametrize("p0,n_q", [(0, 130), (192, 257)])
def test_pair_counts_match_oracle(kind, p0, n_q):
    h_q, h_kv = 6, 2
    n_k = p0 + n_q
    q, k, v = _inputs(3 + p0, p0, n_q, h_q, h_kv)
    sparse = kind != "dense"
    cfg = S.Config(n_q=n_q, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=128, dca_local=32, rope_base=1e6, yarn_s=4.0,
                   vs_k_vertical=12 if sparse else 0, vs_k_slash=20 if sparse else 0,
                   slash_exact=1 if kind == "exact" else 0)
    vi_h, so_h = _pattern(4 + n_q, h_q, n_k, 12, 20) if sparse else (None, None)
    if sparse:
        so_h[1, :5] = -1              # padding, as per-head budgets leave it
        so_h[1] = np.sort(so_h[1])
    out = torch.empty((n_q, h_q, 128), dtype=torch.int16, device="cuda")
    ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    cover = torch.zeros(1, dtype=torch.int64, device="cuda")
    att = torch.zeros(1, dtype=torch.int64, device="cuda")
    S.dca_sparse_prefill(dev(q), dev(k), dev(v), np.arange(p0, n_k, dtype=np.int32), cfg, out, ws,
                         v_idx=dev(vi_h) if sparse else None, s_off=dev(so_h) if sparse else None,
                         cover_pairs=cover, attended_pairs=att)
    torch.cuda.synchronize()
    fb, fa = O.flop_counts(n_q, h_q, 128, p0, n_k, vi_h, so_h, exact=(kind == "exact"))
    assert 4 * 128 * int(cover.item()) == fb
    assert 4 * 128 * int(att.item()) == fa
