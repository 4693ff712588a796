"""The allocation-free prefill entry point (static per-GPU scratch) against
dca_sparse_prefill with a caller workspace: two calls in a row, the second
smaller, dense and sparse; outputs and LSE must be bitwise equal (the same
kernels run on the same inputs, only the scratch differs)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_dual_chunk_amd as S  # noqa: E402
from tests.gpu_helpers import dev, host_u16, run_index  # noqa: E402
from workloads import f32_to_bf16_bits  # noqa: E402


def _inputs(seed, p0, n_q, h_q, h_kv):
    rng = np.random.default_rng(seed)
    n_k = p0 + n_q
    q = f32_to_bf16_bits(rng.standard_normal((n_q, h_q, 128)).astype(np.float32))
    kf = rng.standard_normal((n_k, h_kv, 128)).astype(np.float32)
    kf[:4] *= 8
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    return dict(q=q, k=k, v=v, positions=np.arange(p0, n_k, dtype=np.int32), p0=p0, n_q=n_q, n_k=n_k)


def _both(inp, cfg, v_idx=None, s_off=None):
    """(out, lse) of dca_sparse_prefill with a workspace and of dca_sparse_prefill_noalloc."""
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    pos = dev(inp["positions"])
    vi = dev(np.asarray(v_idx, dtype=np.int32)) if v_idx is not None else None
    so = dev(np.asarray(s_off, dtype=np.int32)) if s_off is not None else None
    res = []
    for noalloc in (False, True):
        out = torch.full(q.shape, -1, dtype=torch.int16, device="cuda")
        lse = torch.full((cfg.h_q, cfg.n_q), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            S.dca_sparse_prefill_noalloc(q, k, v, pos, cfg, out, v_idx=vi, s_off=so, lse_out=lse)
        else:
            ws = torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")
            S.dca_sparse_prefill(q, k, v, pos, cfg, out, ws, v_idx=vi, s_off=so, lse_out=lse)
        torch.cuda.synchronize()
        res.append((host_u16(out), lse.cpu().numpy()))
    return res


@pytest.mark.parametrize("sparse", [False, True])
def test_noalloc_matches_workspace_entry_two_calls(sparse):
    # the second call is smaller than the first: it must not depend on what the first left behind
    for seed, p0, n_q in ((11, 512, 300), (12, 128, 100)):
        inp = _inputs(seed, p0, n_q, 4, 2)
        cfg = S.Config(n_q=n_q, n_k=p0 + n_q, h_q=4, h_kv=2, dca_chunk=256, dca_local=64, rope_base=1e6,
                       yarn_s=4.0, vs_last_q=64, vs_k_vertical=40 if sparse else 0,
                       vs_k_slash=6 if sparse else 0, split_k=2 if p0 == 512 else 0)
        v_idx = s_off = None
        if sparse:
            v_idx, s_off = run_index(inp, cfg)
        (o_ws, l_ws), (o_na, l_na) = _both(inp, cfg, v_idx, s_off)
        assert np.array_equal(o_ws, o_na), (seed, sparse)
        assert np.array_equal(l_ws, l_na, equal_nan=False), (seed, sparse)
        assert not np.isnan(l_na).any()
