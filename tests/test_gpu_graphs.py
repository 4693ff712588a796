"""HIP-graph capture of the generation-step calls.

A generation loop launches the same few kernels per token, so a serving loop
captures them once and replays the graph.  dca_decode and moe_forward enqueue
only kernels on the caller's stream (no allocation, no memset node, no host
synchronisation), so they can be captured.  Each test captures one call,
then replays it several times with new inputs written in place between the
replays (eager work and a synchronisation in between) and checks every replay
bit for bit against an eager call on the same inputs.
"""
import numpy as np
import pytest

from workloads import f32_to_bf16_bits
from workloads import moe as WM

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_dual_chunk_amd as S  # noqa: E402
from tests.gpu_helpers import dev  # noqa: E402


def _bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_decode_graph_replays_equal_eager_calls():
    n_k, n_t, h_q, h_kv = 1500, 2, 28, 4
    rng = np.random.default_rng(5)
    k, v = _bits(rng, (n_k, h_kv, 128)), _bits(rng, (n_k, h_kv, 128))
    cfg = S.Config(n_q=n_t, n_k=n_k, h_q=h_q, h_kv=h_kv, dca_chunk=512, dca_local=128, rope_base=1e7, yarn_s=4.0)
    cache = S.KeyCache.allocate(n_k, h_kv)
    vd = dev(v)
    S.dca_key_cache_append(dev(k), 0, cfg, cache)
    q_buf = torch.empty((n_t, h_q, 128), dtype=torch.int16, device="cuda")
    out_g = torch.empty_like(q_buf)
    lse_g = torch.empty((h_q, n_t), dtype=torch.float32, device="cuda")
    ws_g = torch.empty(S.dca_decode_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    q_buf.copy_(dev(_bits(rng, (n_t, h_q, 128))))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.dca_decode(q_buf, cache, vd, cfg, out_g, ws_g, lse_out=lse_g)
    out_e = torch.empty_like(q_buf)
    lse_e = torch.empty_like(lse_g)
    ws_e = torch.empty_like(ws_g)
    for r in range(4):
        q_buf.copy_(dev(_bits(rng, (n_t, h_q, 128))))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        S.dca_decode(q_buf, cache, vd, cfg, out_e, ws_e, lse_out=lse_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {r}"


def test_moe_graph_replays_equal_eager_calls():
    w = WM.MoeWorkload("t", 16, 16, 4, 256, 256)
    w13, w2 = WM.make_weights(w, 3)
    cfg = S.MoeConfig(n_tokens=w.n_tokens, n_experts=w.n_experts, top_k=w.top_k, d_model=w.d_model, d_ff=w.d_ff)
    a, b = dev(w13), dev(w2)
    pa, pb = torch.empty_like(a), torch.empty_like(b)
    S.moe_pack_weights(a, b, cfg, pa, pb)
    x_buf = torch.empty((w.n_tokens, w.d_model), dtype=torch.int16, device="cuda")
    ids_buf = torch.empty((w.n_tokens, w.top_k), dtype=torch.int32, device="cuda")
    wts_buf = torch.empty((w.n_tokens, w.top_k), dtype=torch.float32, device="cuda")

    def fill(seed):
        x, ids, wts = WM.make_tokens(w.scaled(skew=float(seed % 3)), seed)
        x_buf.copy_(dev(x))
        ids_buf.copy_(torch.from_numpy(ids))
        wts_buf.copy_(torch.from_numpy(wts))

    out_g = torch.empty_like(x_buf)
    ws_g = torch.empty(S.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    fill(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.moe_forward(x_buf, ids_buf, wts_buf, pa, pb, cfg, out_g, ws_g)
    out_e = torch.empty_like(x_buf)
    ws_e = torch.empty_like(ws_g)
    for r in range(4):
        fill(r + 1)                    # new tokens and a new routing (other experts) in place
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        S.moe_forward(x_buf, ids_buf, wts_buf, pa, pb, cfg, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}"
