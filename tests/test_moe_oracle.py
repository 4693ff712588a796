"""Pins of the fp64 MoE oracle (oracle/moe_oracle.py), no GPU.

- an independent pure-Python loop version on tiny shapes (dropped slots included);
- a single expert with weight 1 is the SwiGLU MLP written with torch's silu and
  matmul in float64;
- diagonal weights give the closed form w gamma silu(alpha x) beta x, which
  tells the gate rows (W1) from the up rows (W3);
- zero routing weights and dropped slots give zero; slots add linearly.
"""
import numpy as np
import pytest

from oracle import moe_oracle as M
from workloads import f32_to_bf16_bits
from workloads import moe as WM


def _tiny(seed, T=4, E=3, k=2, d=8, d_ff=4, drop=True):
    w = WM.MoeWorkload("tiny", T, E, k, d, d_ff)
    x, ids, wts = WM.make_tokens(w, seed)
    w13, w2 = WM.make_weights(w, seed)
    if drop:
        ids = ids.copy()
        ids[1, 0] = -1
        ids[2, 1] = E + 5
    return x, ids, wts, w13, w2


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_equals_plain_loops(seed):
    x, ids, wts, w13, w2 = _tiny(seed)
    a = M.moe_forward(x, ids, wts, w13, w2)
    b = M.moe_forward_loops(x, ids, wts, w13, w2)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_single_expert_is_the_swiglu_mlp():
    torch = pytest.importorskip("torch")
    x, ids, wts, w13, w2 = _tiny(5, T=6, E=1, k=1, d=16, d_ff=8, drop=False)
    wts = np.ones_like(wts)
    got = M.moe_forward(x, ids, wts, w13, w2)
    X = torch.from_numpy(M.bf16_to_f64(x))
    W = torch.from_numpy(M.bf16_to_f64(w13[0]))
    W2 = torch.from_numpy(M.bf16_to_f64(w2[0]))
    ref = (torch.nn.functional.silu(X @ W[:8].T) * (X @ W[8:].T)) @ W2.T
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


def test_diagonal_weights_closed_form():
    d = 8
    alpha, beta, gamma, wt = 0.5, 2.0, 0.25, 0.75
    eye = np.eye(d, dtype=np.float32)
    w13 = f32_to_bf16_bits(np.concatenate([alpha * eye, beta * eye])[None])
    w2 = f32_to_bf16_bits((gamma * eye)[None])
    xv = np.array([[-3.0, -1.0, -0.5, 0.0, 0.25, 1.0, 2.0, 4.0]], dtype=np.float32)
    x = f32_to_bf16_bits(xv)
    got = M.moe_forward(x, np.zeros((1, 1), np.int32), np.full((1, 1), wt, np.float32), w13, w2)
    xd = xv.astype(np.float64)[0]
    ref = wt * gamma * (alpha * xd) / (1 + np.exp(-alpha * xd)) * beta * xd
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-15)
    swapped = wt * gamma * (beta * xd) / (1 + np.exp(-beta * xd)) * alpha * xd
    assert np.abs(got[0] - swapped).max() > 1e-2


def test_zero_weights_and_dropped_slots_give_zero():
    x, ids, wts, w13, w2 = _tiny(3, drop=False)
    assert not M.moe_forward(x, ids, np.zeros_like(wts), w13, w2).any()
    assert not M.moe_forward(x, np.full_like(ids, -1), wts, w13, w2).any()


def test_slots_add_linearly():
    x, ids, wts, w13, w2 = _tiny(4, drop=False)
    whole = M.moe_forward(x, ids, wts, w13, w2)
    parts = 0
    for s in range(ids.shape[1]):
        one = np.full_like(ids, -1)
        one[:, s] = ids[:, s]
        parts = parts + M.moe_forward(x, one, wts, w13, w2)
    np.testing.assert_allclose(whole, parts, rtol=0, atol=1e-13)


def test_token_subset_matches_the_whole():
    x, ids, wts, w13, w2 = _tiny(6, T=7, drop=True)
    whole = M.moe_forward(x, ids, wts, w13, w2)
    sub = M.moe_forward(x, ids, wts, w13, w2, tokens=[5, 1, 2])
    np.testing.assert_allclose(sub, whole[[5, 1, 2]], rtol=0, atol=1e-14)


def test_generator_routing_is_a_top_k_softmax():
    w = WM.MOE_DECODE_64.scaled(n_tokens=33)
    _, ids, wts = WM.make_tokens(w, 0)
    assert ids.shape == (33, 8) and wts.shape == (33, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=1e-6)
    assert (np.diff(wts, axis=1) <= 0).all()      # kept in descending logit order
