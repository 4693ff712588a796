"""CPU fp64 oracle of the fused MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module; the GPU library never
calls it and shares no code with it.

Source: xllm-io paper-review page, section 4 "Inference & deployment", "MoE
kernel optimisation" (Figure 8) for the layer, section 3 (model table) for the
SwiGLU feed-forward.  Per token t and routed slot s with expert e and weight w:
    g = W1_e x_t, u = W3_e x_t, a = silu(g) * u, y = W2_e a, out_t += w * y
with silu(z) = z / (1 + exp(-z)); slots whose expert id is outside
[0, n_experts) contribute nothing.  Readings where the pages are silent: the
router's ids and weights are inputs; W1 and W3 are stacked as one
[2 d_ff][d_model] matrix per expert (gate rows first).  Everything is float64
here, without the GPU's bf16 rounding of the activations.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def moe_forward(x, topk_ids, topk_weights, w13, w2, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 output [len(tokens)][d_model] for the given tokens (default: all).

    The tokens routed to one expert are taken together so that each expert's
    weights are converted once; each token's slots are then summed in slot order.
    """
    T, k = topk_ids.shape
    E = w13.shape[0]
    d_ff = w13.shape[1] // 2
    toks = list(range(T)) if tokens is None else list(tokens)
    X = bf16_to_f64(x[toks])
    ys = {}
    for e in sorted({int(i) for t in toks for i in topk_ids[t] if 0 <= int(i) < E}):
        pairs = [(r, s) for r, t in enumerate(toks) for s in range(k) if int(topk_ids[t, s]) == e]
        W13 = bf16_to_f64(w13[e])
        W2 = bf16_to_f64(w2[e])
        Xe = X[[r for r, _ in pairs]]
        g = Xe @ W13[:d_ff].T
        u = Xe @ W13[d_ff:].T
        y = (silu(g) * u) @ W2.T
        for (r, s), row in zip(pairs, y):
            ys[(r, s)] = row
    out = np.zeros((len(toks), w13.shape[2]), dtype=np.float64)
    for r, t in enumerate(toks):
        for s in range(k):
            if (r, s) in ys:
                out[r] += float(topk_weights[t, s]) * ys[(r, s)]
    return out


def moe_forward_loops(x, topk_ids, topk_weights, w13, w2) -> np.ndarray:
    """The same layer as plain Python loops with math.exp, for tiny shapes."""
    import math
    T, k = topk_ids.shape
    E, two_ff, d = w13.shape
    d_ff = two_ff // 2
    X = bf16_to_f64(x)
    A = bf16_to_f64(w13)
    B = bf16_to_f64(w2)
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for s in range(k):
            e = int(topk_ids[t, s])
            if not 0 <= e < E:
                continue
            act = []
            for r in range(d_ff):
                g = sum(A[e, r, c] * X[t, c] for c in range(d))
                u = sum(A[e, d_ff + r, c] * X[t, c] for c in range(d))
                act.append(g / (1.0 + math.exp(-g)) * u)
            for c in range(d):
                y = sum(B[e, c, r] * act[r] for r in range(d_ff))
                out[t][c] += float(topk_weights[t, s]) * y
    return np.array(out)
