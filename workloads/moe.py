"""Seeded synthetic inputs of the fused MoE layer (the memory-bound MoE kernel
of the xllm-io paper-review page, section 4, "MoE kernel optimisation").

Shapes and the generator only; nothing of the layer's arithmetic.  The pages
give no MoE shape (the MoE model they name is reachable only through an API),
so the workloads take the 7B model's hidden size (28 heads x 128 = 3584, from
the page's model table) with 64 experts of intermediate size 2560 and 8
experts per token, at generation batch sizes.  Values: activations standard
normal, rounded to bfloat16.  Weights are drawn directly as bfloat16 bit
patterns from random bytes (gigabytes of them are needed): a random sign, a
random 7-bit mantissa and a binary exponent uniform in -9 .. -6, so the
magnitudes lie in [2^-9, 2^-5) with an RMS of about 0.014, near
1/sqrt(fan-in).  Routing: each token draws standard normal router
logits, keeps its top_k experts and weights them by the softmax of the kept
logits; ``skew`` adds a Zipf-like popularity bias (log 1/(e+1)^skew) so that
some experts get many slots and some none.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import _normal_bf16

WEIGHT_EXP_FIELD = 118       # bfloat16 exponent field of 2^-9; plus 0..3


@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    name: str
    n_tokens: int
    n_experts: int
    top_k: int
    d_model: int
    d_ff: int
    skew: float = 0.0

    def scaled(self, **kw) -> "MoeWorkload":
        return dataclasses.replace(self, **kw)


MOE_DECODE_64 = MoeWorkload("moe_64x2560_top8_d3584_64_tokens", 64, 64, 8, 3584, 2560)
MOE_DECODE_1 = MOE_DECODE_64.scaled(name="moe_64x2560_top8_d3584_1_token", n_tokens=1)
MOE_DECODE_256 = MOE_DECODE_64.scaled(name="moe_64x2560_top8_d3584_256_tokens", n_tokens=256)
MOE_WORKLOADS = {w.name: w for w in (MOE_DECODE_1, MOE_DECODE_64, MOE_DECODE_256)}


def _random_weights(seed_seq, shape) -> np.ndarray:
    rng = np.random.default_rng(seed_seq)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 26
    for a in range(0, n, step):
        b = min(n, a + step)
        r = np.frombuffer(rng.bytes(2 * (b - a)), dtype=np.uint16)
        # sign and mantissa kept, exponent field 118 + (2 random bits)
        out[a:b] = (r & np.uint16(0x807F)) | ((np.uint16(WEIGHT_EXP_FIELD) + ((r >> np.uint16(7)) & np.uint16(3)))
                                             << np.uint16(7))
    return out.reshape(shape)


def make_weights(w: MoeWorkload, seed: int = 0):
    """w13 [E][2 d_ff][d_model] (gate rows, then up rows) and w2 [E][d_model][d_ff], bf16 bits."""
    w13 = _random_weights([seed, 11], (w.n_experts, 2 * w.d_ff, w.d_model))
    w2 = _random_weights([seed, 12], (w.n_experts, w.d_model, w.d_ff))
    return w13, w2


def make_tokens(w: MoeWorkload, seed: int = 0):
    """x [T][d_model] bf16 bits, topk_ids [T][top_k] int32, topk_weights [T][top_k] float32."""
    x = _normal_bf16([seed, 13], (w.n_tokens, w.d_model))
    rng = np.random.default_rng([seed, 14])
    logits = rng.standard_normal((w.n_tokens, w.n_experts))
    if w.skew:
        logits = logits - w.skew * np.log(np.arange(1, w.n_experts + 1, dtype=np.float64))
    ids = np.argsort(-logits, axis=1, kind="stable")[:, : w.top_k].astype(np.int32)
    kept = np.take_along_axis(logits, ids, axis=1)
    e = np.exp(kept - kept.max(axis=1, keepdims=True))
    wts = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return x, ids, wts
