"""GPU parity of the fused MoE layer (moe_forward) against the fp64 oracle.

Cases: small shapes spanning several 128-row weight tiles of both products;
skewed routing so that some experts get none and one gets more than 32 and
more than 64 slots (the 2-tile and multi-pass paths); dropped slots (ids
outside [0, E)); a single token; bitwise determinism; and the benchmark's
64-expert, top-8, 3584 x 2560 shape at 1 and 64 tokens, checked on sampled
tokens.  Tolerance (bf16 activations between the products, bf16 output):
max-abs <= 4e-3 and mean-abs <= 4e-4 on outputs of magnitude up to ~0.5 (the
bf16 output rounding alone is up to 2^-9 |out| ~ 1e-3; measured max errors
3e-5 .. 1.6e-3).  More than 1024 slots (600 tokens x 2) takes the slot sort
through two rounds.  Shapes with few routable experts (min(E, slots) x d_ff/128 < 512)
run one-wave workgroups, the others four-wave ones; both kinds are covered.
"""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as M
from workloads import moe as WM

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_dual_chunk_amd as S  # noqa: E402
from tests.gpu_helpers import dev, host_u16  # noqa: E402

MAX_ABS = 4e-3
MEAN_ABS = 4e-4


def log(msg):
    print(f"[moe] {msg}", file=sys.stderr, flush=True)


def packed(w13, w2):
    """Device copies of the weights in the packed layout moe_forward reads."""
    E, two_ff, d = w13.shape
    cfg = S.MoeConfig(n_tokens=1, n_experts=E, top_k=1, d_model=d, d_ff=two_ff // 2)
    a, b = dev(w13), dev(w2)
    pa, pb = torch.empty_like(a), torch.empty_like(b)
    S.moe_pack_weights(a, b, cfg, pa, pb)
    torch.cuda.synchronize()
    return pa, pb


def pack_reference(w):
    """The packed layout of [n][R][C] as the header states it, with numpy."""
    n, R, C = w.shape
    t = w.reshape(n, R // 32, 32, C // 64, 2, 4, 8)          # [n][t][l%32][s][l/32][j][8]
    return np.ascontiguousarray(t.transpose(0, 1, 3, 5, 4, 2, 6)).reshape(n, R, C)


def test_moe_pack_layout_bit_exact():
    w = WM.MoeWorkload("t", 1, 3, 1, 384, 256)
    w13, w2 = WM.make_weights(w, 9)
    pa, pb = packed(w13, w2)
    assert np.array_equal(host_u16(pa), pack_reference(w13))
    assert np.array_equal(host_u16(pb), pack_reference(w2))


def run(x, ids, wts, w13, w2, d_weights=None):
    T, k = ids.shape
    E, two_ff, d = w13.shape
    cfg = S.MoeConfig(n_tokens=T, n_experts=E, top_k=k, d_model=d, d_ff=two_ff // 2)
    W13, W2 = d_weights if d_weights is not None else packed(w13, w2)
    out = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ws = torch.empty(S.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    S.moe_forward(dev(x), torch.from_numpy(np.ascontiguousarray(ids)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(wts)).cuda(), W13, W2, cfg, out, ws)
    torch.cuda.synchronize()
    return host_u16(out)


def check(got_bits, ref, what):
    got = M.bf16_to_f64(got_bits)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"{what}: max {err.max():.3e} mean {err.mean():.3e}"
    return err.max()


@pytest.mark.parametrize("T,E,k,d,d_ff,skew", [(5, 6, 2, 256, 128, 0.0), (40, 8, 3, 384, 640, 0.0),
                                                (200, 8, 2, 256, 256, 3.0), (1, 16, 4, 512, 384, 0.0),
                                                (600, 12, 2, 256, 128, 1.0), (64, 128, 2, 256, 512, 0.0),
                                                (300, 128, 4, 256, 512, 2.0),
                                                (3, 4, 4, 256, 128, 0.0)])   # top_k = n_experts: every expert, every token
def test_moe_small_against_oracle(T, E, k, d, d_ff, skew):
    w = WM.MoeWorkload("t", T, E, k, d, d_ff, skew=skew)
    x, ids, wts = WM.make_tokens(w, T + E)
    w13, w2 = WM.make_weights(w, T + E)
    counts = np.bincount(ids.ravel(), minlength=E)
    log(f"T {T} E {E} k {k} d {d} d_ff {d_ff} skew {skew}: slots per expert {counts.tolist()}")
    if skew >= 3:
        assert counts.max() > 64 and (counts == 0).any()
    got = run(x, ids, wts, w13, w2)
    mx = check(got, M.moe_forward(x, ids, wts, w13, w2), "small")
    log(f"max abs error {mx:.2e}")


@pytest.mark.parametrize("T,dead", [(30, 7),      # 90 slots: one pass per expert, no k parts
                                    (12, 5)])     # 36 slots: the products run in k parts
def test_moe_dropped_slots(T, dead):
    w = WM.MoeWorkload("t", T, 6, 3, 256, 256)
    x, ids, wts = WM.make_tokens(w, 1)
    w13, w2 = WM.make_weights(w, 1)
    ids = ids.copy()
    ids[::4, 0] = -1
    ids[1::5, 2] = 6
    ids[dead] = -1                                # a token with every slot dropped
    got = run(x, ids, wts, w13, w2)
    check(got, M.moe_forward(x, ids, wts, w13, w2), "dropped")
    assert not M.bf16_to_f64(got[dead]).any()


def test_moe_deterministic():
    w = WM.MoeWorkload("t", 70, 8, 2, 256, 384, skew=1.0)
    x, ids, wts = WM.make_tokens(w, 2)
    w13, w2 = WM.make_weights(w, 2)
    dw = packed(w13, w2)
    assert np.array_equal(run(x, ids, wts, w13, w2, dw), run(x, ids, wts, w13, w2, dw))


_FULL = {}


def _full_weights():
    if not _FULL:
        w = WM.MOE_DECODE_64
        log(f"generating {w.n_experts} experts of {w.d_model} x {w.d_ff}")
        w13, w2 = WM.make_weights(w, 0)
        _FULL["host"] = (w13, w2)
        _FULL["dev"] = packed(w13, w2)
    return _FULL["host"], _FULL["dev"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 64])
def test_moe_benchmark_shape(T):
    w = WM.MOE_DECODE_64.scaled(n_tokens=T)
    (w13, w2), dw = _full_weights()
    x, ids, wts = WM.make_tokens(w, 0)
    got = run(x, ids, wts, w13, w2, dw)
    toks = sorted({0, T - 1, T // 2, T // 3})
    log(f"oracle on tokens {toks}")
    mx = check(got[toks], M.moe_forward(x, ids, wts, w13, w2, tokens=toks), f"T {T}")
    log(f"max abs error {mx:.2e}")
    assert np.isfinite(M.bf16_to_f64(got)).all()
