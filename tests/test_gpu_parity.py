"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, small shapes.

Attention outputs: max-abs <= 2e-2 and mean-abs <= 2e-3 on the bf16 output.
Index selections: bit-exact.  Sizes span several 64-row blocks and 64-key tiles,
ragged tails, several DCA chunks, sinks (the split-precision tiles), split-K.
"""
import math

import numpy as np
import pytest

from oracle import dca_oracle as O
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_dual_chunk_amd as S  # noqa: E402
from tests.gpu_helpers import (bf16_f64, check_close, oracle_cfg, run_index, run_prefill)  # noqa: E402

# The natural-log LSE comes from logits of bf16-rounded rotated q and k: each
# logit carries an error of order 2^-9 * scale * |q| |k| (about 0.005 to 0.01 for
# unit-variance rows, scale 0.115); the LSE inherits at most the largest logit
# error.  1e-2 bounds it for these inputs.
LSE_TOL = 1e-2


def _inputs(seed, p0, n_q, h_q, h_kv, sinks=False, periodic=0, qscale=1.0):
    rng = np.random.default_rng(seed)
    n_k = p0 + n_q
    q = f32_to_bf16_bits(rng.standard_normal((n_q, h_q, 128)).astype(np.float32) * np.float32(qscale))
    kf = rng.standard_normal((n_k, h_kv, 128)).astype(np.float32)
    if sinks:
        kf[:4] *= 8
    if periodic:
        kf[periodic::periodic] *= 4
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(rng.standard_normal((n_k, h_kv, 128)).astype(np.float32))
    return dict(q=q, k=k, v=v, positions=np.arange(p0, n_k, dtype=np.int32), p0=p0, n_q=n_q, n_k=n_k)


def _cfg(inp, h_q, h_kv, S_, W, base=1e6, s=4.0, **kw):
    return S.Config(n_q=inp["n_q"], n_k=inp["n_k"], h_q=h_q, h_kv=h_kv, dca_chunk=S_, dca_local=W,
                    rope_base=base, yarn_s=s, **kw)


def _oracle(inp, cfg, v_idx=None, s_off=None):
    return O.attention(inp["q"], inp["k"], inp["v"], inp["p0"], oracle_cfg(cfg), v_idx=v_idx, s_off=s_off)


# ------------------------------------------------------------------ dense
def test_tiny_dense_all_rows():
    import workloads as W
    w = W.C1_TINY
    inp = W.make(w, 0, seed=0)
    cfg = S.config_for(w)
    out, lse = run_prefill(inp, cfg, with_lse=True)
    ref, ref_lse = _oracle(inp, cfg)
    check_close(out, ref, "tiny dense")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


@pytest.mark.parametrize("p0,n_q,split", [(320, 333, 0), (0, 200, 1), (128, 1, 0), (640, 190, 3)])
def test_dense_ragged_multichunk_with_sinks(p0, n_q, split):
    inp = _inputs(1 + p0, p0, n_q, 4, 2, sinks=True)
    cfg = _cfg(inp, 4, 2, 256, 64, split_k=split)
    out, lse = run_prefill(inp, cfg, with_lse=True)
    ref, ref_lse = _oracle(inp, cfg)
    check_close(out, ref, f"dense p0={p0} n_q={n_q}")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


def test_dense_window_equals_chunk_and_large_base():
    inp = _inputs(2, 512, 256, 2, 1, sinks=True)
    cfg = _cfg(inp, 2, 1, 128, 128, base=1e7, s=2.0)
    out, _ = run_prefill(inp, cfg)
    check_close(out, _oracle(inp, cfg)[0], "W == S")


# ------------------------------------------------------------------ sparse
def _random_pattern(rng, h_q, n_k, kv, ks, pad=True):
    v_idx = np.full((h_q, kv), -1, dtype=np.int32)
    s_off = np.full((h_q, ks), -1, dtype=np.int32)
    for h in range(h_q):
        nv = kv - (int(rng.integers(0, 3)) if pad else 0)
        ns = ks - (int(rng.integers(0, 3)) if pad else 0)
        v_idx[h, :nv] = np.sort(rng.choice(n_k, size=nv, replace=False))
        s_off[h, :ns] = np.sort(rng.choice(n_k, size=ns, replace=False))
    return v_idx, s_off


@pytest.mark.parametrize("p0,n_q,kv,ks,split", [(512, 300, 40, 25, 0), (1024, 130, 100, 6, 1),
                                               (256, 64, 10, 60, 2)])
def test_sparse_random_pattern(p0, n_q, kv, ks, split):
    inp = _inputs(10 + p0, p0, n_q, 4, 1, sinks=True, periodic=97)
    rng = np.random.default_rng(p0 + n_q)
    v_idx, s_off = _random_pattern(rng, 4, inp["n_k"], kv, ks)
    cfg = _cfg(inp, 4, 1, 256, 32, vs_k_vertical=kv, vs_k_slash=ks, split_k=split)
    out, lse = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    ref, ref_lse = _oracle(inp, cfg, v_idx, s_off)
    check_close(out, ref, "sparse")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


@pytest.mark.parametrize("p0,n_q,split", [(512, 300, 0), (512, 300, 3), (1024, 130, 0), (1024, 130, 2)])
@pytest.mark.parametrize("exact", [0, 1])
def test_sparse_every_key_high_norm(p0, n_q, split, exact):
    """Every key takes split-precision logits (a norm threshold of 1e-3).  With at
    most 1024 such keys per KV head (n_k 812) the plan marks the range tiles
    holding them; for the block cover it lists every covered key with the
    block's extra keys and the range tiles mask them all, including the block's
    own rows (causal masks inside the extra tiles).  With more (n_k 1154) the
    second kernel instance serves every work item, walking them grid-stride and
    testing each tile's runs."""
    inp = _inputs(30 + p0, p0, n_q, 4, 1, sinks=True)
    rng = np.random.default_rng(p0 + 7)
    v_idx, s_off = _random_pattern(rng, 4, inp["n_k"], 40, 25)
    cfg = _cfg(inp, 4, 1, 256, 32, vs_k_vertical=40, vs_k_slash=25, split_k=split, precise_norm=1e-3,
               slash_exact=exact)
    out, lse = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    ref, ref_lse = (_oracle_exact if exact else _oracle)(inp, cfg, v_idx, s_off)
    check_close(out, ref, "every key high-norm")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


def test_sparse_all_offsets_equals_dense():
    inp = _inputs(20, 192, 200, 2, 1, sinks=True)
    n_k = inp["n_k"]
    s_off = np.tile(np.arange(n_k, dtype=np.int32), (2, 1))
    v_idx = np.full((2, 1), -1, dtype=np.int32)
    cfg = _cfg(inp, 2, 1, 128, 32, vs_k_vertical=1, vs_k_slash=n_k)
    out_sp, _ = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off)
    cfg_d = _cfg(inp, 2, 1, 128, 32)
    out_d, _ = run_prefill(inp, cfg_d)
    ref = _oracle(inp, cfg_d)[0]
    check_close(out_sp, ref, "all offsets")
    check_close(out_d, ref, "dense")
    # same key sets, different tile grouping (sparse tiles follow the merged
    # ranges): the two may differ only by rounding
    assert np.abs(bf16_f64(out_sp) - bf16_f64(out_d)).max() <= 2e-2


def test_sparse_vertical_only():
    inp = _inputs(21, 384, 150, 2, 2)
    rng = np.random.default_rng(5)
    v_idx, _ = _random_pattern(rng, 2, inp["n_k"], 50, 1, pad=False)
    s_off = np.full((2, 0), -1, dtype=np.int32)
    cfg = _cfg(inp, 2, 2, 128, 16, vs_k_vertical=50, vs_k_slash=0)
    out, _ = run_prefill(inp, cfg, v_idx=v_idx, s_off=np.full((2, 1), -1, np.int32))
    check_close(out, _oracle(inp, cfg, v_idx, s_off)[0], "vertical only")


def test_determinism_bitwise():
    inp = _inputs(30, 256, 256, 4, 2, sinks=True)
    rng = np.random.default_rng(1)
    v_idx, s_off = _random_pattern(rng, 4, inp["n_k"], 30, 20)
    cfg = _cfg(inp, 4, 2, 128, 32, vs_k_vertical=30, vs_k_slash=20, split_k=2)
    a, la = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    b, lb = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ------------------------------------------------------------------ head counts
# Workgroups map to the 8 dies per KV group when the KV-head count divides 8
# (1, 2, 4, 8); other counts (3, 5, 16 here) take the all-heads mapping.  Also
# one query head per KV head (no grouping).  Dense workgroups: two blocks when
# p0 and S are multiples of 128, else two heads of one block when a group has
# an even number of heads, else one block of one head.
@pytest.mark.parametrize("h_q,h_kv,p0,n_q,split", [(6, 3, 0, 200, 0),      # two-block workgroups
                                                   (6, 3, 192, 150, 2),    # head pairs, split
                                                   (8, 4, 320, 190, 0),    # head pairs, die-per-group mapping
                                                   (8, 2, 64, 130, 3),     # head pairs, four heads per group
                                                   (10, 5, 256, 64, 1),
                                                   (16, 16, 128, 130, 0),
                                                   (4, 4, 64, 100, 0)])    # one block of one head
def test_dense_head_counts(h_q, h_kv, p0, n_q, split):
    inp = _inputs(60 + h_kv + p0, p0, n_q, h_q, h_kv, sinks=True)
    cfg = _cfg(inp, h_q, h_kv, 256, 64, split_k=split)
    out, lse = run_prefill(inp, cfg, with_lse=True)
    ref, ref_lse = _oracle(inp, cfg)
    check_close(out, ref, f"dense h_q {h_q} h_kv {h_kv}")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


@pytest.mark.parametrize("h_q,h_kv,p0,n_q,split,exact", [(6, 3, 512, 200, 0, 0), (6, 3, 320, 130, 3, 0),
                                                         (16, 16, 256, 100, 2, 0), (6, 3, 512, 200, 2, 1)])
def test_sparse_head_counts(h_q, h_kv, p0, n_q, split, exact):
    inp = _inputs(70 + h_kv + p0, p0, n_q, h_q, h_kv, sinks=True, periodic=97)
    rng = np.random.default_rng(h_q + p0)
    v_idx, s_off = _random_pattern(rng, h_q, inp["n_k"], 30, 25)
    cfg = _cfg(inp, h_q, h_kv, 256, 32, vs_k_vertical=30, vs_k_slash=25, split_k=split, slash_exact=exact)
    out, lse = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    ref, ref_lse = O.attention(inp["q"], inp["k"], inp["v"], inp["p0"], oracle_cfg(cfg), v_idx=v_idx,
                               s_off=s_off, exact=bool(exact))
    check_close(out, ref, f"sparse h_q {h_q} h_kv {h_kv} exact {exact}")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


# ------------------------------------------------------------------ index
def _check_index(inp, cfg, heads=None):
    v_gpu, s_gpu = run_index(inp, cfg)
    v_ref, s_ref, gaps = O.vs_index(inp["q"], inp["k"], inp["p0"], oracle_cfg(cfg), heads=heads)
    for h, gv, gs in gaps:
        assert gv is None or gv >= 1e-9, f"oracle gap too small at head {h}: {gv}"
        assert gs is None or gs >= 1e-9, f"oracle gap too small at head {h}: {gs}"
        assert np.array_equal(v_gpu[h], v_ref[h]), f"vertical mismatch head {h}"
        assert np.array_equal(s_gpu[h], s_ref[h]), f"slash mismatch head {h}"
    return v_gpu, s_gpu


@pytest.mark.parametrize("p0,n_q,S_,last", [(192, 200, 128, 64), (192, 100, 256, 64), (0, 40, 64, 64),
                                             (1024, 256, 512, 32)])
def test_index_bit_exact(p0, n_q, S_, last):
    inp = _inputs(40 + p0 + n_q, p0, n_q, 4, 2, sinks=True, periodic=128)
    cfg = _cfg(inp, 4, 2, S_, 32, vs_k_vertical=20, vs_k_slash=40, vs_last_q=last)
    _check_index(inp, cfg)


@pytest.mark.parametrize("h_q,h_kv", [(6, 3), (16, 16)])
def test_index_head_counts(h_q, h_kv):
    inp = _inputs(45 + h_kv, 448, 160, h_q, h_kv, sinks=True, periodic=128)
    cfg = _cfg(inp, h_q, h_kv, 256, 32, vs_k_vertical=20, vs_k_slash=40)
    _check_index(inp, cfg)


def test_index_zero_query_ties():
    inp = _inputs(50, 256, 128, 2, 1)
    inp["q"][:] = 0
    cfg = _cfg(inp, 2, 1, 128, 32, vs_k_vertical=20, vs_k_slash=33)
    v_gpu, s_gpu = run_index(inp, cfg)
    for h in range(2):
        assert v_gpu[h].tolist() == list(range(20))
        assert s_gpu[h].tolist() == list(range(33))


def test_index_k_at_least_candidates():
    inp = _inputs(51, 0, 40, 2, 1)
    cfg = _cfg(inp, 2, 1, 64, 16, vs_k_vertical=50, vs_k_slash=45)
    v_gpu, s_gpu = run_index(inp, cfg)
    for h in range(2):
        assert v_gpu[h].tolist() == list(range(40)) + [-1] * 10
        assert s_gpu[h].tolist() == list(range(40)) + [-1] * 5


def test_index_planted_structure():
    rng = np.random.default_rng(13)
    p0, n_q = 4096, 256
    inp = _inputs(52, p0, n_q, 1, 1)
    one = lambda x: f32_to_bf16_bits(np.array([x], np.float32))[0]
    inp["q"] = f32_to_bf16_bits(rng.standard_normal((n_q, 1, 128)).astype(np.float32) * np.float32(0.05))
    inp["k"] = f32_to_bf16_bits(rng.standard_normal((p0 + n_q, 1, 128)).astype(np.float32) * np.float32(0.05))
    inp["q"][:, 0, 63] = one(10.0)
    strong, weak = [777, 2900], [100, 1500, 3333]
    inp["k"][strong, 0, 63] = one(10.0)
    inp["k"][weak, 0, 63] = one(8.0)
    cfg = _cfg(inp, 1, 1, 8192, 512, vs_k_vertical=5, vs_k_slash=129)
    v_gpu, s_gpu = run_index(inp, cfg)
    assert v_gpu[0].tolist() == sorted(strong + weak)
    p_rows = p0 + np.arange(n_q - 64, n_q)
    expect = sorted({0} | set((p_rows - strong[0]).tolist()) | set((p_rows - strong[1]).tolist()))
    assert s_gpu[0].tolist() == expect


def test_index_deterministic():
    inp = _inputs(53, 512, 128, 2, 1, sinks=True)
    cfg = _cfg(inp, 2, 1, 256, 32, vs_k_vertical=30, vs_k_slash=50)
    a = run_index(inp, cfg)
    b = run_index(inp, cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_index_then_prefill_end_to_end():
    """The GPU index fed to the GPU attention equals the oracle path end to end."""
    inp = _inputs(54, 768, 256, 4, 2, sinks=True, periodic=64)
    cfg = _cfg(inp, 4, 2, 256, 64, vs_k_vertical=24, vs_k_slash=48)
    v_gpu, s_gpu = _check_index(inp, cfg)
    out, _ = run_prefill(inp, cfg, v_idx=v_gpu, s_off=s_gpu)
    v_ref, s_ref, _ = O.vs_index(inp["q"], inp["k"], inp["p0"], oracle_cfg(cfg))
    check_close(out, _oracle(inp, cfg, v_ref, s_ref)[0], "index + prefill")


# ------------------------------------------------------------------ exact diagonals, per-head budgets
@pytest.mark.parametrize("p0,n_q,kv,ks,split", [(512, 300, 40, 25, 0), (1024, 130, 100, 6, 1),
                                               (256, 64, 10, 60, 2), (768, 200, 7, 90, 3)])
def test_sparse_exact_diagonals(p0, n_q, kv, ks, split):
    inp = _inputs(80 + p0, p0, n_q, 4, 1, sinks=True, periodic=97)
    rng = np.random.default_rng(p0 + n_q + 1)
    v_idx, s_off = _random_pattern(rng, 4, inp["n_k"], kv, ks)
    cfg = _cfg(inp, 4, 1, 256, 32, vs_k_vertical=kv, vs_k_slash=ks, split_k=split, slash_exact=1)
    out, lse = run_prefill(inp, cfg, v_idx=v_idx, s_off=s_off, with_lse=True)
    ref, ref_lse = _oracle_exact(inp, cfg, v_idx, s_off)
    check_close(out, ref, "exact diagonals")
    assert np.abs(lse - ref_lse).max() <= LSE_TOL


def _oracle_exact(inp, cfg, v_idx, s_off):
    return O.attention(inp["q"], inp["k"], inp["v"], inp["p0"], oracle_cfg(cfg), v_idx=v_idx, s_off=s_off,
                       exact=True)


def test_exact_self_diagonal_returns_own_values():
    """Offset 0 only, no vertical column: every row attends itself alone, so the output
    is its own value row, bit for bit."""
    inp = _inputs(81, 640, 200, 2, 1, sinks=True)
    none = np.full((2, 1), -1, np.int32)
    cfg = _cfg(inp, 2, 1, 256, 32, vs_k_vertical=1, vs_k_slash=1, slash_exact=1)
    out, _ = run_prefill(inp, cfg, v_idx=none, s_off=none)
    for h in range(2):
        assert np.array_equal(out[:, h], inp["v"][inp["p0"]:, 0])


def test_exact_all_offsets_equals_dense():
    inp = _inputs(82, 192, 200, 2, 1, sinks=True)
    n_k = inp["n_k"]
    s_off = np.tile(np.arange(n_k, dtype=np.int32), (2, 1))
    cfg = _cfg(inp, 2, 1, 128, 32, vs_k_vertical=1, vs_k_slash=n_k, slash_exact=1)
    out, _ = run_prefill(inp, cfg, v_idx=np.full((2, 1), -1, np.int32), s_off=s_off)
    check_close(out, _oracle(inp, _cfg(inp, 2, 1, 128, 32))[0], "exact, all offsets")


def test_index_per_head_budgets():
    inp = _inputs(83, 1024, 256, 4, 2, sinks=True, periodic=128)
    cfg = _cfg(inp, 4, 2, 512, 32, vs_k_vertical=20, vs_k_slash=40)
    budgets = [[20, 40], [5, 12], [0, 1], [20, 3]]
    v_gpu, s_gpu = run_index(inp, cfg, budgets=budgets)
    v_ref, s_ref, gaps = O.vs_index(inp["q"], inp["k"], inp["p0"], oracle_cfg(cfg), budgets=budgets)
    for h, gv, gs in gaps:
        assert gv is None or gv >= 1e-9
        assert gs is None or gs >= 1e-9
    assert np.array_equal(v_gpu, v_ref) and np.array_equal(s_gpu, s_ref)
    # the exact-diagonal prefill from this index, end to end
    ecfg = _cfg(inp, 4, 2, 512, 32, vs_k_vertical=20, vs_k_slash=40, slash_exact=1)
    out, _ = run_prefill(inp, ecfg, v_idx=v_gpu, s_off=s_gpu)
    check_close(out, _oracle_exact(inp, ecfg, v_ref, s_ref)[0], "budgets + exact")
