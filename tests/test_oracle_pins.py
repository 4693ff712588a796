"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a printed
closed form, an independent formulation (complex rotation, torch SDPA), a
brute-force loop, a special case with a closed-form answer, or a planted
structure whose selection is known by construction.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import dca_oracle as O
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(rng, shape, scale=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _cfg(h_q, h_kv, S, W, base=1e6, s=4.0, kv=0, ks=0, last=64):
    return dict(h_q=h_q, h_kv=h_kv, dca_chunk=S, dca_local=W, rope_base=base, yarn_s=s,
                vs_k_vertical=kv, vs_k_slash=ks, vs_last_q=last)


def _rope_complex(x, pos, base):
    """RoPE as a complex multiply: z_k = x_k + i x_{k+d/2} turns by pos * exp(-(2k/d) ln base)."""
    d = x.shape[-1]
    h = d // 2
    theta = np.exp(-(2.0 * np.arange(h) / d) * math.log(base))
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def _sdpa_causal_fp64(q, k, v, scale, mask=None):
    """Reference attention via torch SDPA in float64 on the CPU; q [R][d], k, v [N][d]."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None, None],
                                                             scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- P1: YaRN
def test_yarn_closed_form_matches_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "yarn_scale.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for s, root, inv_t, scale in rows:
        s = float(s)
        assert abs(O.yarn_logit_factor(s) - float(inv_t)) <= 1e-15 * float(inv_t)
        assert abs(O.softmax_scale(s, 128) - float(scale)) <= 1e-15 * float(scale)
        assert abs(math.sqrt(O.yarn_logit_factor(s)) - float(root)) <= 2e-16 * float(root)


def test_yarn_no_extrapolation_below_one():
    assert O.yarn_logit_factor(0.5) == 1.0
    assert O.yarn_logit_factor(1.0) == 1.0


# ---------------------------------------------------------------- RoPE convention
def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128))
    pos = rng.integers(0, 300000, size=50)
    for base in (1e6, 1e7):
        assert np.allclose(O.rope(x, pos, base), _rope_complex(x, pos, base), rtol=0, atol=1e-9)


def test_rope_identity_norm_and_relative_property():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 128))
    y = rng.standard_normal((8, 128))
    assert np.array_equal(O.rope(x, np.zeros(8, dtype=np.int64), 1e7), x)
    r = O.rope(x, np.arange(8) * 1000, 1e7)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # <R(a) x, R(b) y> depends on a - b only
    a, b = 5000, 1234
    lhs = np.sum(O.rope(x, a, 1e7) * O.rope(y, b, 1e7), axis=1)
    rhs = np.sum(O.rope(x, a - b, 1e7) * y, axis=1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)


# ---------------------------------------------------------------- P3: DCA invariants
@pytest.mark.parametrize("S,W", [(8, 3), (16, 16), (16, 1), (64, 8)])
def test_dca_position_invariants_exhaustive(S, W):
    n = 5 * S + 3
    p = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    causal = j <= p
    mode = O.dca_mode(p, j, S)
    pq = O.dca_query_position(p + 0 * j, mode, S, W)
    pk = O.dca_key_position(j + 0 * p, S)
    dist = pq - pk
    true = p - j
    assert dist[causal].min() >= 0
    assert dist[causal].max() <= S + W - 1
    intra = causal & (mode == O.INTRA)
    assert np.array_equal(dist[intra], true[intra])
    succ = causal & (mode == O.SUCC)
    r = (p % S) + 0 * j
    assert np.array_equal(dist[succ & (r < W)], true[succ & (r < W)])
    assert np.all(dist[succ & (r >= W)] == (S + W - 1 - pk)[succ & (r >= W)])
    inter = causal & (mode == O.INTER)
    assert np.all(dist[inter] >= W)
    # modes: same chunk, previous chunk, earlier chunks
    assert np.array_equal(mode == O.INTRA, (p // S) == (j // S))
    assert np.array_equal(mode == O.SUCC, (p // S) == (j // S) + 1)


# ---------------------------------------------------------------- P2: DCA == plain causal RoPE
@pytest.mark.parametrize("n,S,W", [(192, 256, 64), (256, 256, 64), (300, 256, 64)])
def test_dca_reduces_to_plain_rope_attention(n, S, W):
    """n <= S: one chunk, absolute positions.  n <= S + W: the successive rows with r < W
    keep true distances, so the result is still plain causal RoPE attention."""
    assert n <= S + W
    rng = np.random.default_rng(3)
    h_q, h_kv, d = 4, 2, 128
    q, k, v = _bf16(rng, (n, h_q, d)), _bf16(rng, (n, h_kv, d)), _bf16(rng, (n, h_kv, d))
    cfg = _cfg(h_q, h_kv, S, W, base=1e6, s=4.0)
    out, lse = O.attention(q, k, v, 0, cfg)
    pos = np.arange(n)
    scale = 0.1145934591559474949781697571548776140946  # golden s = 4, d = 128
    for h in range(h_q):
        g = h // 2
        qr = _rope_complex(O.bf16_to_f64(q[:, h]), pos, 1e6)
        kr = _rope_complex(O.bf16_to_f64(k[:, g]), pos, 1e6)
        ref = _sdpa_causal_fp64(qr, kr, O.bf16_to_f64(v[:, g]), scale)
        assert np.abs(out[:, h] - ref).max() <= 1e-12


def test_dca_differs_from_plain_rope_beyond_window():
    """Past S + W the remap must change the result (else the modes were never used)."""
    rng = np.random.default_rng(4)
    n, S, W, d = 160, 64, 16, 128
    q, k, v = _bf16(rng, (n, 1, d)), _bf16(rng, (n, 1, d)), _bf16(rng, (n, 1, d))
    out, _ = O.attention(q, k, v, 0, _cfg(1, 1, S, W))
    pos = np.arange(n)
    ref = _sdpa_causal_fp64(_rope_complex(O.bf16_to_f64(q[:, 0]), pos, 1e6),
                            _rope_complex(O.bf16_to_f64(k[:, 0]), pos, 1e6), O.bf16_to_f64(v[:, 0]),
                            O.softmax_scale(4.0, d))
    err = np.abs(out[:, 0] - ref).max(axis=1)
    assert err[: S + W].max() <= 1e-12
    assert err[S + W:].max() > 1e-6


# ---------------------------------------------------------------- P4: all selected == dense
def test_all_slashes_selected_equals_dense():
    rng = np.random.default_rng(5)
    p0, n_q, S, W, d = 128, 128, 64, 16, 128
    n_k = p0 + n_q
    q, k, v = _bf16(rng, (n_q, 2, d)), _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    cfg = _cfg(2, 1, S, W)
    dense = O.attention(q, k, v, p0, cfg)
    s_off = np.tile(np.arange(n_k, dtype=np.int32), (2, 1))
    v_idx = np.full((2, 0), -1, dtype=np.int32)
    sp = O.attention(q, k, v, p0, cfg, v_idx=v_idx, s_off=s_off)
    assert np.array_equal(dense[0], sp[0]) and np.array_equal(dense[1], sp[1])
    # every column as a vertical, no slashes beyond the forced diagonal
    v_all = np.tile(np.arange(n_k, dtype=np.int32), (2, 1))
    sp2 = O.attention(q, k, v, p0, cfg, v_idx=v_all, s_off=np.full((2, 0), -1, dtype=np.int32))
    assert np.array_equal(dense[0], sp2[0])


# ---------------------------------------------------------------- P5: diagonal only == block-local causal
def test_diagonal_only_is_block_local_causal_attention():
    rng = np.random.default_rng(6)
    p0, n_q, S, W, d = 192, 160, 128, 32, 128   # p0 > S: blocks sit in later chunks
    n_k = p0 + n_q
    q, k, v = _bf16(rng, (n_q, 1, d)), _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    cfg = _cfg(1, 1, S, W)
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=np.full((1, 3), -1, np.int32),
                           s_off=np.array([[0, -1, -1]], np.int32))
    scale = O.softmax_scale(4.0, d)
    for b0 in range(0, n_q, 64):
        rows = np.arange(b0, min(n_q, b0 + 64))
        pos = p0 + rows
        qr = _rope_complex(O.bf16_to_f64(q[rows, 0]), pos, 1e6)
        kr = _rope_complex(O.bf16_to_f64(k[pos, 0]), pos, 1e6)
        ref = _sdpa_causal_fp64(qr, kr, O.bf16_to_f64(v[pos, 0]), scale)
        assert np.abs(out[rows, 0] - ref).max() <= 1e-12


# ---------------------------------------------------------------- P6: constant logits
def test_zero_query_gives_mean_of_values_and_log_count():
    rng = np.random.default_rng(7)
    p0, n_q, d = 64, 100, 128
    n_k = p0 + n_q
    q = np.zeros((n_q, 2, d), dtype=np.uint16)
    k, v = _bf16(rng, (n_k, 1, d), 3.0), _bf16(rng, (n_k, 1, d))
    cfg = _cfg(2, 1, 32, 8)
    vf = O.bf16_to_f64(v[:, 0])
    out, lse = O.attention(q, k, v, p0, cfg)
    for i in range(n_q):
        p = p0 + i
        assert np.allclose(out[i, 0], vf[: p + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, i] - math.log(p + 1)) <= 1e-13
    v_idx = np.array([[3, 10, 40], [0, 1, 2]], np.int32)
    s_off = np.array([[5, 100], [70, -1]], np.int32)
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=v_idx, s_off=s_off)
    for h in range(2):
        for i in range(n_q):
            p = p0 + i
            i0 = p0 + (i // 64) * 64
            keys = set(range(i0, i0 + 64))
            for dl in s_off[h]:
                if dl >= 0:
                    keys |= set(range(i0 - dl, i0 - dl + 64))
            keys |= set(int(c) for c in v_idx[h])
            A = sorted(j for j in keys if 0 <= j <= p)
            assert np.allclose(out[i, h], vf[A].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[h, i] - math.log(len(A))) <= 1e-13


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(8)
    n, d = 96, 128
    q, k = _bf16(rng, (n, 1, d)), _bf16(rng, (n, 1, d))
    v = np.full((n, 1, d), f32_to_bf16_bits(np.array([1.5], np.float32))[0], dtype=np.uint16)
    out, _ = O.attention(q, k, v, 0, _cfg(1, 1, 32, 8))
    assert np.allclose(out, 1.5, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P7: brute force on tiny inputs
def _tiny(seed, n_q, p0, h_q=2, h_kv=1, d=8, sink=False):
    rng = np.random.default_rng(seed)
    n_k = p0 + n_q
    q = _bf16(rng, (n_q, h_q, d))
    k = _bf16(rng, (n_k, h_kv, d), 1.0)
    if sink:
        k[:2] = f32_to_bf16_bits(bf16_bits_to_f32(k[:2]) * 8)
    v = _bf16(rng, (n_k, h_kv, d))
    return q, k, v


def _nested(bits):
    return O.bf16_to_f64(bits).tolist()


@pytest.mark.parametrize("p0,n_q", [(0, 48), (64, 40), (128, 7)])
def test_attention_matches_brute_force_dense(p0, n_q):
    q, k, v = _tiny(10 + p0, n_q, p0, sink=True)
    cfg = _cfg(2, 1, 8, 3, base=1e4)
    out, lse = O.attention(q, k, v, p0, cfg)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), p0, cfg)
    assert np.abs(out - np.array(bo)).max() <= 1e-12
    assert np.abs(lse - np.array(bl)).max() <= 1e-12


@pytest.mark.parametrize("p0,n_q", [(0, 48), (128, 40)])
def test_attention_matches_brute_force_sparse(p0, n_q):
    q, k, v = _tiny(20 + p0, n_q, p0)
    cfg = _cfg(2, 1, 8, 3, base=1e4)
    rng = np.random.default_rng(p0)
    n_k = p0 + n_q
    v_idx = np.sort(rng.choice(n_k, size=(2, 5), replace=True), axis=1).astype(np.int32)
    s_off = np.sort(rng.choice(n_k, size=(2, 3), replace=False), axis=1).astype(np.int32)
    s_off[1, 0] = -1
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=v_idx, s_off=s_off)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), p0, cfg,
                             v_idx=v_idx.tolist(), s_off=s_off.tolist())
    assert np.abs(out - np.array(bo)).max() <= 1e-12
    assert np.abs(lse - np.array(bl)).max() <= 1e-12


@pytest.mark.parametrize("p0,n_q,last", [(0, 48, 16), (40, 24, 64), (16, 30, 64)])
def test_index_matches_brute_force(p0, n_q, last):
    q, k, v = _tiny(30 + p0, n_q, p0, sink=True)
    cfg = _cfg(2, 1, 8, 3, base=1e4, kv=6, ks=9, last=last)
    v_idx, s_off, gaps = O.vs_index(q, k, p0, cfg)
    bv, bs, bvert, bslash = brute.vs_index(_nested(q), _nested(k), p0, cfg)
    vert, slash, _ = O.vs_scores(q, k, p0, cfg)
    assert np.abs(vert - np.array(bvert)).max() <= 1e-12
    assert np.abs(slash - np.array(bslash)).max() <= 1e-12
    for h, gv, gs in gaps:
        if gv is not None and gv < 1e-9:
            continue  # a near-tie: the brute force may order it differently by rounding
        assert v_idx[h].tolist() == bv[h]
        if gs is None or gs >= 1e-9:
            assert s_off[h].tolist() == bs[h]


# ---------------------------------------------------------------- P8: LSE merge
def test_lse_merge_of_any_partition_equals_single_softmax():
    rng = np.random.default_rng(9)
    p0, n_q, S, W, d = 128, 64, 64, 16, 128
    n_k = p0 + n_q
    q, k, v = _bf16(rng, (n_q, 1, d)), _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    keys = np.arange(n_k)
    p_rows = p0 + np.arange(n_q)
    causal = keys[None, :] <= p_rows[:, None]
    args = (O.bf16_to_f64(q[:, 0]), p_rows, O.bf16_to_f64(k[:, 0]), O.bf16_to_f64(v[:, 0]), keys)
    rest = (S, W, 1e6, O.softmax_scale(4.0, d))
    full = O.attend_rows(*args, causal, *rest)
    # by DCA mode (the three modes' partials merged by log-sum-exp) and by a random partition
    mode = O.dca_mode(p_rows[:, None], keys[None, :], S)
    parts = [O.attend_rows(*args, causal & (mode == m), *rest) for m in (O.INTRA, O.SUCC, O.INTER)]
    out, lse = O.lse_merge(parts)
    assert np.abs(out - full[0]).max() <= 1e-13 and np.abs(lse - full[1]).max() <= 1e-13
    lab = rng.integers(0, 5, size=n_k)
    parts = [O.attend_rows(*args, causal & (lab[None, :] == t), *rest) for t in range(5)]
    parts.append((np.zeros((n_q, d)), np.full(n_q, -np.inf)))   # an empty partial weighs nothing
    out, lse = O.lse_merge(parts)
    assert np.abs(out - full[0]).max() <= 1e-13 and np.abs(lse - full[1]).max() <= 1e-13


# ---------------------------------------------------------------- P9: index special cases
def test_index_zero_query_ties_break_by_lowest_index():
    rng = np.random.default_rng(11)
    p0, n_q, d = 256, 128, 128
    n_k = p0 + n_q
    q = np.zeros((n_q, 1, d), dtype=np.uint16)
    k = _bf16(rng, (n_k, 1, d))
    cfg = _cfg(1, 1, 128, 32, kv=20, ks=33)
    v_idx, s_off, _ = O.vs_index(q, k, p0, cfg)
    assert v_idx[0].tolist() == list(range(20))
    assert s_off[0].tolist() == list(range(33))


def test_index_k_at_least_candidates_gives_all():
    rng = np.random.default_rng(12)
    p0, n_q = 0, 40
    q, k = _bf16(rng, (n_q, 1, 128)), _bf16(rng, (n_q, 1, 128))
    v_idx, s_off, _ = O.vs_index(q, k, p0, _cfg(1, 1, 16, 4, kv=50, ks=45))
    assert v_idx[0].tolist() == list(range(40)) + [-1] * 10
    assert s_off[0].tolist() == list(range(40)) + [-1] * 5


def test_index_planted_structure_is_selected():
    """Keys loaded on the lowest-frequency RoPE pair get large logits for every scoring row
    (the rotation barely turns them).  Two strong and three weaker planted keys must be
    the vertical picks, and the two strong keys' diagonals (one run of 64 offsets each,
    since each of the 64 rows meets the key at a different offset) the slash picks."""
    rng = np.random.default_rng(13)
    p0, n_q, d, S = 4096, 256, 128, 8192
    n_k = p0 + n_q
    q = _bf16(rng, (n_q, 1, d), 0.05)
    k = _bf16(rng, (n_k, 1, d), 0.05)
    lo = d // 2 - 1           # lowest-frequency pair (lo, lo + d/2)
    one = lambda x: f32_to_bf16_bits(np.array([x], np.float32))[0]
    q[:, 0, lo] = one(10.0)
    strong = [777, 2900]
    weak = [100, 1500, 3333]
    k[strong, 0, lo] = one(10.0)
    k[weak, 0, lo] = one(8.0)
    cfg = _cfg(1, 1, S, 512, base=1e6, kv=5, ks=2 * 64 + 1)
    v_idx, s_off, gaps = O.vs_index(q, k, p0, cfg)
    assert v_idx[0].tolist() == sorted(strong + weak)
    assert gaps[0][1] >= 1e-3 and gaps[0][2] >= 1e-3
    p_rows = p0 + np.arange(n_q - 64, n_q)
    expect = {0} | set((p_rows - strong[0]).tolist()) | set((p_rows - strong[1]).tolist())
    assert set(s_off[0].tolist()) == expect and len(expect) == 129
    assert s_off[0].tolist() == sorted(expect)


# ---------------------------------------------------------------- P10: GQA
def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(14)
    n, d = 130, 128
    q, k, v = _bf16(rng, (n, 6, d)), _bf16(rng, (n, 2, d)), _bf16(rng, (n, 2, d))
    out_g, lse_g = O.attention(q, k, v, 0, _cfg(6, 2, 64, 16))
    k_rep, v_rep = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    out_r, lse_r = O.attention(q, k_rep, v_rep, 0, _cfg(6, 6, 64, 16))
    assert np.array_equal(out_g, out_r) and np.array_equal(lse_g, lse_r)


# ---------------------------------------------------------------- cover counting
def test_cover_sizes_match_materialised_covers():
    rng = np.random.default_rng(15)
    for trial in range(6):
        p0 = int(rng.integers(0, 8)) * 64
        n_q = int(rng.integers(1, 400))
        n_k = p0 + n_q
        v_idx = np.sort(rng.integers(-1, n_k, size=int(rng.integers(0, 30)))).astype(np.int32)
        s_off = np.sort(rng.integers(-1, n_k, size=int(rng.integers(0, 20)))).astype(np.int32)
        sizes = O.cover_sizes(n_q, p0, n_k, v_idx, s_off)
        for b in range(len(sizes)):
            keys = O.block_cover(p0 + 64 * b, n_k, v_idx, s_off, dense=False)
            assert sizes[b] == len(keys)
            assert keys.max() < min(p0 + 64 * b + 64, n_k)


def test_flop_counts_dense_closed_form():
    # c2 shape: 28 heads, 32768 rows, dense: F_blocks = 4 d h * sum_b 64 * 64 (b+1)
    fb, fa = O.flop_counts(32768, 28, 128, 0, 32768)
    assert fb == 4 * 128 * 28 * 64 * 64 * (512 * 513 // 2)
    assert fa == 4 * 128 * 28 * (32768 * 32769 // 2)


def _brute_attended(n_q, p0, n_k, v_idx, s_off, exact):
    """sum over heads and rows of |A_h(i)|, from the brute-force module's own key sets."""
    tot = 0
    for h in range(len(v_idx)):
        for i in range(n_q):
            p = p0 + i
            if exact:
                keys = brute._exact_keys(p, v_idx[h].tolist(), s_off[h].tolist())
            else:
                i0 = p0 + (i // 64) * 64
                keys = [j for j in brute._cover(i0, n_k, v_idx[h].tolist(), s_off[h].tolist()) if j <= p]
            tot += len(keys)
    return tot


@pytest.mark.parametrize("exact", [False, True])
def test_attended_pairs_match_brute_enumeration(exact):
    """F_attended of a sparse call (block cover and exact diagonals) equals 4 d times the
    number of (row, key) pairs the brute force attends, on random patterns with padding,
    duplicates, out-of-range entries and partial last blocks."""
    rng = np.random.default_rng(17 + exact)
    for trial in range(8):
        h_q = 2
        p0 = int(rng.integers(0, 6)) * 64
        n_q = int(rng.integers(1, 260))
        n_k = p0 + n_q
        v_idx = np.sort(rng.integers(-1, n_k + 3, size=(h_q, int(rng.integers(0, 25)))), axis=1).astype(np.int32)
        s_off = np.sort(rng.integers(-1, n_k + 3, size=(h_q, int(rng.integers(0, 20)))), axis=1).astype(np.int32)
        fb, fa = O.flop_counts(n_q, h_q, 8, p0, n_k, v_idx, s_off, exact=exact)
        assert fa == 4 * 8 * _brute_attended(n_q, p0, n_k, v_idx, s_off, exact)
        fb_block, _ = O.flop_counts(n_q, h_q, 8, p0, n_k, v_idx, s_off)
        assert fb == fb_block     # the computed tiles are the same in both readings


def test_attended_pairs_closed_forms():
    n_q, p0, h_q, d = 200, 128, 3, 128
    n_k = p0 + n_q
    none = np.full((h_q, 4), -1, dtype=np.int32)
    # offset 0 only, no columns: every row attends only itself (exact), its block's
    # causal prefix (block cover)
    _, fa = O.flop_counts(n_q, h_q, d, p0, n_k, none, none, exact=True)
    assert fa == 4 * d * h_q * n_q
    rows = [64, 64, 64, 8]
    _, fa = O.flop_counts(n_q, h_q, d, p0, n_k, none, none)
    assert fa == 4 * d * h_q * sum(r * (r + 1) // 2 for r in rows)
    # every offset selected: both readings attend the dense causal set
    all_off = np.tile(np.arange(n_k, dtype=np.int32), (h_q, 1))
    _, fa_dense = O.flop_counts(n_q, h_q, d, p0, n_k)
    assert fa_dense == 4 * d * h_q * sum(p + 1 for p in range(p0, n_k))
    for exact in (False, True):
        _, fa = O.flop_counts(n_q, h_q, d, p0, n_k, none, all_off, exact=exact)
        assert fa == fa_dense
    # every column selected, offset 0 only: exact attends all j <= p (columns) once
    all_col = np.tile(np.arange(n_k, dtype=np.int32), (h_q, 1))
    _, fa = O.flop_counts(n_q, h_q, d, p0, n_k, all_col, none, exact=True)
    assert fa == fa_dense


# ---------------------------------------------------------------- generator
def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(16).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------- decode (generation step)
@pytest.mark.parametrize("n_k,n_t", [(45, 1), (45, 3), (37, 2)])
def test_decode_matches_brute_force(n_k, n_t):
    """Newest tokens at positions n_k - n_t .. n_k - 1 (not on a 64 boundary), several DCA
    chunks, a sink; key blocks of 16 exercise the partial merge."""
    rng = np.random.default_rng(40 + n_k + n_t)
    d = 8
    q = _bf16(rng, (n_t, 2, d))
    k = _bf16(rng, (n_k, 1, d))
    k[:2] = f32_to_bf16_bits(bf16_bits_to_f32(k[:2]) * 8)
    v = _bf16(rng, (n_k, 1, d))
    cfg = _cfg(2, 1, 8, 3, base=1e4)
    out, lse = O.decode_attention(q, k, v, cfg, key_block=16)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), n_k - n_t, cfg)
    assert np.abs(out - np.array(bo)).max() <= 1e-12
    assert np.abs(lse - np.array(bl)).max() <= 1e-12


def test_decode_within_window_is_plain_rope_attention():
    """n_k <= S + W: the DCA positions of every pair equal the true ones."""
    rng = np.random.default_rng(41)
    S, W, n_k, n_t, d = 256, 64, 300, 3, 128
    q, k, v = _bf16(rng, (n_t, 4, d)), _bf16(rng, (n_k, 2, d)), _bf16(rng, (n_k, 2, d))
    cfg = _cfg(4, 2, S, W, base=1e6, s=4.0)
    out, _ = O.decode_attention(q, k, v, cfg)
    p_rows = np.arange(n_k - n_t, n_k)
    mask = np.where(np.arange(n_k)[None, :] <= p_rows[:, None], 0.0, -np.inf)
    for h in range(4):
        g = h // 2
        qr = _rope_complex(O.bf16_to_f64(q[:, h]), p_rows, 1e6)
        kr = _rope_complex(O.bf16_to_f64(k[:, g]), np.arange(n_k), 1e6)
        ref = _sdpa_causal_fp64(qr, kr, O.bf16_to_f64(v[:, g]), O.softmax_scale(4.0, d), mask=mask)
        assert np.abs(out[:, h] - ref).max() <= 1e-12


def test_decode_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(42)
    n_k, n_t, d = 1000, 4, 128
    q = np.zeros((n_t, 2, d), dtype=np.uint16)
    k, v = _bf16(rng, (n_k, 1, d), 3.0), _bf16(rng, (n_k, 1, d))
    out, lse = O.decode_attention(q, k, v, _cfg(2, 1, 64, 16), key_block=256)
    vf = O.bf16_to_f64(v[:, 0])
    for t in range(n_t):
        p = n_k - n_t + t
        assert np.allclose(out[t, 1], vf[: p + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[1, t] - math.log(p + 1)) <= 1e-12


# ---------------------------------------------------------------- exact-diagonal slashes, per-head budgets
def _pattern(rng, h_q, n_k, kv, ks):
    v_idx = np.full((h_q, kv), -1, np.int32)
    s_off = np.full((h_q, ks), -1, np.int32)
    for h in range(h_q):
        nv, ns = kv - int(rng.integers(0, 2)), ks - int(rng.integers(0, 2))
        v_idx[h, :nv] = np.sort(rng.choice(n_k, nv, replace=False))
        s_off[h, :ns] = np.sort(rng.choice(n_k, ns, replace=False))
    return v_idx, s_off


@pytest.mark.parametrize("p0,n_q", [(0, 48), (128, 40)])
def test_exact_diagonals_match_brute_force(p0, n_q):
    q, k, v = _tiny(60 + p0, n_q, p0, sink=True)
    n_k = p0 + n_q
    v_idx, s_off = _pattern(np.random.default_rng(p0), 2, n_k, 5, 9)
    cfg = _cfg(2, 1, 8, 3, base=1e4, kv=5, ks=9)
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=v_idx, s_off=s_off, exact=True)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), p0, cfg, v_idx.tolist(), s_off.tolist(),
                             exact=True)
    assert np.abs(out - np.array(bo)).max() <= 1e-12
    assert np.abs(lse - np.array(bl)).max() <= 1e-12


def test_exact_self_diagonal_only_returns_own_value():
    """Only delta = 0 and no vertical: each row attends itself, out = v_i, lse = its own logit."""
    rng = np.random.default_rng(61)
    p0, n_q, d = 64, 70, 128
    n_k = p0 + n_q
    q, k, v = _bf16(rng, (n_q, 2, d)), _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    cfg = _cfg(2, 1, 32, 8, kv=1, ks=1)
    none = np.full((2, 1), -1, np.int32)
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=none, s_off=none, exact=True)
    vf = O.bf16_to_f64(v[:, 0])
    assert np.array_equal(out[:, 0], vf[p0:]) and np.array_equal(out[:, 1], vf[p0:])
    # r_i = p_i mod 32 for both query and key: the logit is scale * |q|.|k| turned by the same angle
    for i in (0, 33, 69):
        p = p0 + i
        ql = O.rope(O.bf16_to_f64(q[i, 0]), p % 32, 1e6)
        kl = O.rope(O.bf16_to_f64(k[p, 0]), p % 32, 1e6)
        assert abs(lse[0, i] - O.softmax_scale(4.0, d) * float(ql @ kl)) <= 1e-12


def test_exact_all_offsets_equals_dense():
    rng = np.random.default_rng(62)
    p0, n_q, d = 128, 100, 128
    n_k = p0 + n_q
    q, k, v = _bf16(rng, (n_q, 2, d)), _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    cfg = _cfg(2, 1, 64, 16, kv=1, ks=n_k)
    s_off = np.tile(np.arange(n_k, dtype=np.int32), (2, 1))
    out, lse = O.attention(q, k, v, p0, cfg, v_idx=np.full((2, 1), -1, np.int32), s_off=s_off, exact=True)
    ref, ref_lse = O.attention(q, k, v, p0, _cfg(2, 1, 64, 16))
    assert np.abs(out - ref).max() <= 1e-12 and np.abs(lse - ref_lse).max() <= 1e-12


def test_exact_zero_query_gives_mean_over_the_exact_set():
    rng = np.random.default_rng(63)
    p0, n_q, d = 64, 60, 128
    n_k = p0 + n_q
    q = np.zeros((n_q, 1, d), np.uint16)
    k, v = _bf16(rng, (n_k, 1, d)), _bf16(rng, (n_k, 1, d))
    v_idx = np.array([[2, 50, 90]], np.int32)
    s_off = np.array([[1, 7, 64, -1]], np.int32)
    out, lse = O.attention(q, k, v, p0, _cfg(1, 1, 32, 8, kv=3, ks=4), v_idx=v_idx, s_off=s_off, exact=True)
    vf = O.bf16_to_f64(v[:, 0])
    for i in range(n_q):
        p = p0 + i
        A = sorted({p - dl for dl in (0, 1, 7, 64) if p - dl >= 0} | {c for c in (2, 50, 90) if c <= p})
        assert np.allclose(out[i, 0], vf[A].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, i] - math.log(len(A))) <= 1e-13


def test_index_per_head_budgets_match_brute_force():
    q, k, _ = _tiny(70, 40, 64)
    cfg = _cfg(2, 1, 8, 3, base=1e4, kv=6, ks=9, last=16)
    budgets = [(6, 9), (2, 4)]
    v_idx, s_off, _ = O.vs_index(q, k, 64, cfg, budgets=budgets)
    bv, bs, _, _ = brute.vs_index(_nested(q), _nested(k), 64, cfg, budgets=budgets)
    assert v_idx.tolist() == bv and s_off.tolist() == bs
    assert (v_idx[1, 2:] == -1).all() and (s_off[1, 4:] == -1).all()
    full_v, full_s, _ = O.vs_index(q, k, 64, cfg)
    assert np.array_equal(full_v[0], v_idx[0]) and np.array_equal(full_s[0], s_off[0])
