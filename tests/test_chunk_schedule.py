"""The equal-time chunk schedule (dynamic chunked pipeline parallelism's chunk
sizing; paper-review page, section 4, "Pipeline parallelism", Figure 9).

The oracle (oracle/chunk_schedule.py) states the cost model and finds the
min-max partition by dynamic programming.  It is pinned here by closed forms
of the cost (the dense triangle sum, the sparse cover's two limits), by an exhaustive
enumeration of every partition on tiny inputs, and by the linear-partition
bounds total/m <= optimum <= total/m + the largest block for additive costs.
The library's search (host code, no GPU) must then reach the oracle's optimum
on random models, return a valid partition of exactly min(m, blocks) chunks,
and report the largest cost of the bounds it returns.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import chunk_schedule as CS

import sparse_dual_chunk_amd as S


def _tri(x):
    return x * (x + 1) // 2


# ---------------------------------------------------------------- oracle pins
@pytest.mark.parametrize("a,b", [(0, 64), (0, 640), (128, 1024), (1984, 4096)])
def test_dense_pair_cost_is_the_triangle_sum(a, b):
    """Blocks of 64 rows, block beta covers 64 * (64 beta + 64) pairs: 4096 (T(B_b) - T(B_a))."""
    m = CS.ChunkCost(pair=1.0)
    assert CS.chunk_cost(a, b, m) == 4096 * (_tri(b // 64) - _tri(a // 64))


def test_ragged_last_block_and_cap_closed_forms():
    m = CS.ChunkCost(pair=1.0)
    # rows 64..100: one block of 37 rows with causal extent 101
    assert CS.chunk_cost(64, 101, m) == 37 * 101
    # a sparse block's expected cover: its extent while the budget is far larger,
    # the budget when the extent is far larger
    assert CS.chunk_cost(0, 64, CS.ChunkCost(pair=1.0, cap=10 ** 9)) == pytest.approx(64 * 64, rel=1e-6)
    far = CS.chunk_cost(64 * 10 ** 5, 64 * 10 ** 5 + 64, CS.ChunkCost(pair=1.0, cap=1000))
    assert far == pytest.approx(64 * 1000, rel=1e-3)
    # and it never exceeds either bound
    for e0 in (0, 640, 6400):
        c = CS.chunk_cost(e0, e0 + 64, CS.ChunkCost(pair=1.0, cap=2000))
        assert c <= 64 * min(e0 + 64, 2000)
    # fixed, per-row and index terms
    mf = CS.ChunkCost(call=7.0, row=0.5, index_key=0.25, pair=0.0)
    assert CS.chunk_cost(256, 640, mf) == 7.0 + 0.5 * 384 + 0.25 * 640


def _enumerate_best(n, n_chunks, max_rows, m):
    cand = CS.boundaries(n)
    inner = cand[1:-1]
    best = math.inf
    for k in range(0, min(n_chunks - 1, len(inner)) + 1):
        for cut in itertools.combinations(inner, k):
            b = [0, *cut, n]
            if any(y - x > max_rows for x, y in zip(b[:-1], b[1:])):
                continue
            best = min(best, max(CS.schedule_costs(b, m)))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_dp_equals_exhaustive_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(64 * 3, 64 * 9))
    m = CS.ChunkCost(call=float(rng.uniform(0, 2e4)), row=float(rng.uniform(0, 50)),
                     index_key=float(rng.uniform(0, 20)), pair=1.0, cap=int(rng.choice([0, 200, 333])))
    n_chunks = int(rng.integers(1, 5))
    max_rows = int(rng.choice([n, 256, 320]))
    if math.ceil(len(CS.boundaries(n)[:-1]) / (max_rows // 64)) > n_chunks:
        max_rows = n
    assert CS.optimal_max_cost(n, n_chunks, max_rows, m) == pytest.approx(_enumerate_best(n, n_chunks, max_rows, m),
                                                                          rel=1e-15)


@pytest.mark.parametrize("n_blocks,n_chunks", [(40, 4), (64, 8), (33, 5)])
def test_dp_within_the_linear_partition_bounds(n_blocks, n_chunks):
    """Additive costs (pairs only): total/m <= optimum <= total/m + largest block."""
    n = 64 * n_blocks
    m = CS.ChunkCost(pair=1.0)
    total = CS.chunk_cost(0, n, m)
    largest = CS.chunk_cost(n - 64, n, m)
    opt = CS.optimal_max_cost(n, n_chunks, n, m)
    assert total / n_chunks <= opt <= total / n_chunks + largest


# ---------------------------------------------------------------- the library against the oracle
def _lib_cost(m: CS.ChunkCost):
    return S.chunk_cost(per_call=m.call, per_row=m.row, per_index_key=m.index_key, per_pair=m.pair,
                        cover_cap=m.cap)


@pytest.mark.parametrize("seed", range(12))
def test_library_schedule_reaches_the_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(64, 64 * 40))
    if seed % 3 == 0:
        n = n // 64 * 64
    m = CS.ChunkCost(call=float(rng.choice([0.0, rng.uniform(0, 5e4)])), row=float(rng.uniform(0, 100)),
                     index_key=float(rng.choice([0.0, rng.uniform(0, 50)])), pair=float(rng.uniform(0.1, 2.0)),
                     cap=int(rng.choice([0, 300, 1000])))
    nb = len(CS.boundaries(n)) - 1
    n_chunks = int(rng.integers(1, 9))
    max_rows = int(rng.choice([64 * 1000, 64 * 6, 64 * 10]))
    if math.ceil(nb / (max_rows // 64)) > n_chunks:
        max_rows = 64 * 1000
    bounds, mx = S.dca_chunk_schedule(n, n_chunks, max_rows, _lib_cost(m))
    ok, why = CS.check_valid(bounds, n, n_chunks, max_rows)
    assert ok, why
    assert len(bounds) - 1 == min(n_chunks, nb)
    costs = CS.schedule_costs(bounds, m)
    assert mx == pytest.approx(max(costs), rel=1e-12)
    assert max(costs) == pytest.approx(CS.optimal_max_cost(n, n_chunks, max_rows, m), rel=1e-9)


def test_library_rejects_impossible_and_bad_requests():
    m = S.chunk_cost(per_pair=1.0)
    with pytest.raises(S.DcaError):
        S.dca_chunk_schedule(64 * 100, 3, 64 * 20, m)           # 3 chunks of 20 blocks cannot hold 100 blocks
    with pytest.raises(S.DcaError):
        S.dca_chunk_schedule(1000, 2, 32, m)                     # max_rows below one block
    with pytest.raises(S.DcaError):
        S.dca_chunk_schedule(1000, 2, 1000, S.chunk_cost(per_pair=-1.0))
    # more chunks than blocks: one chunk per block
    b, _ = S.dca_chunk_schedule(200, 10, 1000, m)
    assert b == [0, 64, 128, 192, 200]


def test_million_token_dense_schedule_follows_the_square_root_law():
    """Pairs only, 1M tokens, 32 chunks: equal triangle areas put bound c near n sqrt(c / 32);
    the largest chunk costs at most the ideal share plus one chunk-boundary block, far below
    the fixed 32K-row chunks' largest."""
    n, m_chunks = 1 << 20, 32
    m = CS.ChunkCost(pair=1.0)
    bounds, mx = S.dca_chunk_schedule(n, m_chunks, n, _lib_cost(m))
    total = 4096 * _tri(n // 64)
    assert total / m_chunks <= mx <= total / m_chunks + 64 * n
    for c in range(1, m_chunks):
        ideal = n * math.sqrt(c / m_chunks)
        assert abs(bounds[c] - ideal) <= 0.002 * n, (c, bounds[c], ideal)
    fixed = CS.schedule_costs(CS.fixed_chunks(n, 32768), m)
    assert mx < 0.6 * max(fixed)


def test_default_costs_follow_the_heads_and_budgets():
    cfg = S.Config(n_q=64, n_k=64, h_q=28, h_kv=4, dca_chunk=262144, dca_local=4096, rope_base=1e7, yarn_s=4.0,
                   vs_k_vertical=4096, vs_k_slash=16384)
    d = S.dca_chunk_cost_default(cfg, False)
    s = S.dca_chunk_cost_default(cfg, True)
    assert d.cover_cap == 0 and d.per_index_key == 0.0
    assert s.cover_cap == 64 * 16384 + 4096 and s.per_index_key > 0
    assert d.per_pair == pytest.approx(28 * 5.5e-7)
    half = S.dca_chunk_cost_default(S.Config(**{**cfg.__dict__, "h_q": 14, "h_kv": 2}), False)
    assert half.per_pair == pytest.approx(d.per_pair / 2)
