"""CPU oracle of the equal-time chunk schedule (the single-GPU half of DCPP).

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark may import this
module; the GPU library never calls it and shares no code with it.

Source: xllm-io paper-review page, section 4 "Inference & deployment",
"Pipeline parallelism" (Figure 9): dynamic chunked pipeline parallelism sizes
the chunks of a chunked prefill by the attention kernel's cost, so that every
chunk takes about the same time and the pipeline has few bubbles.

The pages give no cost formula.  The reading taken here: a chunk of query rows
[a, b) of one sequence (its prefix then ends at key b) costs

    call + row * (b - a) + index_key * b
         + pair * sum over the 64-row blocks [i0, i0 + r) inside [a, b)
                  of r * cover(i0 + r)

i.e. a fixed cost per call, a per-row cost (query rotations, output, merge),
the index build over the whole prefix (zero for a dense prefill) and the
attention's computed (row, key) pairs of each block.  A dense block computes
its causal extent E = i0 + r.  A sparse block's cover is the union of its
selected diagonals' 64-key footprints and vertical columns, at most
cap = 64 k_s + k_v keys; with those keys' worth of footprints scattered
uniformly over the extent, the expected union is E (1 - exp(-cap / E)), which
is E while cap >> E and tends to cap when E >> cap (cap <= 0: dense).
Chunks start on multiples of 64.

The schedule splits n tokens into at most ``m`` chunks of at most
``max_rows`` rows and minimises the largest chunk cost.  The oracle finds that
optimum by exhaustive dynamic programming over the 64-row block boundaries,
which is only practical for small n; it exists to check the library's fast
search.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

QBLOCK = 64


@dataclasses.dataclass
class ChunkCost:
    call: float = 0.0
    row: float = 0.0
    pair: float = 1.0
    index_key: float = 0.0
    cap: int = 0


def chunk_cost(a: int, b: int, m: ChunkCost) -> float:
    """Cost of the chunk of rows [a, b) under the model in the module docstring."""
    assert 0 <= a < b and a % QBLOCK == 0
    pairs = 0
    i0 = a
    while i0 < b:
        r = min(QBLOCK, b - i0)
        extent = float(i0 + r)
        if m.cap > 0:
            extent = extent * (1.0 - math.exp(-m.cap / extent))
        pairs += r * extent
        i0 += r
    return m.call + m.row * (b - a) + m.index_key * b + m.pair * pairs


def boundaries(n: int) -> List[int]:
    """Candidate chunk boundaries: multiples of 64 below n, then n."""
    return list(range(0, n, QBLOCK)) + [n]


def optimal_max_cost(n: int, n_chunks: int, max_rows: int, m: ChunkCost) -> float:
    """min over partitions of [0, n) into at most n_chunks chunks (rows <= max_rows)
    of the largest chunk cost, by dynamic programming over block boundaries."""
    cand = boundaries(n)
    nb = len(cand)
    INF = math.inf
    # best[c][j]: smallest max cost of covering [0, cand[j]) with c chunks
    best = [[INF] * nb for _ in range(n_chunks + 1)]
    best[0][0] = 0.0
    for c in range(1, n_chunks + 1):
        for j in range(1, nb):
            for i in range(j):
                if cand[j] - cand[i] > max_rows or best[c - 1][i] == INF:
                    continue
                v = max(best[c - 1][i], chunk_cost(cand[i], cand[j], m))
                if v < best[c][j]:
                    best[c][j] = v
    return min(best[c][nb - 1] for c in range(1, n_chunks + 1))


def schedule_costs(bounds: Sequence[int], m: ChunkCost) -> List[float]:
    return [chunk_cost(a, b, m) for a, b in zip(bounds[:-1], bounds[1:])]


def fixed_chunks(n: int, size: int) -> List[int]:
    """The fixed-size schedule: chunks of ``size`` rows, the last one ragged."""
    return list(range(0, n, size)) + [n]


def check_valid(bounds: Sequence[int], n: int, n_chunks: int, max_rows: int) -> Tuple[bool, str]:
    """A schedule is valid if it starts at 0, ends at n, rises, starts every chunk
    on a multiple of 64, keeps every chunk within max_rows and uses at most n_chunks."""
    if bounds[0] != 0 or bounds[-1] != n:
        return False, "ends"
    if len(bounds) - 1 > n_chunks:
        return False, "too many chunks"
    for a, b in zip(bounds[:-1], bounds[1:]):
        if not a < b:
            return False, "not rising"
        if a % QBLOCK:
            return False, "start not a multiple of 64"
        if b - a > max_rows:
            return False, "chunk too long"
    return True, ""
