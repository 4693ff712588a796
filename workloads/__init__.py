"""Seeded synthetic workloads for DCA + vertical-slash sparse prefill attention.

This module holds only the workload shapes and the seeded input generator.  It
computes nothing of the attention method itself (no rotation, no scaling, no
softmax), so both the CPU oracle and the GPU path can take their inputs from
it without sharing any of the method's arithmetic.

Shapes follow the Qwen2.5-1M technical report as summarised on the
xllm-io paper-review page, section 3 (model table: 7B has 28 query / 4 KV
heads, 14B has 40 / 8) and the agentlenshq release blog, "Sparse Attention"
(chunked prefill with 32,768-token chunks).  Values are standard normal,
rounded to bfloat16; attention-sink keys (rows 0-3) are scaled by 8 and
periodic keys (every 4096th row from 4096 on) by 4.  Both factors are powers
of two, so the scaled values stay exactly representable in bfloat16.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

HEAD_DIM = 128
QBLOCK = 64          # rows of one query block (the granule of the sparse cover)
SINK_ROWS = 4
SINK_SCALE = 8.0
PERIOD = 4096
PERIOD_SCALE = 4.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer workload.

    ``chunks`` lists (p0, n_q) per prefill call: the query rows are positions
    p0 .. p0+n_q-1 and the KV prefix is keys 0 .. p0+n_q-1.
    """
    name: str
    h_q: int
    h_kv: int
    dca_chunk: int          # S
    dca_local: int          # W
    rope_base: float
    yarn_s: float
    k_vertical: int         # 0 and k_slash 0 => dense
    k_slash: int
    chunks: tuple
    sinks: bool
    periodic: bool
    head_dim: int = HEAD_DIM
    vs_last_q: int = 64

    @property
    def sparse(self) -> bool:
        return self.k_vertical > 0 or self.k_slash > 0

    @property
    def n_k_total(self) -> int:
        return max(p0 + nq for p0, nq in self.chunks)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes measured by the benchmark and the parity tests.
C1_TINY = Workload("tiny_dense_2k", 4, 1, 512, 128, 1e6, 4.0, 0, 0,
                   ((0, 2048),), sinks=False, periodic=False)
C2_7B_DENSE_32K = Workload("7b_dense_32k", 28, 4, 8192, 1024, 1e7, 4.0, 0, 0,
                           ((0, 32768),), sinks=True, periodic=False)
C3_7B_CHUNK_128K = Workload("7b_chunk_at_98304_of_128k", 28, 4, 32768, 2048, 1e7, 4.0,
                            1024, 4096, ((98304, 32768),), sinks=True, periodic=True)
C4_14B_256K = Workload("14b_256k_in_8_chunks", 40, 8, 65536, 2048, 1e7, 4.0, 2048, 8192,
                       tuple((32768 * c, 32768) for c in range(8)), sinks=True, periodic=True)
C5_7B_1M = Workload("7b_last_chunk_of_1m", 28, 4, 262144, 4096, 1e7, 4.0, 4096, 16384,
                    ((1048576 - 32768, 32768),), sinks=True, periodic=True)

WORKLOADS = {w.name: w for w in (C1_TINY, C2_7B_DENSE_32K, C3_7B_CHUNK_128K, C4_14B_256K, C5_7B_1M)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed_seq, shape, chunk_rows: int = 1 << 16) -> np.ndarray:
    """Standard normal bfloat16 bits, drawn row-block by row-block from one stream.

    Drawing in row blocks from one generator yields the same values as one big
    draw (the stream is consumed in C order), while bounding the float32
    temporary to ``chunk_rows`` rows.
    """
    rng = np.random.default_rng(seed_seq)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    inner = shape[1:]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0,) + inner, dtype=np.float32))
    return out


def _scale_rows_pow2(bits: np.ndarray, rows, factor: float) -> None:
    """Multiply whole bf16 rows by a power of two, in place (exact)."""
    if len(rows) == 0:
        return
    vals = bf16_bits_to_f32(bits[rows]) * np.float32(factor)
    bits[rows] = f32_to_bf16_bits(vals)


def make_keys_values(w: Workload, n_k: int, seed: int = 0):
    """K and V for keys 0..n_k-1, shape [n_k][h_kv][d], bfloat16 bits.

    The prefix of a longer draw equals a shorter draw, so every chunk of a
    chunked prefill sees the same keys.
    """
    shape = (n_k, w.h_kv, w.head_dim)
    k = _normal_bf16([seed, 1], shape)
    v = _normal_bf16([seed, 2], shape)
    if w.sinks:
        _scale_rows_pow2(k, np.arange(min(SINK_ROWS, n_k)), SINK_SCALE)
    if w.periodic:
        _scale_rows_pow2(k, np.arange(PERIOD, n_k, PERIOD), PERIOD_SCALE)
    return k, v


def make_queries(w: Workload, p0: int, n_q: int, seed: int = 0) -> np.ndarray:
    """Q rows for positions p0..p0+n_q-1, shape [n_q][h_q][d], bfloat16 bits."""
    return _normal_bf16([seed, 0, p0], (n_q, w.h_q, w.head_dim))


def make(w: Workload, chunk: int = 0, seed: int = 0, kv: Optional[tuple] = None) -> dict:
    """Inputs of one prefill call: q, k, v (bf16 bits), host positions, p0."""
    p0, n_q = w.chunks[chunk]
    n_k = p0 + n_q
    if kv is None:
        k, v = make_keys_values(w, n_k, seed)
    else:
        k, v = kv[0][:n_k], kv[1][:n_k]
    q = make_queries(w, p0, n_q, seed)
    positions = np.arange(p0, p0 + n_q, dtype=np.int32)
    return dict(q=q, k=k, v=v, positions=positions, p0=p0, n_q=n_q, n_k=n_k)


def sample_blocks(n_q: int, h_q: int, seed: int = 0, n_random: int = 2) -> List[tuple]:
    """(head, q-block) pairs checked at full size: blocks 0, 1, mid, last plus seeded random ones."""
    nb = (n_q + QBLOCK - 1) // QBLOCK
    rng = np.random.default_rng([seed, 7])
    pairs = []
    for h in range(h_q):
        picks = {0, min(1, nb - 1), nb // 2, nb - 1}
        picks.update(int(x) for x in rng.integers(0, nb, size=n_random))
        pairs.extend((h, b) for b in sorted(picks))
    return pairs
