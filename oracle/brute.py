"""Pure-Python brute force of the same definitions as the vectorised oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle.dca_oracle``).  Scalar loops with
``math.exp``, ``math.cos`` and ``math.sin`` on tiny inputs, written
independently of the numpy oracle, so that a mistake in either shows up as a
disagreement.  Positions, modes and covers are rebuilt here from the
definitions, not imported.
"""
from __future__ import annotations

import math
from typing import List, Optional


def _rot(x: List[float], pos: int, base: float) -> List[float]:
    d = len(x)
    h = d // 2
    out = [0.0] * d
    for k in range(h):
        ang = pos * (base ** (-(2.0 * k) / d))
        c, s = math.cos(ang), math.sin(ang)
        out[k] = x[k] * c - x[k + h] * s
        out[k + h] = x[k] * s + x[k + h] * c
    return out


def _dot(a, b) -> float:
    t = 0.0
    for x, y in zip(a, b):
        t += x * y
    return t


def _scale(s: float, d: int) -> float:
    f = 1.0 if s <= 1.0 else (0.1 * math.log(s) + 1.0) ** 2
    return f / math.sqrt(d)


def _dca_pair_positions(p: int, j: int, S: int, W: int):
    mi, mj, r = p // S, j // S, p % S
    if mj == mi:
        pq = r
    elif mj == mi - 1:
        pq = min(S + r, S + W - 1)
    else:
        pq = S + W - 1
    return pq, j % S


def _cover(i0: int, n_k: int, vcols, soffs) -> List[int]:
    hi = min(i0 + 64, n_k)
    if vcols is None and soffs is None:
        return list(range(hi))
    keys = set()
    for delta in [0] + [x for x in soffs if x >= 0]:
        for t in range(64):
            j = i0 - delta + t
            if 0 <= j < hi:
                keys.add(j)
    for c in vcols:
        if 0 <= c < hi:
            keys.add(c)
    return sorted(keys)


def _exact_keys(p: int, vcols, soffs) -> List[int]:
    keys = set()
    for delta in [0] + [x for x in soffs if x >= 0]:
        if p - delta >= 0:
            keys.add(p - delta)
    for c in vcols:
        if 0 <= c <= p:
            keys.add(c)
    return sorted(keys)


def attention(q, k, v, p0: int, cfg: dict, v_idx=None, s_off=None, exact: bool = False):
    """q [n_q][h_q][d], k, v [n_k][h_kv][d] as nested float lists.  ``exact``: a row
    attends the keys exactly on its selected diagonals and vertical columns.

    Returns (out [n_q][h_q][d], lse [h_q][n_q]).
    """
    n_q, h_q, d = len(q), len(q[0]), len(q[0][0])
    n_k = len(k)
    S, W, base = cfg["dca_chunk"], cfg["dca_local"], cfg["rope_base"]
    G = h_q // cfg["h_kv"]
    sc = _scale(cfg["yarn_s"], d)
    out = [[[0.0] * d for _ in range(h_q)] for _ in range(n_q)]
    lse = [[-math.inf] * n_q for _ in range(h_q)]
    for h in range(h_q):
        g = h // G
        for i in range(n_q):
            p = p0 + i
            i0 = p0 + (i // 64) * 64
            if exact and v_idx is not None:
                keys = _exact_keys(p, v_idx[h], s_off[h])
            else:
                cov = _cover(i0, n_k, None if v_idx is None else v_idx[h], None if s_off is None else s_off[h])
                keys = [j for j in cov if j <= p]
            if not keys:
                continue
            logits = []
            for j in keys:
                pq, pk = _dca_pair_positions(p, j, S, W)
                logits.append(sc * _dot(_rot(q[i][h], pq, base), _rot(k[j][g], pk, base)))
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            z = sum(w)
            for t, j in enumerate(keys):
                for c in range(d):
                    out[i][h][c] += w[t] * v[j][g][c] / z
            lse[h][i] = m + math.log(z)
    return out, lse


def vs_index(q, k, p0: int, cfg: dict, budgets=None):
    """Vertical / slash scores and top-k selections, by loops over (row, key).
    ``budgets``: per-head (k_v, k_s), padded to the config's k with -1."""
    n_q, h_q, d = len(q), len(q[0]), len(q[0][0])
    n_k = len(k)
    S, base = cfg["dca_chunk"], cfg["rope_base"]
    G = h_q // cfg["h_kv"]
    sc = _scale(cfg["yarn_s"], d)
    n_s = min(cfg.get("vs_last_q", 64), n_q)
    p_last = p0 + n_q - 1
    kv, ks = cfg["vs_k_vertical"], cfg["vs_k_slash"]
    verts, slashes, vsel, ssel = [], [], [], []
    for h in range(h_q):
        g = h // G
        vert = [0.0] * n_k
        slash = [0.0] * (p_last + 1)
        for i in range(n_q - n_s, n_q):
            p = p0 + i
            logits = []
            for j in range(p + 1):
                pq = (p % S) if (j // S == p // S) else (S + p % S)
                logits.append(sc * _dot(_rot(q[i][h], pq, base), _rot(k[j][g], j % S, base)))
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            z = sum(w)
            for j in range(p + 1):
                vert[j] += w[j] / z
                slash[p - j] += w[j] / z
        verts.append(vert)
        slashes.append(slash)
        kvh, ksh = (kv, ks) if budgets is None else budgets[h]
        vsel.append(_topk(vert, kvh, forced=()) + [-1] * (kv - kvh))
        ssel.append(_topk(slash, ksh, forced=(0,)) + [-1] * (ks - ksh))
    return vsel, ssel, verts, slashes


def _topk(scores, k: int, forced=()):
    n = len(scores)
    key = [(math.inf if i in forced else s) for i, s in enumerate(scores)]
    order = sorted(range(n), key=lambda i: (-key[i], i))
    chosen = sorted(order[:min(k, n)])
    return chosen + [-1] * (k - len(chosen))
