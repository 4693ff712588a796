"""CPU fp64 oracle for DCA + vertical-slash sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code with the GPU library: it is a plain, slow
restatement of what the method computes, in float64, with numpy.

Sources (the Qwen2.5-1M technical report, as summarised on the pages):
  * xllm-io paper-review page, section 4 "Inference & deployment":
      - Dual Chunk Attention, Figure 2: relative positions are remapped to
        small values seen in training; three modes: intra-chunk, inter-chunk
        and successive-chunk (the last keeps short-range relative positions
        continuous between adjacent chunks).
      - YaRN attention scaling: softmax(q^T k / (t sqrt(D))) with
        sqrt(1/t) = 0.1 ln(s) + 1, s = inference / training length ratio.
      - Sparse attention, Figure 4: MInference vertical-slash sparsity, with
        critical tokens chosen per chunk of a chunked prefill, and continuous
        relative positions restored when key tokens are selected.
  * agentlenshq release blog, "Sparse Attention": prefill chunk of 32,768.

Where the pages leave a step open, the readings below are taken (the register
in the design notes lists every one):
  * DCA positions: key position = j mod S.  Query position: intra-chunk
    r_i = p_i mod S; successive chunk min(S + r_i, S + W - 1); any earlier
    chunk S + W - 1.
  * RoPE: half-split pairs (x_k, x_{k+d/2}), angle = position * base^(-2k/d).
  * YaRN: factor (0.1 ln s + 1)^2 on the logits (1 when s <= 1), applied in all
    modes, with the usual 1/sqrt(d).
  * Index scoring: the last ``vs_last_q`` rows of the chunk; continuous
    positions (query at r_i for keys of its own chunk, at S + r_i for any
    earlier chunk, unclamped); row softmax over causal keys; vertical score =
    column sum, slash score = diagonal sum over offsets delta = p_i - j;
    delta = 0 always selected; ranking by (score desc, index asc); emitted
    ascending; -1 pads when fewer candidates than slots.
  * Sparse semantics: block cover with a 64-row granule.  For the query block
    starting at absolute position i0, each selected offset delta (and delta = 0)
    covers keys [i0 - delta, i0 - delta + 63]; the vertical columns are added;
    the union is clipped to [0, i0 + 63] and each row then attends its causal
    part.  Empty sets give O = 0, lse = -inf.
  * Exact-diagonal variant (optional): a row at position p attends key j <= p
    when p - j is a selected offset (or 0) or j a selected vertical column,
    with no 64-row granule.  Per-head budgets (optional): each head keeps its
    own k best of each list, padded to the configured k with -1.
  * Generation step (decode): the newest tokens attend every cached key up to
    their own position with the same DCA positions, densely (the pages apply
    the sparse attention to the prefill).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

QBLOCK = 64


# ----------------------------------------------------------------------------
# Scalars: YaRN factor and RoPE frequencies
# ----------------------------------------------------------------------------
def yarn_logit_factor(s: float) -> float:
    """1/t from the YaRN equation sqrt(1/t) = 0.1 ln(s) + 1 (paper-review page, section 4)."""
    if s <= 1.0:
        return 1.0
    root = 0.1 * math.log(s) + 1.0
    return root * root


def softmax_scale(s: float, d: int) -> float:
    """Logit multiplier 1 / (t sqrt(D)) of the YaRN-scaled softmax."""
    return yarn_logit_factor(s) / math.sqrt(d)


def rope_inv_freq(base: float, d: int) -> np.ndarray:
    """theta_k = base^(-2k/d) for k < d/2, each by a scalar libm pow call."""
    return np.array([math.pow(base, -(2.0 * k) / d) for k in range(d // 2)], dtype=np.float64)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of ``x`` (fp64) by RoPE at positions ``pos``.

    Half-split pairing: component k pairs with k + d/2 and turns by
    pos * theta_k.  ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(base, d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns as float64."""
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# DCA position remapping (paper-review page, section 4, Figure 2)
# ----------------------------------------------------------------------------
INTRA, SUCC, INTER = 0, 1, 2


def dca_mode(p_i, j, S: int):
    """0 intra-chunk (same chunk), 1 successive chunk (previous), 2 inter-chunk (earlier)."""
    mi = np.asarray(p_i) // S
    mj = np.asarray(j) // S
    return np.where(mj == mi, INTRA, np.where(mj == mi - 1, SUCC, INTER))


def dca_query_position(p_i, mode, S: int, W: int):
    """Remapped query position for a (row, key) pair of the given mode."""
    r = np.asarray(p_i) % S
    return np.where(mode == INTRA, r, np.where(mode == SUCC, np.minimum(S + r, S + W - 1), S + W - 1))


def dca_key_position(j, S: int):
    return np.asarray(j) % S


# ----------------------------------------------------------------------------
# Attention over an explicit key set, one query head and a group of rows
# ----------------------------------------------------------------------------
def attend_rows(q_rows: np.ndarray, p_rows: np.ndarray, k_keys: np.ndarray, v_keys: np.ndarray,
                key_ids: np.ndarray, allowed: np.ndarray, S: int, W: int, base: float,
                scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of rows over keys, with DCA positions per (row, key) pair.

    q_rows [R][d] raw (unrotated) fp64; k_keys, v_keys [N][d] raw fp64 for the
    absolute key ids ``key_ids`` [N]; ``allowed`` [R][N] bool marks the pairs
    each row attends.  Returns (out [R][d], lse [R]) with natural-log lse;
    rows with no allowed key get out = 0, lse = -inf.
    """
    R, d = q_rows.shape
    k_rot = rope(k_keys, dca_key_position(key_ids, S), base)
    logits = np.full((R, len(key_ids)), -np.inf)
    # The three DCA modes partition the (row, key) pairs; each uses its own
    # query rotation.
    mode = dca_mode(p_rows[:, None], key_ids[None, :], S)
    for m in (INTRA, SUCC, INTER):
        sel = (mode == m) & allowed
        if not sel.any():
            continue
        qpos = dca_query_position(p_rows, np.full(R, m), S, W)
        q_rot = rope(q_rows, qpos, base)
        full = scale * (q_rot @ k_rot.T)
        logits[sel] = full[sel]
    return _softmax_out(logits, v_keys)


def _softmax_out(logits: np.ndarray, v_keys: np.ndarray):
    R = logits.shape[0]
    mx = logits.max(axis=1) if logits.shape[1] else np.full(R, -np.inf)
    out = np.zeros((R, v_keys.shape[1]))
    lse = np.full(R, -np.inf)
    ok = np.isfinite(mx)
    if ok.any():
        e = np.exp(logits[ok] - mx[ok, None])
        ssum = e.sum(axis=1)
        out[ok] = (e @ v_keys) / ssum[:, None]
        lse[ok] = mx[ok] + np.log(ssum)
    return out, lse


# ----------------------------------------------------------------------------
# Vertical-slash cover (block cover, 64-row granule)
# ----------------------------------------------------------------------------
def block_cover(i0: int, n_k: int, v_idx_h: Optional[np.ndarray], s_off_h: Optional[np.ndarray],
                dense: bool) -> np.ndarray:
    """Sorted absolute key ids covered for the query block starting at position i0.

    Dense: every key 0..min(i0+63, n_k-1).  Sparse: for delta in the slash set
    plus delta = 0, keys i0-delta .. i0-delta+63; plus the vertical columns;
    clipped to [0, min(i0+63, n_k-1)].  Negative entries are padding and ignored.
    """
    hi = min(i0 + QBLOCK, n_k)
    if dense:
        return np.arange(0, hi, dtype=np.int64)
    covered = np.zeros(hi, dtype=bool)
    offs = np.asarray(s_off_h if s_off_h is not None else [], dtype=np.int64)
    offs = np.concatenate([[0], offs[offs >= 0]])
    for delta in offs:
        lo_k = i0 - int(delta)
        covered[max(lo_k, 0):max(min(lo_k + QBLOCK, hi), 0)] = True
    cols = np.asarray(v_idx_h if v_idx_h is not None else [], dtype=np.int64)
    cols = cols[(cols >= 0) & (cols < hi)]
    covered[cols] = True
    return np.flatnonzero(covered).astype(np.int64)


def exact_cover_mask(p_rows: np.ndarray, keys: np.ndarray, v_idx_h: Optional[np.ndarray],
                     s_off_h: Optional[np.ndarray]) -> np.ndarray:
    """Exact-diagonal semantics: row at position p attends key j <= p iff p - j is a
    selected slash offset (or 0), or j is a selected vertical column.  Returns the
    [R][N] bool mask over ``keys``; negative entries are padding."""
    offs = np.asarray(s_off_h if s_off_h is not None else [], dtype=np.int64)
    offs = np.unique(np.concatenate([[0], offs[offs >= 0]]))
    cols = np.asarray(v_idx_h if v_idx_h is not None else [], dtype=np.int64)
    cols = cols[cols >= 0]
    delta = p_rows[:, None] - keys[None, :]
    on_slash = np.isin(delta, offs)
    on_vert = np.isin(keys, cols)[None, :]
    return (delta >= 0) & (on_slash | on_vert)


def slash_intervals(s_off_h: Optional[np.ndarray]) -> np.ndarray:
    """Union of the slash footprints [-delta, -delta+64) (and delta = 0) as disjoint
    half-open intervals in offset space relative to a block start, ascending."""
    offs = np.asarray(s_off_h if s_off_h is not None else [], dtype=np.int64)
    offs = np.unique(np.concatenate([[0], offs[offs >= 0]]))
    los = np.sort(-offs)
    out = []
    for lo in los:
        if out and lo <= out[-1][1]:
            out[-1][1] = max(out[-1][1], lo + QBLOCK)
        else:
            out.append([lo, lo + QBLOCK])
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def cover_sizes(n_q: int, p0: int, n_k: int, v_idx_h, s_off_h) -> np.ndarray:
    """|C_h(b)| for every query block b of one head, via merged slash intervals.

    Same sets as :func:`block_cover`, counted without materialising them, so
    the full-size block counts stay cheap.
    """
    nb = (n_q + QBLOCK - 1) // QBLOCK
    iv = slash_intervals(s_off_h)
    cols = np.asarray(v_idx_h if v_idx_h is not None else [], dtype=np.int64)
    cols = np.unique(cols[cols >= 0])
    sizes = np.zeros(nb, dtype=np.int64)
    for b in range(nb):
        i0 = p0 + b * QBLOCK
        hi = min(i0 + QBLOCK, n_k)
        lo_abs = np.clip(i0 + iv[:, 0], 0, hi)
        hi_abs = np.clip(i0 + iv[:, 1], 0, hi)
        in_ranges = int((hi_abs - lo_abs).sum())
        c = cols[cols < hi]
        pos = np.searchsorted(i0 + iv[:, 0], c, side="right") - 1
        inside = (pos >= 0) & (c < i0 + iv[np.maximum(pos, 0), 1])
        sizes[b] = in_ranges + int((~inside).sum())
    return sizes


def attention_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, p0: int, h: int, b: int, cfg: dict,
                    v_idx: Optional[np.ndarray] = None, s_off: Optional[np.ndarray] = None, exact: bool = False):
    """Output rows of query block b for query head h.  q, k, v are bf16 bit arrays.

    ``exact``: the exact-diagonal semantics of :func:`exact_cover_mask` instead of
    the 64-row block cover (sparse calls only).
    Returns (out [rows][d], lse [rows], cover keys).
    """
    n_q = q.shape[0]
    n_k = k.shape[0]
    G = cfg["h_q"] // cfg["h_kv"]
    g = h // G
    r0, r1 = b * QBLOCK, min(n_q, (b + 1) * QBLOCK)
    p_rows = np.arange(p0 + r0, p0 + r1)
    i0 = p0 + r0
    dense = v_idx is None and s_off is None
    keys = block_cover(i0, n_k, None if dense else v_idx[h], None if dense else s_off[h], dense)
    if exact and not dense:
        allowed = exact_cover_mask(p_rows, keys, v_idx[h], s_off[h])
    else:
        allowed = keys[None, :] <= p_rows[:, None]
    out, lse = attend_rows(bf16_to_f64(q[r0:r1, h]), p_rows, bf16_to_f64(k[keys, g]), bf16_to_f64(v[keys, g]),
                           keys, allowed, cfg["dca_chunk"], cfg["dca_local"], cfg["rope_base"],
                           softmax_scale(cfg["yarn_s"], q.shape[2]))
    return out, lse, keys


def attention(q, k, v, p0: int, cfg: dict, v_idx=None, s_off=None, heads=None, exact: bool = False):
    """Full prefill attention for one call (dense if v_idx and s_off are None;
    ``exact`` selects the exact-diagonal semantics for sparse calls).

    Returns (out [n_q][h_q][d] fp64, lse [h_q][n_q] fp64).
    """
    n_q, h_q, d = q.shape
    out = np.zeros((n_q, h_q, d))
    lse = np.full((h_q, n_q), -np.inf)
    nb = (n_q + QBLOCK - 1) // QBLOCK
    for h in (range(h_q) if heads is None else heads):
        for b in range(nb):
            o, l, _ = attention_block(q, k, v, p0, h, b, cfg, v_idx, s_off, exact)
            r0 = b * QBLOCK
            out[r0:r0 + len(l), h] = o
            lse[h, r0:r0 + len(l)] = l
    return out, lse


def decode_attention(q, k, v, cfg: dict, heads=None, key_block: int = 1 << 18):
    """One generation step: the n_t rows of ``q`` are the newest tokens, at
    positions n_k - n_t .. n_k - 1, and each attends every cached key j <= its
    position with the DCA positions of its (row, key) pairs (the generation
    side of the same attention: no sparsity, which the pages apply to the
    prefill).  q [n_t][h_q][d], k, v [n_k][h_kv][d] bf16 bits.

    Keys are taken ``key_block`` at a time and the blocks' softmax partials
    merged by ``lse_merge`` (exact), so a million-key cache fits in memory.
    Returns (out [n_t][h_q][d] fp64, lse [h_q][n_t] fp64).
    """
    n_t, h_q, d = q.shape
    n_k = k.shape[0]
    G = h_q // cfg["h_kv"]
    S, W, base = cfg["dca_chunk"], cfg["dca_local"], cfg["rope_base"]
    scale = softmax_scale(cfg["yarn_s"], d)
    p_rows = np.arange(n_k - n_t, n_k)
    out = np.zeros((n_t, h_q, d))
    lse = np.full((h_q, n_t), -np.inf)
    for h in (range(h_q) if heads is None else heads):
        g = h // G
        qr = bf16_to_f64(q[:, h])
        parts = []
        for j0 in range(0, n_k, key_block):
            keys = np.arange(j0, min(n_k, j0 + key_block))
            allowed = keys[None, :] <= p_rows[:, None]
            parts.append(attend_rows(qr, p_rows, bf16_to_f64(k[keys, g]), bf16_to_f64(v[keys, g]), keys, allowed,
                                     S, W, base, scale))
        o, l = lse_merge(parts) if len(parts) > 1 else parts[0]
        out[:, h] = o
        lse[h] = l
    return out, lse


def lse_merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Merge softmax partials (O_p normalised [R][d], lse_p [R]) into (O, lse).

    m = max_p lse_p; O = sum_p e^{lse_p - m} O_p / sum_p e^{lse_p - m};
    lse = m + ln sum_p e^{lse_p - m}.  Partials with lse = -inf weigh 0.
    """
    lses = np.stack([p[1] for p in parts])
    outs = np.stack([p[0] for p in parts])
    m = lses.max(axis=0)
    ok = np.isfinite(m)
    w = np.zeros_like(lses)
    w[:, ok] = np.exp(lses[:, ok] - m[ok])
    tot = w.sum(axis=0)
    out = np.zeros(outs.shape[1:])
    out[ok] = np.einsum("pr,prd->rd", w[:, ok], outs[:, ok]) / tot[ok, None]
    lse = np.full(m.shape, -np.inf)
    lse[ok] = m[ok] + np.log(tot[ok])
    return out, lse


# ----------------------------------------------------------------------------
# Vertical-slash index (paper-review page, section 4, Figure 4)
# ----------------------------------------------------------------------------
def vs_scores(q, k, p0: int, cfg: dict, heads=None):
    """Vertical and slash scores per query head, from the last scoring rows.

    Returns (vert [h_q][n_k], slash [h_q][p_last+1], scoring positions).  The
    forced slash offset 0 is not applied here.
    """
    n_q, h_q, d = q.shape
    n_k = k.shape[0]
    S = cfg["dca_chunk"]
    base = cfg["rope_base"]
    scale = softmax_scale(cfg["yarn_s"], d)
    G = h_q // cfg["h_kv"]
    n_s = min(cfg.get("vs_last_q", 64), n_q)
    rows = np.arange(n_q - n_s, n_q)
    p_rows = p0 + rows
    p_last = p0 + n_q - 1
    keys = np.arange(n_k)
    heads = range(h_q) if heads is None else heads
    vert = np.zeros((h_q, n_k))
    slash = np.zeros((h_q, p_last + 1))
    k_rot_cache = {}
    for h in heads:
        g = h // G
        if g not in k_rot_cache:
            k_rot_cache = {g: rope(bf16_to_f64(k[:, g]), dca_key_position(keys, S), base)}
        k_rot = k_rot_cache[g]
        qh = bf16_to_f64(q[rows, h])
        logits = np.full((n_s, n_k), -np.inf)
        same = (keys[None, :] // S) == (p_rows[:, None] // S)
        causal = keys[None, :] <= p_rows[:, None]
        for same_chunk in (True, False):
            qpos = (p_rows % S) if same_chunk else (S + p_rows % S)
            full = scale * (rope(qh, qpos, base) @ k_rot.T)
            sel = (same == same_chunk) & causal
            logits[sel] = full[sel]
        mx = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - mx)
        a = e / e.sum(axis=1, keepdims=True)
        vert[h] = a.sum(axis=0)
        for t in range(n_s):
            # row t contributes A[t, j] to offset delta = p_t - j for j <= p_t
            pt = p_rows[t]
            slash[h, :pt + 1] += a[t, pt::-1]
    return vert, slash, p_rows


def topk_ascending(scores: np.ndarray, k: int, forced: Sequence[int] = ()):
    """Indices of the k best scores by (score desc, index asc), emitted ascending.

    ``forced`` indices rank first.  Pads with -1 when fewer candidates exist.
    Returns (indices [k] int32, relative gap at the cut or None).
    """
    n = scores.shape[0]
    key = scores.astype(np.float64).copy()
    for f in forced:
        if 0 <= f < n:
            key[f] = np.inf
    order = np.lexsort((np.arange(n), -key))      # primary: -score asc; secondary: index asc
    take = min(k, n)
    chosen = np.sort(order[:take]).astype(np.int32)
    out = np.full(k, -1, dtype=np.int32)
    out[:take] = chosen
    gap = None
    if 0 < take < n:
        s_k, s_next = key[order[take - 1]], key[order[take]]
        if np.isfinite(s_k) and s_k > 0:
            gap = float((s_k - s_next) / s_k)
        else:
            gap = float("inf") if s_k != s_next else 0.0
    return out, gap


def vs_index(q, k, p0: int, cfg: dict, heads=None, budgets=None):
    """Vertical column ids [h_q][k_v] and slash offsets [h_q][k_s], plus the cut gaps.

    ``budgets`` [h_q][2] (optional): per-head (k_v, k_s), each at most the
    config's k_v, k_s; a head's row holds its own k best, padded with -1.
    """
    h_q = q.shape[1]
    kv, ks = cfg["vs_k_vertical"], cfg["vs_k_slash"]
    vert, slash, _ = vs_scores(q, k, p0, cfg, heads)
    v_idx = np.full((h_q, kv), -1, dtype=np.int32)
    s_off = np.full((h_q, ks), -1, dtype=np.int32)
    gaps = []
    for h in (range(h_q) if heads is None else heads):
        kv_h, ks_h = (kv, ks) if budgets is None else (int(budgets[h][0]), int(budgets[h][1]))
        v_idx[h, :kv_h], gv = topk_ascending(vert[h], kv_h)
        s_off[h, :ks_h], gs = topk_ascending(slash[h], ks_h, forced=(0,))
        gaps.append((h, gv, gs))
    return v_idx, s_off, gaps


# ----------------------------------------------------------------------------
# Work counts
# ----------------------------------------------------------------------------
def _selected_offsets(s_off_h) -> np.ndarray:
    offs = np.asarray(s_off_h if s_off_h is not None else [], dtype=np.int64)
    return np.unique(np.concatenate([[0], offs[offs >= 0]]))


def _selected_columns(v_idx_h) -> np.ndarray:
    cols = np.asarray(v_idx_h if v_idx_h is not None else [], dtype=np.int64)
    return np.unique(cols[cols >= 0])


def exact_attended_pairs(n_q: int, p0: int, v_idx_h, s_off_h) -> int:
    """sum_i |A(i)| of one head under the exact-diagonal semantics, by inclusion-exclusion:
    a row at position p attends the keys p - delta (delta a selected offset or 0, delta <= p)
    and the selected columns j <= p; a key that is both is counted once.  The keys counted
    twice are the pairs (column j, offset delta) with p0 <= j + delta <= p_last."""
    offs = _selected_offsets(s_off_h)
    cols = _selected_columns(v_idx_h)
    p = np.arange(p0, p0 + n_q, dtype=np.int64)
    on_diag = int(np.searchsorted(offs, p, side="right").sum())
    on_col = int(np.searchsorted(cols, p, side="right").sum())
    p_last = p0 + n_q - 1
    lo = np.searchsorted(offs, p0 - cols, side="left")
    hi = np.searchsorted(offs, p_last - cols, side="right")
    both = int((hi - lo).sum())
    return on_diag + on_col - both


def flop_counts(n_q: int, h_q: int, d: int, p0: int, n_k: int, v_idx=None, s_off=None, exact: bool = False):
    """(F_blocks, F_attended) for one call.

    F_blocks = 4 d sum_h sum_b rows(b) |C_h(b)|: the canonical block cover,
    counted over every row of each block.  F_attended = 4 d sum_h sum_i |A_h(i)|
    counts only the (row, key) pairs each row attends.

    Dense: |A(i)| = p_i + 1.  Block cover: the cover of block b always holds the
    block's own keys [i0, i0 + rows) (offset 0 is always selected) and nothing
    above them, so |A(i)| = |C_h(b)| - rows + (p_i - i0 + 1) and a block adds
    rows (|C_h(b)| - rows) + rows (rows + 1) / 2.  Exact diagonals
    (``exact``): :func:`exact_attended_pairs`; F_blocks is the block cover in
    both sparse readings (the same tiles are computed).
    """
    dense = v_idx is None and s_off is None
    nb = (n_q + QBLOCK - 1) // QBLOCK
    rows = np.array([min(n_q, (b + 1) * QBLOCK) - b * QBLOCK for b in range(nb)], dtype=np.int64)
    fb = 0
    fa = 0
    for h in range(h_q):
        if dense:
            sizes = np.array([min(p0 + b * QBLOCK + QBLOCK, n_k) for b in range(nb)], dtype=np.int64)
            fb += int((rows * sizes).sum())
            fa += int((np.arange(p0, p0 + n_q, dtype=np.int64) + 1).sum())
        else:
            sizes = cover_sizes(n_q, p0, n_k, v_idx[h], s_off[h])
            fb += int((rows * sizes).sum())
            if exact:
                fa += exact_attended_pairs(n_q, p0, v_idx[h], s_off[h])
            else:
                fa += int((rows * (sizes - rows) + rows * (rows + 1) // 2).sum())
    return 4 * d * fb, 4 * d * fa
