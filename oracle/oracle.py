"""Plain CPU oracle for block-sparse attention in the SpargeAttention2 form (numpy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
``cpu_baseline`` leg of the benchmark may import or call this module. The product path never
does, and this module imports nothing from the GPU package.

Pages this follows (cited by short tag below):

* [SA2]  "SpargeAttention2とは？Top-k+Top-pハイブリッドマスキングでビデオ生成を16.2倍高速化"
         (ai-papers.net). Sections cited: "Top-kとTop-pの限界を解剖する" (Top-k/Top-p
         limits, Fig. 2 uniform PP, Fig. 3 skewed PP) and "ハイブリッドマスキングと蒸留微調整"
         (hybrid masking).
* [SVG2] "Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via
         Semantic-Aware Permutation" (gist.science summary). Sections cited: "1. 問題定義"
         (positional blocks of consecutive tokens, mean/max pooled representatives) and
         "2. 手法" B (centroid scores, sort, accumulate until the threshold p is reached) and
         A (permutation equivalence).
* [SPR]  "Partition the Support, Reconstruct the Residual: Training-Free Sparse Attention for
         Video Generation and World Models" (physicalainews.jp), original abstract: queries that
         share a block route share one key-block support; executed-pair density.

What is computed, step by step (all arithmetic in float64 on the exact stored input values):

1. Partition the token axis into consecutive blocks of ``bq`` queries and ``bk`` keys; the last
   block of each may be partial.
2. Mean-pool Q and K over the valid tokens of each block.
3. Pooled scores ``S = scale * <Qbar_i, Kbar_j>`` and a softmax over j for each query block i.
4. Order each row by descending probability, the lower block index first on exact equality.
5. Top-k keeps the first ``k = min(nKB, ceil(k_frac * nKB - 1e-9))`` entries of that order.
6. Top-p keeps the shortest prefix whose running sum reaches ``p`` (``>= p``); ``p <= 0`` keeps
   nothing and a running sum that never reaches ``p`` keeps the whole row.
7. The union of the two prefixes of one order is the longer prefix: ``L = max(k, m*)``.
8. Attention for every valid query of block i over exactly the keys of the kept blocks, written
   literally as dense scores with the dropped keys set to -inf followed by a softmax; an empty
   key set gives O = 0 and LSE = -inf.

Every function below is pinned by CPU tests against closed forms, library routines and brute
force; none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Window inside which two probabilities, or a running sum and p, count as tied when a GPU mask
# row is compared with this oracle's row.
TIE_TOL = 1e-6


def _as_f64(x) -> np.ndarray:
    """Upcast stored input values (fp32 or bf16 read back as fp32/fp64) to float64 exactly."""
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# Step 1 and 2: positional blocks and mean pooling  ([SVG2] "1. 問題定義")
# ---------------------------------------------------------------------------------------------

def num_blocks(n: int, bsz: int) -> int:
    """Number of consecutive-token blocks of size ``bsz`` that cover ``n`` tokens."""
    return -(-n // bsz)


def block_sizes(n: int, bsz: int) -> np.ndarray:
    """Valid token count of each block; only the last one can be short."""
    nb = num_blocks(n, bsz)
    return np.array([min(bsz, n - i * bsz) for i in range(nb)], dtype=np.int64)


def pool_blocks(x, bsz: int) -> np.ndarray:
    """Mean of the token rows of each consecutive block, over valid tokens only.

    ``x`` is ``[B, H, N, d]``; the result is ``[B, H, ceil(N / bsz), d]`` float64.
    Positional grouping of consecutive tokens with a mean-pooled representative is the block
    construction of [SVG2] "1. 問題定義"; mean (not max) pooling is the reading taken here.
    """
    x = _as_f64(x)
    b, h, n, d = x.shape
    nb = num_blocks(n, bsz)
    out = np.empty((b, h, nb, d), dtype=np.float64)
    for i in range(nb):
        lo, hi = i * bsz, min(n, (i + 1) * bsz)
        out[:, :, i, :] = x[:, :, lo:hi, :].mean(axis=2)
    return out


# ---------------------------------------------------------------------------------------------
# Step 3: pooled probability pattern (PP)  ([SA2] Fig. 2/3 "each row"; [SVG2] "2. 手法" B)
# ---------------------------------------------------------------------------------------------

def pooled_probabilities(q_pool, k_pool, scale: float) -> np.ndarray:
    """Row softmax of the scaled pooled scores: ``P[b,h,i,:] = softmax_j(scale * Qbar_i . Kbar_j)``.

    The probability pattern is estimated from block representatives instead of the full score
    matrix ([SVG2] "2. 手法" B); [SA2] visualises it per query row (Fig. 2, Fig. 3).
    """
    qp = _as_f64(q_pool)
    kp = _as_f64(k_pool)
    s = scale * np.matmul(qp, np.swapaxes(kp, -1, -2))
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------------------------
# Steps 4-7: Top-k, Top-p and their union  ([SA2] "Top-kとTop-pの限界を解剖する",
# "ハイブリッドマスキングと蒸留微調整"; [SVG2] "2. 手法" B)
# ---------------------------------------------------------------------------------------------

def topk_count(k_frac: float, nkb: int) -> int:
    """Top-k size from a kept fraction: ``min(nKB, ceil(k_frac * nKB - 1e-9))``.

    The ceiling keeps at least the requested fraction; the 1e-9 absorbs representation noise
    such as 0.25 * 16 landing a hair above 4.
    """
    if not (0.0 <= k_frac <= 1.0):
        raise ValueError("k_frac must lie in [0, 1]")
    return int(min(nkb, max(0, math.ceil(k_frac * nkb - 1e-9))))


def row_order(prob_row: np.ndarray) -> np.ndarray:
    """Block indices by descending probability; exact equality ranks the lower index first."""
    j = np.arange(prob_row.shape[0])
    return np.lexsort((j, -prob_row))


def topp_count(sorted_probs: np.ndarray, p: float) -> int:
    """Length of the shortest prefix of the descending order whose running sum is ``>= p``.

    [SA2] selects from the top until the cumulative probability passes p; [SVG2] "2. 手法" B
    selects until it reaches p. The inclusive reading (``>=``) is taken. ``p <= 0`` gives 0, and
    a running sum that never reaches ``p`` (possible only by rounding when p is near 1) keeps
    every block.
    """
    if p <= 0.0:
        return 0
    c = np.cumsum(sorted_probs)          # sequential left-to-right float64 sum
    hit = np.nonzero(c >= p)[0]
    return int(hit[0]) + 1 if hit.size else int(sorted_probs.shape[0])


def select_row(prob_row: np.ndarray, k: int, p: float):
    """Hybrid Top-k U Top-p for one query block.

    Both rules keep a prefix of the same descending order, so their union ([SA2] hybrid
    masking) is the longer prefix, of length ``max(k, m*)``. Returns (mask_row, order, m*, L).
    """
    order = row_order(prob_row)
    m_star = topp_count(prob_row[order], p)
    L = max(k, m_star)
    mask = np.zeros(prob_row.shape[0], dtype=np.uint8)
    mask[order[:L]] = 1
    return mask, order, m_star, L


def select_mask(probs, k_frac: float, p: float):
    """Block mask ``[B,H,nQB,nKB]`` (uint8, 1 = keep) plus per-row ``m*`` and ``L``."""
    probs = _as_f64(probs)
    nkb = probs.shape[-1]
    k = topk_count(k_frac, nkb)
    flat = probs.reshape(-1, nkb)
    mask = np.zeros(flat.shape, dtype=np.uint8)
    m_star = np.zeros(flat.shape[0], dtype=np.int64)
    length = np.zeros(flat.shape[0], dtype=np.int64)
    for r in range(flat.shape[0]):
        mask[r], _, m_star[r], length[r] = select_row(flat[r], k, p)
    shp = probs.shape[:-1]
    return mask.reshape(probs.shape), {"k": k, "m_star": m_star.reshape(shp), "L": length.reshape(shp)}


def block_mask(q, k, bq: int, bk: int, k_frac: float, p: float, scale: float | None = None):
    """Steps 1-7: pooled probability pattern and the hybrid mask for given Q and K."""
    d = np.shape(q)[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    probs = pooled_probabilities(pool_blocks(q, bq), pool_blocks(k, bk), scale)
    mask, info = select_mask(probs, k_frac, p)
    info["probs"] = probs
    return mask, info


# ---------------------------------------------------------------------------------------------
# Step 8: masked dense attention  ([SVG2] "2. 手法" C: sparse K/V, dense contiguous Q;
# [SPR] abstract: queries sharing a block route share its key support)
# ---------------------------------------------------------------------------------------------

def attend_block(q_blk, k_all, v_all, key_keep: np.ndarray, scale: float):
    """Softmax attention of the query rows ``q_blk`` over the keys where ``key_keep`` is True.

    Written literally: dense scores against every key, dropped keys set to -inf, then a softmax
    over the row. Returns (O ``[nq, d]``, LSE ``[nq]`` natural log). No kept key gives O = 0 and
    LSE = -inf.
    """
    q_blk = _as_f64(q_blk)
    s = scale * (q_blk @ _as_f64(k_all).T)
    s[:, ~key_keep] = -np.inf
    nq = q_blk.shape[0]
    dv = np.shape(v_all)[-1]
    if not key_keep.any():
        return np.zeros((nq, dv)), np.full(nq, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ _as_f64(v_all)) / l
    return o, (m + np.log(l))[:, 0]


def masked_attention(q, k, v, mask, bq: int, bk: int, scale: float | None = None, blocks=None):
    """Block-sparse attention output by its definition.

    Every query of block i attends to all keys of the key blocks j with ``mask[b,h,i,j] == 1``
    and to no other key; padded key positions past N do not exist. ``blocks`` is an optional
    iterable of ``(b, h, i)`` query blocks to compute (a sample); ``None`` computes all.
    Returns (O ``[B,H,N,d]`` float64, LSE ``[B,H,N]``); rows outside the sample are NaN.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nqb = num_blocks(n, bq)
    o = np.full((b_, h_, n, v.shape[-1]), np.nan)
    lse = np.full((b_, h_, n), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(b_) for h in range(h_) for i in range(nqb)]
    for (b, h, i) in blocks:
        lo, hi = i * bq, min(n, (i + 1) * bq)
        key_keep = np.repeat(np.asarray(mask[b, h, i], dtype=bool), bk)[:n]
        o[b, h, lo:hi], lse[b, h, lo:hi] = attend_block(q[b, h, lo:hi], k[b, h], v[b, h], key_keep, scale)
    return o, lse


def sparse_attention(q, k, v, bq: int, bk: int, k_frac: float, p: float, scale: float | None = None, blocks=None):
    """Steps 1-8 end to end. Returns (O, LSE, mask, info)."""
    mask, info = block_mask(q, k, bq, bk, k_frac, p, scale)
    o, lse = masked_attention(q, k, v, mask, bq, bk, scale, blocks)
    return o, lse, mask, info


def executed_flops(mask, n: int, bq: int, bk: int, d: int) -> int:
    """Executed (algorithmic) FLOPs of the kept pairs: ``4 d * sum nq(i) * nk(j)`` over kept (i, j).

    QK^T and PV each cost 2 d per (query, key) pair; only valid tokens of kept block pairs count,
    which is the executed-pair notion of [SPR]'s abstract.
    """
    nq = block_sizes(n, bq).astype(np.float64)
    nk = block_sizes(n, bk).astype(np.float64)
    m = np.asarray(mask, dtype=np.float64)
    return int(round(4 * d * float((m * nq[:, None] * nk[None, :]).sum())))


# ---------------------------------------------------------------------------------------------
# Comparison of a mask from elsewhere against the oracle's, with ties reported
# ---------------------------------------------------------------------------------------------

def _admissible_lengths(sorted_probs: np.ndarray, k: int, p: float, tol: float) -> set[int]:
    """Kept counts reachable when running sums within ``tol`` of ``p`` may fall either side."""
    nkb = sorted_probs.shape[0]
    if p <= 0.0:
        lo_m = hi_m = 0
    else:
        c = np.cumsum(sorted_probs)
        lo_hit = np.nonzero(c >= p - tol)[0]
        hi_hit = np.nonzero(c >= p + tol)[0]
        lo_m = int(lo_hit[0]) + 1 if lo_hit.size else nkb
        hi_m = int(hi_hit[0]) + 1 if hi_hit.size else nkb
    return {max(k, m) for m in range(lo_m, hi_m + 1)}


def compare_masks(probs, mask_ref, mask_test, k_frac: float, p: float, tol: float = TIE_TOL):
    """Classify every row of ``mask_test`` against the oracle's ``mask_ref``.

    A differing row is a *tie* when (a) its kept count equals ``max(k, m')`` for a Top-p count
    ``m'`` whose running sum lies within ``tol`` of ``p``, and (b) its kept set is a top set of
    that size up to probabilities within ``tol`` of each other (every kept probability is at
    least every dropped one minus ``tol``). Any other difference is a *mismatch*.
    Returns a dict of counts and the flat indices of tied and mismatched rows.
    """
    probs = _as_f64(probs)
    nkb = probs.shape[-1]
    k = topk_count(k_frac, nkb)
    pf = probs.reshape(-1, nkb)
    rf = np.asarray(mask_ref).reshape(-1, nkb).astype(bool)
    tf = np.asarray(mask_test).reshape(-1, nkb).astype(bool)
    diff_rows = np.nonzero((rf != tf).any(axis=1))[0]
    ties, mismatches = [], []
    for r in diff_rows:
        row = pf[r]
        order = row_order(row)
        kept = tf[r]
        cnt = int(kept.sum())
        ok_len = cnt in _admissible_lengths(row[order], k, p, tol)
        if cnt in (0, nkb):
            ok_set = True
        else:
            ok_set = row[kept].min() >= row[~kept].max() - tol
        (ties if (ok_len and ok_set) else mismatches).append(int(r))
    return {
        "rows": int(pf.shape[0]),
        "rows_equal": int(pf.shape[0] - diff_rows.size),
        "ties": len(ties),
        "mismatches": len(mismatches),
        "tie_rows": ties,
        "mismatch_rows": mismatches,
        "blocks_differing": int((rf != tf).sum()),
    }


def ambiguous_rows(probs, k_frac: float, p: float, tol: float = TIE_TOL) -> np.ndarray:
    """Flat indices of rows whose oracle mask sits within ``tol`` of a decision boundary."""
    probs = _as_f64(probs)
    nkb = probs.shape[-1]
    k = topk_count(k_frac, nkb)
    out = []
    for r, row in enumerate(probs.reshape(-1, nkb)):
        order = row_order(row)
        sp = row[order]
        lens = _admissible_lengths(sp, k, p, tol)
        L = max(k, topp_count(sp, p))
        near_tie = 0 < L < nkb and sp[L - 1] - sp[L] <= tol
        if len(lens) > 1 or near_tie:
            out.append(r)
    return np.array(out, dtype=np.int64)
