"""Plain CPU oracle for fixed-pattern block masks and the two-pass SQuad composition (numpy,
float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
``cpu_baseline`` leg of the benchmark may import or call this module. The product path never
does, and this module imports nothing from the GPU package.

Pages this follows:

* [SQ]  "SQuad: Sub-Quadratic Attention Distillation for Efficient Video Generation"
        (gist.science), section "手法" (SQuad attention operator): a local pass mixes tokens
        inside fixed windows of w tokens; a global pass mixes, across all windows, the tokens at
        the same relative position inside their window; the local pass's output is the value
        stream of the global pass.
* [SVD] "Sparse-vDiT: Unleashing the Power of Sparse Attention to Accelerate Video Diffusion
        Transformers" (aibr.jp), section "3. 中核となる技術的要素": diagonal, multi-diagonal and
        vertical-stripe attention patterns.
* [SVG2] "Sparse VideoGen2" (gist.science), "2. 手法" A: permuting tokens, with the outputs
        permuted back, leaves attention unchanged.

Token-level patterns (t a query token, u a key token, all indices 0-based in raster order):

* local(w):          floor(t / w) == floor(u / w)
* global(w):         t mod w == u mod w
* diagonal(b):       |t - u| <= b
* multi-diagonal(b, P): the distance from t - u to the nearest multiple of P is <= b
* stripe(P):         u mod P == 0 (every query sees the key tokens that start a period)

A block mask keeps block pair (i, j) when at least one (query token of block i, key token of
block j) pair satisfies the pattern: the block-granular cover of the token pattern, i.e. the
tiles a block-sparse kernel visits. Here it is found by brute force over all token pairs.

The SQuad operator itself is token-exact: each pass attends over exactly the key tokens its
token pattern admits (``squad_local``, ``squad_global``), never over a block cover.
"""

from __future__ import annotations

import math

import numpy as np

from .oracle import attend_block, block_sizes, num_blocks

LOCAL, GLOBAL, DIAG, MULTIDIAG, STRIPE = 1, 2, 4, 8, 16


def token_pattern(kinds: int, t: np.ndarray, u: np.ndarray, window: int = 0, band: int = 0,
                  period: int = 0) -> np.ndarray:
    """Union of the selected token-level patterns for query tokens t and key tokens u
    (broadcasting arrays of int64)."""
    t = np.asarray(t, dtype=np.int64)
    u = np.asarray(u, dtype=np.int64)
    keep = np.zeros(np.broadcast(t, u).shape, dtype=bool)
    if kinds & LOCAL:
        keep |= (t // window) == (u // window)
    if kinds & GLOBAL:
        keep |= (t % window) == (u % window)
    if kinds & DIAG:
        keep |= np.abs(t - u) <= band
    if kinds & MULTIDIAG:
        r = np.mod(t - u, period)
        keep |= np.minimum(r, period - r) <= band
    if kinds & STRIPE:
        keep |= np.broadcast_to((u % period) == 0, keep.shape)
    return keep


def pattern_block_mask(kinds: int, n: int, bq: int, bk: int, window: int = 0, band: int = 0,
                       period: int = 0, rows=None) -> np.ndarray:
    """Block mask ``[nQB, nKB]`` (uint8) of the pattern union, by brute force over token pairs.
    ``rows`` restricts the work to some query blocks (the other rows are returned as 0)."""
    nqb, nkb = num_blocks(n, bq), num_blocks(n, bk)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    u = np.arange(n, dtype=np.int64)
    kblk = u // bk
    for i in (range(nqb) if rows is None else rows):
        t = np.arange(i * bq, min(n, (i + 1) * bq), dtype=np.int64)
        hit = token_pattern(kinds, t[:, None], u[None, :], window, band, period).any(axis=0)
        out[i, np.unique(kblk[hit])] = 1
    return out


def window_transpose(n: int, w: int) -> np.ndarray:
    """perm with x_perm[s] = x[perm[s]]: the tokens at the same position r inside their w-token
    window become contiguous (s = r * (n / w) + m holds token m * w + r). Needs w | n."""
    if n % w:
        raise ValueError("the window must divide the token count")
    nw = n // w
    s = np.arange(n, dtype=np.int64)
    return (s % nw) * w + s // nw


def _attend_set(q_rows, k_rows, v_rows, scale: float):
    """Softmax attention of every query row over exactly the given key rows: the pattern admits
    those keys and no other, so this is the masked dense row with the other keys at -inf (their
    exponentials are exactly zero). Returns (O, LSE natural log)."""
    return attend_block(q_rows, k_rows, v_rows, np.ones(np.shape(k_rows)[0], dtype=bool), scale)


def squad_local(q, k, v, window: int, scale: float | None = None, windows=None):
    """SQuad local pass ([SQ] "手法", "1. SQuad アテンション・オペレーター"): token t attends to
    the tokens u of its own window of ``window`` consecutive raster tokens, floor(t / w) ==
    floor(u / w); the last window is partial when w does not divide N.

    ``windows`` optionally restricts the work to some window indices (other rows stay NaN).
    Returns (O, LSE), ``[B, H, N, d]`` and ``[B, H, N]`` float64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = np.full((b_, h_, n, v.shape[-1]), np.nan)
    lse = np.full((b_, h_, n), np.nan)
    nwin = -(-n // window)
    for b in range(b_):
        for h in range(h_):
            for c in (range(nwin) if windows is None else windows):
                rows = slice(c * window, min(n, (c + 1) * window))
                o[b, h, rows], lse[b, h, rows] = _attend_set(q[b, h, rows], k[b, h, rows], v[b, h, rows], scale)
    return o, lse


def squad_global(q, k, v, window: int, scale: float | None = None, positions=None):
    """SQuad global pass ([SQ] "手法"): token t attends to the tokens u at the same relative
    position inside their windows, t mod w == u mod w, across all windows.

    ``positions`` optionally restricts the work to some positions r in [0, w) (the rows t with
    t mod w == r; other rows stay NaN). Returns (O, LSE) as ``squad_local``."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = np.full((b_, h_, n, v.shape[-1]), np.nan)
    lse = np.full((b_, h_, n), np.nan)
    for b in range(b_):
        for h in range(h_):
            for r in (range(min(window, n)) if positions is None else positions):
                rows = np.arange(r, n, window)
                o[b, h, rows], lse[b, h, rows] = _attend_set(q[b, h, rows], k[b, h, rows], v[b, h, rows], scale)
    return o, lse


def squad_attention(q, k, v, window: int, scale: float | None = None, positions=None):
    """Two-pass SQuad operator ([SQ] "手法"): the local pass of (Q, K, V), then the global pass
    of (Q, K, O_local): the local output is the global pass's value stream; queries and keys
    are the same in both passes (the distilled projections are out of scope).

    The local pass is computed for every window, since each position class takes one token from
    every window. ``positions`` restricts the global pass (a sample). Returns
    (O, O_local, LSE, LSE_local) in float64."""
    o_local, lse_local = squad_local(q, k, v, window, scale)
    o, lse = squad_global(q, k, o_local, window, scale, positions)
    return o, o_local, lse, lse_local


def squad_pairs(n: int, window: int) -> int:
    """(query, key) token pairs the two SQuad passes attend over: the squared window lengths plus
    the squared position-class sizes. N w + N^2 / w when w divides N."""
    wl = np.array([min(window, n - c * window) for c in range(-(-n // window))], dtype=np.int64)
    pc = np.array([len(range(r, n, window)) for r in range(min(window, n))], dtype=np.int64)
    return int((wl * wl).sum() + (pc * pc).sum())


def block_density(mask: np.ndarray) -> float:
    return float(np.asarray(mask, dtype=np.float64).mean())


__all__ = ["LOCAL", "GLOBAL", "DIAG", "MULTIDIAG", "STRIPE", "token_pattern", "pattern_block_mask",
           "window_transpose", "squad_local", "squad_global", "squad_attention", "squad_pairs", "block_density",
           "block_sizes"]
