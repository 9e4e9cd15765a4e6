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
block j) pair satisfies the pattern: the block-granular cover of the token pattern, which is what
a block-sparse kernel can run. Here it is found by brute force over all token pairs.
"""

from __future__ import annotations

import numpy as np

from .oracle import block_sizes, masked_attention, num_blocks

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


def squad_attention(q, k, v, window: int, bq: int, bk: int, scale: float | None = None):
    """Two-pass SQuad composition ([SQ] "手法") on block masks:

    1. local pass: masked attention of (Q, K, V) with the local(w) block mask;
    2. global pass: in the window-transposed token order, where the tokens that share a position
       inside their window form contiguous runs of n / w, masked attention of (Q, K, O_local) with
       the local(n / w) block mask, i.e. the global(w) pattern, then the output is put back in
       raster order ([SVG2] "2. 手法" A).

    Returns (O, O_local); arrays are ``[B, H, N, d]`` float64."""
    n = np.shape(q)[-2]
    m_local = pattern_block_mask(LOCAL, n, bq, bk, window=window)
    shp = np.shape(q)[:2] + m_local.shape
    o_local, _ = masked_attention(q, k, v, np.broadcast_to(m_local, shp), bq, bk, scale)
    perm = window_transpose(n, window)
    m_glob = pattern_block_mask(LOCAL, n, bq, bk, window=n // window)
    qp, kp, vp = (np.asarray(x, dtype=np.float64)[..., perm, :] for x in (q, k, o_local))
    o_perm, _ = masked_attention(qp, kp, vp, np.broadcast_to(m_glob, shp), bq, bk, scale)
    o = np.empty_like(o_perm)
    o[..., perm, :] = o_perm
    return o, o_local


def block_density(mask: np.ndarray) -> float:
    return float(np.asarray(mask, dtype=np.float64).mean())


__all__ = ["LOCAL", "GLOBAL", "DIAG", "MULTIDIAG", "STRIPE", "token_pattern", "pattern_block_mask",
           "window_transpose", "squad_attention", "block_density", "block_sizes"]
