"""Plain CPU oracle for the gradients of block-sparse attention (numpy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
``cpu_baseline`` leg of the benchmark may import or call this module. The product path never
does, and this module imports nothing from the GPU package.

Why it exists: the SpargeAttention2 page ("SpargeAttention2とは？..." on ai-papers.net, section
"ハイブリッドマスキングと蒸留微調整") fine-tunes the sparse model by distillation, which needs the
gradients of the block-sparse attention with respect to Q, K and V for the same mask.

What is computed, for every query token t of query block i, over the keys u of the kept key
blocks of row i (the forward's definition), with s = scale * <Q_t, K_u>, P = softmax_u(s),
O_t = sum_u P_u V_u and an upstream gradient dO:

    dV_u  += P_tu * dO_t
    dP_tu  = <dO_t, V_u>
    dS_tu  = P_tu * (dP_tu - sum_u' P_tu' dP_tu')        (the softmax Jacobian)
    dQ_t   = scale * sum_u dS_tu K_u
    dK_u  += scale * dS_tu Q_t

A query block with no kept key block contributes nothing (its O is 0 and does not depend on the
inputs); keys of blocks no query block keeps get zero gradients.
"""

from __future__ import annotations

import math

import numpy as np

from .oracle import _as_f64, num_blocks


def masked_attention_bwd(q, k, v, mask, dout, bq: int, bk: int, scale: float | None = None,
                         q_blocks=None, k_blocks=None):
    """(dQ, dK, dV) ``[B, H, N, d]`` float64 of the block-masked attention, by the definition
    above, one query block at a time with dense scores and dropped keys set to -inf.

    ``q_blocks`` / ``k_blocks`` optionally restrict the work to a sample: lists of (b, h, i) query
    blocks whose dQ rows and of (b, h, j) key blocks whose dK / dV rows are wanted (the query
    blocks that keep a sampled key block are then visited as needed). Rows outside the sample
    are NaN; with both None everything is computed."""
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nqb, nkb = num_blocks(n, bq), num_blocks(n, bk)
    full = q_blocks is None and k_blocks is None
    dq = np.zeros_like(q) if full else np.full_like(q, np.nan)
    dk = np.zeros_like(k) if full else np.full_like(k, np.nan)
    dv = np.zeros_like(v) if full else np.full_like(v, np.nan)
    want_q = set(q_blocks or [])
    want_k = set(k_blocks or [])
    for (b, h, j) in want_k:
        dk[b, h, j * bk:(j + 1) * bk] = 0.0
        dv[b, h, j * bk:(j + 1) * bk] = 0.0
    for b in range(b_):
        for h in range(h_):
            for i in range(nqb):
                row = np.asarray(mask[b, h, i], dtype=bool)
                need_q = full or (b, h, i) in want_q
                need_k = full or any(row[j] and (b, h, j) in want_k for j in range(nkb))
                lo, hi = i * bq, min(n, (i + 1) * bq)
                if need_q and not full:
                    dq[b, h, lo:hi] = 0.0
                keep = np.repeat(row, bk)[:n]
                if not (need_q or need_k) or not keep.any():
                    continue
                s = scale * (q[b, h, lo:hi] @ k[b, h].T)
                s[:, ~keep] = -np.inf
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                g = dout[b, h, lo:hi]
                dp = g @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                if need_q:
                    dq[b, h, lo:hi] = scale * (ds @ k[b, h])
                if full:
                    dv[b, h] += p.T @ g
                    dk[b, h] += scale * (ds.T @ q[b, h, lo:hi])
                elif need_k:
                    for j in range(nkb):
                        if row[j] and (b, h, j) in want_k:
                            kl, kh = j * bk, min(n, (j + 1) * bk)
                            dv[b, h, kl:kh] += p[:, kl:kh].T @ g
                            dk[b, h, kl:kh] += scale * (ds[:, kl:kh].T @ q[b, h, lo:hi])
    return dq, dk, dv


def masked_attention_bwd_scales(q, k, v, mask, dout, bq: int, bk: int, scale: float | None = None,
                                q_blocks=None, k_blocks=None):
    """Elementwise error scales of the three gradients: the same products with every term replaced
    by its absolute value, the standard forward-error scale of a sum of products, plus the
    spread of a relative error in D = rowsum(dO * O) through dS:

        dQ:  scale * (|dS| |K| + (P * e) |K|),   dK:  scale * (|dS|^T |Q| + (P * e)^T |Q|),
        dV:  P^T |dO|,                            with e_t = sum_c |dO_tc O_tc|.

    Same arguments, sampling and NaN convention as masked_attention_bwd."""
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nqb, nkb = num_blocks(n, bq), num_blocks(n, bk)
    full = q_blocks is None and k_blocks is None
    sq = np.zeros_like(q) if full else np.full_like(q, np.nan)
    sk = np.zeros_like(k) if full else np.full_like(k, np.nan)
    sv = np.zeros_like(v) if full else np.full_like(v, np.nan)
    want_q = set(q_blocks or [])
    want_k = set(k_blocks or [])
    for (b, h, j) in want_k:
        sk[b, h, j * bk:(j + 1) * bk] = 0.0
        sv[b, h, j * bk:(j + 1) * bk] = 0.0
    for b in range(b_):
        for h in range(h_):
            ak, aq = np.abs(k[b, h]), np.abs(q[b, h])
            for i in range(nqb):
                row = np.asarray(mask[b, h, i], dtype=bool)
                need_q = full or (b, h, i) in want_q
                need_k = full or any(row[j] and (b, h, j) in want_k for j in range(nkb))
                lo, hi = i * bq, min(n, (i + 1) * bq)
                if need_q and not full:
                    sq[b, h, lo:hi] = 0.0
                keep = np.repeat(row, bk)[:n]
                if not (need_q or need_k) or not keep.any():
                    continue
                s = scale * (q[b, h, lo:hi] @ k[b, h].T)
                s[:, ~keep] = -np.inf
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                g = dout[b, h, lo:hi]
                o = p @ v[b, h]
                dp = g @ v[b, h].T
                ds = np.abs(p * (dp - (p * dp).sum(axis=1, keepdims=True)))
                pe = p * np.abs(g * o).sum(axis=1, keepdims=True)
                if need_q:
                    sq[b, h, lo:hi] = scale * ((ds + pe) @ ak)
                cols = range(nkb) if full else [j for j in range(nkb) if row[j] and (b, h, j) in want_k]
                for j in cols:
                    if not row[j]:
                        continue
                    kl, kh = j * bk, min(n, (j + 1) * bk)
                    sv[b, h, kl:kh] += p[:, kl:kh].T @ np.abs(g)
                    sk[b, h, kl:kh] += scale * ((ds + pe)[:, kl:kh].T @ aq[lo:hi])
    return sq, sk, sv


__all__ = ["masked_attention_bwd", "masked_attention_bwd_scales"]
