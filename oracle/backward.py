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


def masked_attention_bwd(q, k, v, mask, dout, bq: int, bk: int, scale: float | None = None):
    """(dQ, dK, dV) ``[B, H, N, d]`` float64 of the block-masked attention, by the definition
    above, one query block at a time with dense scores and dropped keys set to -inf."""
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(h_):
            for i in range(num_blocks(n, bq)):
                keep = np.repeat(np.asarray(mask[b, h, i], dtype=bool), bk)[:n]
                if not keep.any():
                    continue
                lo, hi = i * bq, min(n, (i + 1) * bq)
                s = scale * (q[b, h, lo:hi] @ k[b, h].T)
                s[:, ~keep] = -np.inf
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                g = dout[b, h, lo:hi]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, lo:hi] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, lo:hi])
    return dq, dk, dv


__all__ = ["masked_attention_bwd"]
