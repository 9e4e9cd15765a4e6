"""Plain CPU oracle for semantic-aware permutation with centroid Top-p (numpy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
``cpu_baseline`` leg of the benchmark may import or call this module. The product path never
does, and this module imports nothing from the GPU package.

Page: "Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via Semantic-Aware
Permutation" (gist.science summary), section "2. 手法": A (k-means clusters of Q and of K,
tokens permuted so that each cluster is contiguous, output mathematically equal to unpermuted
attention), B (scores between cluster centroids, clusters sorted by estimated score and taken
until the cumulative score reaches p) and C (attention over variable-size blocks: dense
contiguous queries, sparse key/value loads).

Readings taken where the page leaves a step open:

1. k-means is Lloyd's iteration on squared Euclidean distance. Without a warm start, centroid c
   starts at token ``floor((c + 1/2) N / C)`` (evenly spaced). Each iteration assigns every token
   to the nearest centroid (the lowest index on an exact tie; ``||mu||^2 - 2 <x, mu>`` is compared,
   which orders centroids as ``||x - mu||^2`` does), then moves each centroid to the mean of its
   tokens; a cluster left empty keeps its centroid. ``iters`` such iterations are run; the labels
   returned are those of the last assignment.
2. The permutation is the stable sort of tokens by cluster label; cluster c occupies
   ``[offsets[c], offsets[c + 1])`` of the permuted order.
3. The estimated attention mass of key cluster j for query cluster i is its share of a softmax in
   which every key of the cluster is replaced by the cluster centroid: ``n_j exp(S_ij)``
   normalised over j, with ``S_ij = scale <cq_i, ck_j>`` and ``n_j`` the cluster size (an empty
   cluster has no mass). Clusters are taken in descending order (lower index first on exact
   equality) until the running sum reaches p (``>= p``), and at least one is taken: the length
   kept is ``max(1, m*)``, the hybrid rule of the block path with a Top-k of 1. A cluster with no
   tokens has no mass and is never taken (when rounding keeps the running sum below p, the
   prefix stops at the last cluster with mass).
4. Every query of cluster i attends to exactly the keys of the key clusters kept for i.
"""

from __future__ import annotations

import math

import numpy as np

from .oracle import _as_f64, attend_block, row_order, topp_count


def init_centroids(x, C: int) -> np.ndarray:
    """Reading 1: centroid c = token floor((c + 1/2) N / C), per (b, h). ``x`` is [B, H, N, d]."""
    x = _as_f64(x)
    n = x.shape[2]
    idx = np.array([((2 * c + 1) * n) // (2 * C) for c in range(C)], dtype=np.int64)
    return x[:, :, idx].copy()


def kmeans_assign(x, mu) -> np.ndarray:
    """Label of every token: argmin over c of ||mu_c||^2 - 2 <x, mu_c> (lowest c on ties)."""
    x, mu = _as_f64(x), _as_f64(mu)
    dist = (mu * mu).sum(-1)[:, :, None, :] - 2.0 * np.einsum("bhnd,bhcd->bhnc", x, mu)
    return np.argmin(dist, axis=-1).astype(np.int64)   # argmin returns the first minimum


def kmeans_update(x, labels, mu_prev) -> np.ndarray:
    """Mean of each cluster's tokens; an empty cluster keeps its previous centroid."""
    x, mu = _as_f64(x), _as_f64(mu_prev).copy()
    b_, h_, _, _ = x.shape
    for b in range(b_):
        for h in range(h_):
            for c in range(mu.shape[2]):
                sel = labels[b, h] == c
                if sel.any():
                    mu[b, h, c] = x[b, h, sel].mean(axis=0)
    return mu


def kmeans(x, C: int, iters: int, init=None):
    """Reading 1 end to end. Returns (centroids [B,H,C,d], labels [B,H,N])."""
    mu = init_centroids(x, C) if init is None else _as_f64(init).copy()
    labels = None
    for _ in range(iters):
        labels = kmeans_assign(x, mu)
        mu = kmeans_update(x, labels, mu)
    return mu, labels


def kmeans_objective(x, mu, labels) -> float:
    """Sum of squared distances of every token to its centroid (what Lloyd's steps decrease)."""
    x, mu = _as_f64(x), _as_f64(mu)
    picked = np.take_along_axis(mu, labels[..., None].repeat(mu.shape[-1], -1), axis=2)
    return float(((x - picked) ** 2).sum())


def cluster_permutation(labels, C: int):
    """Reading 2: (perm [B,H,N], offsets [B,H,C+1]); perm[t'] is the original token at t'."""
    labels = np.asarray(labels)
    b_, h_, n = labels.shape
    perm = np.empty((b_, h_, n), dtype=np.int64)
    offsets = np.zeros((b_, h_, C + 1), dtype=np.int64)
    for b in range(b_):
        for h in range(h_):
            perm[b, h] = np.argsort(labels[b, h], kind="stable")
            offsets[b, h, 1:] = np.cumsum(np.bincount(labels[b, h], minlength=C))
    return perm, offsets


def cluster_probabilities(cq, ck, sizes, scale: float) -> np.ndarray:
    """Reading 3: ``n_j exp(S_ij)`` normalised over j, [B, H, Cq, Ck]."""
    cq, ck = _as_f64(cq), _as_f64(ck)
    s = scale * np.einsum("bhid,bhjd->bhij", cq, ck)
    n = np.asarray(sizes, dtype=np.float64)[:, :, None, :]
    s = np.where(n > 0, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    w = n * np.exp(s - m)
    return w / w.sum(axis=-1, keepdims=True)


def cluster_select(cq, ck, sizes, scale: float, p: float):
    """Reading 3: (mask uint8 [B,H,Cq,Ck], probabilities)."""
    probs = cluster_probabilities(cq, ck, sizes, scale)
    ck_n = probs.shape[-1]
    flat = probs.reshape(-1, ck_n)
    mask = np.zeros(flat.shape, dtype=np.uint8)
    for r in range(flat.shape[0]):
        order = row_order(flat[r])
        nonzero = int((flat[r] > 0).sum())
        mask[r, order[:min(nonzero, max(1, topp_count(flat[r][order], p)))]] = 1
    return mask.reshape(probs.shape), probs


def cluster_attention(q, k, v, labels_q, labels_k, mask, scale: float | None = None, clusters=None):
    """Reading 4, in the original token order: every query of cluster i over the keys whose
    cluster j has ``mask[b, h, i, j] == 1``. ``clusters`` optionally restricts the work to a
    sample of (b, h, i); rows outside it are NaN. Returns (O [B,H,N,d], LSE [B,H,N])."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = np.full((b_, h_, n, v.shape[-1]), np.nan)
    lse = np.full((b_, h_, n), np.nan)
    if clusters is None:
        clusters = [(b, h, i) for b in range(b_) for h in range(h_) for i in range(mask.shape[2])]
    for (b, h, i) in clusters:
        rows = np.nonzero(labels_q[b, h] == i)[0]
        if rows.size == 0:
            continue
        keep = np.asarray(mask[b, h, i], dtype=bool)[labels_k[b, h]]
        o[b, h, rows], lse[b, h, rows] = attend_block(q[b, h, rows], k[b, h], v[b, h], keep, scale)
    return o, lse


def svg2_attention(q, k, v, Cq: int, Ck: int, iters: int, p: float, scale: float | None = None):
    """Readings 1-4 end to end. Returns (O, LSE, info)."""
    d = np.shape(q)[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    mq, lq = kmeans(q, Cq, iters)
    mk, lk = kmeans(k, Ck, iters)
    _, ok = cluster_permutation(lk, Ck)
    mask, probs = cluster_select(mq, mk, np.diff(ok, axis=-1), scale, p)
    o, lse = cluster_attention(q, k, v, lq, lk, mask, scale)
    return o, lse, {"labels_q": lq, "labels_k": lk, "centroids_q": mq, "centroids_k": mk, "mask": mask,
                    "probs": probs}


__all__ = ["init_centroids", "kmeans_assign", "kmeans_update", "kmeans", "kmeans_objective",
           "cluster_permutation", "cluster_probabilities", "cluster_select", "cluster_attention",
           "svg2_attention"]
