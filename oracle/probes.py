"""Plain CPU oracle for the probe-fitted residual correction (numpy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
``cpu_baseline`` leg of the benchmark may import or call this module. The product path never
does, and this module imports nothing from the GPU package.

Page: "Partition the Support, Reconstruct the Residual: Training-Free Sparse Attention for Video
Generation and World Models" (physicalainews.jp), original abstract: a small set of exact query
rows calibrates, for each call, an affine correction from the sparse output, within the output
subspace observed in the probe residuals.

Reading taken (the abstract gives no more detail beyond the subspace):

1. Probes: per (b, h), ``P`` query blocks at fixed, evenly spaced positions
   ``i_p = floor((p + 1/2) nQB' / P)``, p = 0..P-1, over the nQB' query blocks that are full.
2. Exact rows: dense softmax attention of the probe queries over all N keys, O_e.
3. Residual on the probe rows: R = O_e - O_s, where O_s is the sparse output.
4. Fit per (b, h): X = [O_s, 1] on the probe rows (m x (d+1)); the ridge least-squares map
   A_full = (X^T X + mu I)^-1 X^T R, with mu = ridge * trace(X^T X) / (d + 1).
5. Subspace: the output subspace observed in the probe residuals is the span of the top ``rank``
   right singular vectors V_r of R (the eigenvectors of R^T R of the ``rank`` largest eigenvalues,
   the lower index first on equal eigenvalues). The map is confined to it: A = A_full V_r V_r^T,
   which is also the ridge fit of the projected residual R V_r V_r^T. Every correction row
   [O, 1] A then lies in span(V_r); rank >= d leaves A_full unchanged. With m = P * Bq probe rows
   above d, the span of all residual rows is the whole space, so without a rank below d the
   constraint would restrict nothing.
6. Apply to every row of the head: O_c = O_s + [O_s, 1] A.
"""

from __future__ import annotations

import math

import numpy as np

from .oracle import _as_f64, attend_block, num_blocks


def probe_blocks(n: int, bq: int, probes: int) -> np.ndarray:
    """Query-block indices of the probes (step 1)."""
    nqb = num_blocks(n, bq)
    full = nqb if n % bq == 0 else max(nqb - 1, 1)
    return np.array([min(full - 1, int(math.floor((p + 0.5) * full / probes))) for p in range(probes)],
                    dtype=np.int64)


def probe_rows(n: int, bq: int, probes: int) -> np.ndarray:
    """Token rows of the probes, in probe order."""
    rows = [np.arange(i * bq, min(n, (i + 1) * bq)) for i in probe_blocks(n, bq, probes)]
    return np.concatenate(rows)


def exact_rows(q, k, v, rows, scale: float | None = None) -> np.ndarray:
    """Dense attention output of the given query rows of every (b, h) over all keys (step 2)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b_, h_, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.empty((b_, h_, len(rows), v.shape[-1]))
    keep = np.ones(n, dtype=bool)
    for b in range(b_):
        for h in range(h_):
            out[b, h], _ = attend_block(q[b, h, rows], k[b, h], v[b, h], keep, scale)
    return out


def residual_subspace(r, rank: int) -> np.ndarray:
    """V_r of step 5: the eigenvectors of R^T R (d x d) for its ``rank`` largest eigenvalues, as
    columns, in descending order of eigenvalue (lower index first on equal ones)."""
    r = _as_f64(r)
    evals, evecs = np.linalg.eigh(r.T @ r)
    order = sorted(range(len(evals)), key=lambda i: (-evals[i], i))
    return evecs[:, order[:rank]]


def fit_correction(o_sparse_rows, o_exact_rows, ridge: float, rank: int | None = None) -> np.ndarray:
    """A ``[B, H, d+1, d]`` of steps 4 and 5 from the probe rows of the sparse and exact outputs;
    ``rank`` None (or >= d) skips the projection."""
    xs, xe = _as_f64(o_sparse_rows), _as_f64(o_exact_rows)
    b_, h_, m, d = xs.shape
    a = np.empty((b_, h_, d + 1, d))
    for b in range(b_):
        for h in range(h_):
            x = np.concatenate([xs[b, h], np.ones((m, 1))], axis=1)
            r = xe[b, h] - xs[b, h]
            g = x.T @ x
            mu = ridge * np.trace(g) / (d + 1)
            a[b, h] = np.linalg.solve(g + mu * np.eye(d + 1), x.T @ r)
            if rank is not None and rank < d:
                vr = residual_subspace(r, rank)
                a[b, h] = a[b, h] @ (vr @ vr.T)
    return a


def apply_correction(o_sparse, a) -> np.ndarray:
    """Step 6 on every row: O_s + [O_s, 1] A."""
    o = _as_f64(o_sparse)
    a = _as_f64(a)
    return o + o @ a[:, :, :-1, :] + a[:, :, -1:, :]


def probe_corrected(q, k, v, o_sparse, bq: int, probes: int, ridge: float, scale: float | None = None,
                    rank: int | None = None):
    """Steps 1-6. Returns (O_c, A, probe rows, exact probe outputs)."""
    n = np.shape(q)[-2]
    rows = probe_rows(n, bq, probes)
    oe = exact_rows(q, k, v, rows, scale)
    a = fit_correction(_as_f64(o_sparse)[:, :, rows], oe, ridge, rank)
    return apply_correction(o_sparse, a), a, rows, oe


__all__ = ["probe_blocks", "probe_rows", "exact_rows", "residual_subspace", "fit_correction", "apply_correction",
           "probe_corrected"]
