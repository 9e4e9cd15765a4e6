"""Seeded synthetic Q/K/V generator (numpy RNG; no attention arithmetic lives here).

Recipe for head (b, h) of a workload, with ``rng = numpy.random.default_rng([seed, b, h])`` and
the draws taken in this order:

1. ``F``: white N(0, 1) noise on the latent grid ``[T, Y, X, d]``, smoothed by a separable
   Gaussian of widths ``sigma = (s_t, s_y, s_x)`` tokens (truncated at 3 sigma, reflecting
   borders), then standardised per channel over all tokens. Shared by Q and K, it makes nearby
   tokens attend to each other (the diagonal pattern that video attention maps show).
2. ``Q = F + 0.3 * N(0, 1)``, then ``K = F + 0.3 * N(0, 1)``, then ``V = N(0, 1)``, each
   ``[N, d]`` with tokens in (t, y, x) raster order.
3. Locality-plus-sink workloads: one key index ``s = rng.integers(N)`` gets ``K[s] *= 8``
   (a key every query attends to: the vertical-stripe / attention-sink pattern).
   Stress workload: heads in the first half scale Q and K by 0.05 (near-uniform rows); heads
   in the second half scale 4 distinct keys ``rng.choice(N, 4, replace=False)`` by 20
   (sink-dominated rows).
4. Cast to the storage type with round-to-nearest-even (torch ``.to``).

Heads are generated independently, so any subset of heads reproduces the same values.

Structured values (``make_inputs(..., smooth_v=True)``, used only for the quality figures of the
correction and permutation paths): ``V`` is instead a second field ``G``, drawn from its own
generator ``numpy.random.default_rng([seed, b, h, 1])`` and smoothed and standardised like ``F``
(independent of it), plus ``0.3 * N(0, 1)`` from the same generator. Q, K and the sinks are
unchanged. In a video DiT, V is a projection of the same spatially smooth hidden states as Q and
K, so nearby tokens carry similar values; the i.i.d. default is the harder case for any method
that reconstructs values from neighbours.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np
import torch
from scipy.ndimage import gaussian_filter1d

from .configs import Workload

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(w: Workload) -> torch.dtype:
    return _TORCH_DTYPE[w.dtype]


@lru_cache(maxsize=None)
def _smoother(n: int, sigma: float) -> np.ndarray:
    """The [n, n] matrix of a 1-D Gaussian blur with reflecting borders, truncated at 3 sigma.

    It is scipy's gaussian_filter1d applied to the identity, so ``M @ x`` equals that filter
    along the first axis of ``x``; applying it as a matrix lets BLAS do the work.
    """
    return gaussian_filter1d(np.eye(n, dtype=np.float64), sigma, axis=0, mode="reflect",
                             truncate=3.0).astype(np.float32)


def _blur(f: np.ndarray, sigma: tuple) -> np.ndarray:
    t, y, x, d = f.shape
    if sigma[0] > 0:
        f = np.matmul(_smoother(t, sigma[0]), f.reshape(t, y * x * d)).reshape(t, y, x, d)
    if sigma[1] > 0:
        f = np.matmul(_smoother(y, sigma[1])[None], f.reshape(t, y, x * d)).reshape(t, y, x, d)
    if sigma[2] > 0:
        f = np.matmul(_smoother(x, sigma[2])[None], f.reshape(t * y, x, d)).reshape(t, y, x, d)
    return f


def _head(w: Workload, b: int, h: int, smooth_v: bool = False):
    rng = np.random.default_rng([w.seed, b, h])
    t, y, x = w.grid
    n, d = w.tokens, w.head_dim
    f = _blur(rng.standard_normal((t, y, x, d)).astype(np.float32), w.sigma)
    f = f.reshape(n, d)
    f = (f - f.mean(axis=0, keepdims=True)) / f.std(axis=0, keepdims=True)
    q = f + np.float32(w.noise_std) * rng.standard_normal((n, d)).astype(np.float32)
    k = f + np.float32(w.noise_std) * rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    if smooth_v:
        rv = np.random.default_rng([w.seed, b, h, 1])
        g = _blur(rv.standard_normal((t, y, x, d)).astype(np.float32), w.sigma).reshape(n, d)
        g = (g - g.mean(axis=0, keepdims=True)) / g.std(axis=0, keepdims=True)
        v = g + np.float32(w.noise_std) * rv.standard_normal((n, d)).astype(np.float32)
    sinks = []
    if w.kind == "locality_sink":
        s = int(rng.integers(n))
        k[s] *= np.float32(w.sink_gain)
        sinks = [s]
    elif w.kind == "stress":
        if h < w.heads // 2:
            q *= np.float32(0.05)
            k *= np.float32(0.05)
        else:
            idx = rng.choice(n, 4, replace=False)
            k[idx] *= np.float32(20.0)
            sinks = sorted(int(i) for i in idx)
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    dt = torch_dtype(w)
    return (torch.from_numpy(q).to(dt), torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt), sinks)


def make_inputs(w: Workload, heads=None, threads: int | None = None, smooth_v: bool = False):
    """Q, K, V as CPU tensors ``[B, len(heads), N, d]`` of the workload's storage type.

    Returns a dict with ``q``, ``k``, ``v``, ``heads`` (the head indices generated) and
    ``sinks`` (per (b, head) the boosted key indices).
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    jobs = [(b, h) for b in range(w.batch) for h in heads]
    threads = threads or min(16, len(os.sched_getaffinity(0)), len(jobs))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        res = list(ex.map(lambda bh: _head(w, *bh, smooth_v=smooth_v), jobs))
    dt = torch_dtype(w)
    shape = (w.batch, len(heads), w.tokens, w.head_dim)
    q = torch.empty(shape, dtype=dt)
    k = torch.empty(shape, dtype=dt)
    v = torch.empty(shape, dtype=dt)
    sinks = {}
    for (b, h), (qh, kh, vh, s) in zip(jobs, res):
        hi = heads.index(h)
        q[b, hi], k[b, hi], v[b, hi] = qh, kh, vh
        sinks[(b, h)] = s
    return {"q": q, "k": k, "v": v, "heads": heads, "sinks": sinks}
