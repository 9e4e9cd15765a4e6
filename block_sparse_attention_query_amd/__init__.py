"""Block-sparse attention in the SpargeAttention2 form for MI355X (gfx950).

Thin torch binding over the C ABI in ``include/sparse_attn.h``: it checks tensor placement and
layout, allocates outputs with torch, and passes raw device pointers and torch's current HIP
stream. Every step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and a missing library raises.

    q_pool, k_pool = pool_qk(q, k, bq, bk)
    sel = select_mask(q_pool, k_pool, k_frac, p)          # probs, mask (+ kept lists)
    o = fwd(q, k, v, sel["mask"], bq, bk)
"""

from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (SA_BF16, SA_F32, SA_PAT_DIAG, SA_PAT_GLOBAL, SA_PAT_LOCAL, SA_PAT_MULTIDIAG,  # noqa: F401
                   SA_PAT_STRIPE, SA_SELECT_FUSED_NKB, SparseAttnError)

SELECT_FUSED_NKB = SA_SELECT_FUSED_NKB

__all__ = ["pool_qk", "select_mask", "fwd", "fwd_noalloc", "fwd_lists", "row_order", "fwd_workspace_size", "bwd", "bwd_workspace_size",
           "pattern_mask",
           "window_transpose", "squad_fwd", "squad_attention", "topk_count", "sparse_attention", "probe_correct",
           "probe_workspace_size", "kmeans", "cluster_select", "permute_rows", "cluster_fwd", "svg2_attention",
           "SparseAttnError"]

_DTYPES = {torch.bfloat16: SA_BF16, torch.float32: SA_F32}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_qkv(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dim() != 4:
            raise ValueError("expected [B, H, N, d] tensors")
        if t.dtype != ts[0].dtype or t.shape != ts[0].shape or t.device != ts[0].device:
            raise ValueError("q, k, v must share dtype, shape and device")
    if ts[0].dtype not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")


def _nblocks(n: int, b: int) -> int:
    return -(-n // b)


def topk_count(k_frac: float, nkb: int) -> int:
    """Top-k size the library uses for a kept fraction (host arithmetic of the C ABI)."""
    return int(_lib.lib().sparse_attn_topk_count(float(k_frac), int(nkb)))


def _check_out(t: torch.Tensor, shape, dtype, device) -> torch.Tensor:
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != device:
        raise ValueError(f"output buffer must be a contiguous {dtype} {list(shape)} tensor on {device}")
    return t


def pool_qk(q: torch.Tensor, k: torch.Tensor, bq: int, bk: int, out=None):
    """Mean-pooled Q over blocks of ``bq`` and K over blocks of ``bk`` (float64 outputs).

    ``out`` may pass preallocated ``(q_pool, k_pool)`` buffers.
    """
    _check_qkv(q, k)
    B, H, N, d = q.shape
    qshape, kshape = (B, H, _nblocks(N, bq), d), (B, H, _nblocks(N, bk), d)
    if out is None:
        qp = torch.empty(qshape, dtype=torch.float64, device=q.device)
        kp = torch.empty(kshape, dtype=torch.float64, device=q.device)
    else:
        qp = _check_out(out[0], qshape, torch.float64, q.device)
        kp = _check_out(out[1], kshape, torch.float64, q.device)
    _lib.check(_lib.lib().sparse_attn_pool_qk(q.data_ptr(), k.data_ptr(), _DTYPES[q.dtype], B, H, N, d, bq, bk,
                                              qp.data_ptr(), kp.data_ptr(), _stream(q)))
    return qp, kp


def select_mask(q_pool: torch.Tensor, k_pool: torch.Tensor, k_frac: float, p: float, scale: float | None = None,
                kept_lists: bool = False, out: dict | None = None, probs: bool = True):
    """Pooled probabilities and the hybrid Top-k U Top-p block mask.

    Returns a dict with ``probs`` (float64 ``[B,H,nQB,nKB]``, left out when ``probs`` is False,
    which rows of at most SA_SELECT_FUSED_NKB key blocks allow), ``mask`` (uint8) and, when
    ``kept_lists`` is set, ``kept_idx`` / ``kept_cnt`` (int32). ``out`` may pass a dict of
    preallocated buffers under the same keys.
    """
    for t in (q_pool, k_pool):
        if not t.is_cuda or t.dtype != torch.float64 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("pooled tensors must be contiguous float64 [B, H, n, d] GPU tensors")
    B, H, nqb, d = q_pool.shape
    nkb = k_pool.shape[2]
    if k_pool.shape[:2] != (B, H) or k_pool.shape[3] != d:
        raise ValueError("q_pool and k_pool shapes disagree")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q_pool.device
    want = {"mask": ((B, H, nqb, nkb), torch.uint8)}
    if probs:
        want["probs"] = ((B, H, nqb, nkb), torch.float64)
    if kept_lists:
        want["kept_idx"] = ((B, H, nqb, nkb), torch.int32)
        want["kept_cnt"] = ((B, H, nqb), torch.int32)
    given = out or {}
    out = {name: (_check_out(given[name], shp, dt, dev) if name in given else torch.empty(shp, dtype=dt, device=dev))
           for name, (shp, dt) in want.items()}
    probs_ptr = out["probs"].data_ptr() if probs else None
    mask = out["mask"]
    idx_ptr = cnt_ptr = None
    if kept_lists:
        idx_ptr, cnt_ptr = out["kept_idx"].data_ptr(), out["kept_cnt"].data_ptr()
    _lib.check(_lib.lib().sparse_attn_select_mask(q_pool.data_ptr(), k_pool.data_ptr(), B, H, nqb, nkb, d, scale,
                                                  float(k_frac), float(p), probs_ptr, mask.data_ptr(),
                                                  idx_ptr, cnt_ptr, _stream(q_pool)))
    return out


def fwd_workspace_size(B: int, H: int, N: int, bq: int, bk: int = 64) -> int:
    return int(_lib.lib().sparse_attn_fwd_workspace_size(B, H, N, bq, bk))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor, bq: int, bk: int = 64,
        scale: float | None = None, return_lse: bool = False, workspace: torch.Tensor | None = None,
        out: torch.Tensor | None = None):
    """Block-sparse attention of each query block over its kept key blocks."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    nqb, nkb = _nblocks(N, bq), _nblocks(N, bk)
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (B, H, nqb, nkb) or not mask.is_contiguous() \
            or mask.device != q.device:
        raise ValueError(f"mask must be a contiguous uint8 [{B}, {H}, {nqb}, {nkb}] tensor on {q.device}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ws_bytes = fwd_workspace_size(B, H, N, bq, bk)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    _lib.check(_lib.lib().sparse_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype],
                                          mask.data_ptr(), B, H, N, d, bq, bk, scale, o.data_ptr(),
                                          None if lse is None else lse.data_ptr(), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, lse) if return_lse else o


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor, bq: int, bk: int = 64,
                scale: float | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """``fwd`` through the entry point that allocates nothing on the device (its kept lists live
    in a scratch array inside the library). Pass ``out`` (and ``lse``) to allocate nothing here
    either; returns (o, lse)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    nqb, nkb = _nblocks(N, bq), _nblocks(N, bk)
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (B, H, nqb, nkb) or not mask.is_contiguous() \
            or mask.device != q.device:
        raise ValueError(f"mask must be a contiguous uint8 [{B}, {H}, {nqb}, {nkb}] tensor on {q.device}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out(lse, (B, H, N), torch.float32, q.device)
    _lib.check(_lib.lib().sparse_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype],
                                                  mask.data_ptr(), B, H, N, d, bq, bk, scale, o.data_ptr(),
                                                  None if lse is None else lse.data_ptr(), _stream(q)))
    return o, lse


def row_order(kept_cnt: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Work order of the attention rows for ``fwd_lists(..., row_order=...)`` (int32, one entry
    per row of ``kept_cnt``): longest lists first within each XCD on short grids, the kernels'
    default order otherwise. Scheduling only."""
    if kept_cnt.dtype != torch.int32 or kept_cnt.dim() != 3 or not kept_cnt.is_contiguous() or not kept_cnt.is_cuda:
        raise ValueError("kept_cnt must be a contiguous int32 [B, H, nqb] device tensor")
    B, H, nqb = kept_cnt.shape
    order = torch.empty(B * H * nqb, dtype=torch.int32, device=kept_cnt.device) if out is None else \
        _check_out(out, (B * H * nqb,), torch.int32, kept_cnt.device)
    _lib.check(_lib.lib().sparse_attn_row_order(kept_cnt.data_ptr(), B, H, nqb, order.data_ptr(), _stream(kept_cnt)))
    return order


def fwd_lists(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kept_idx: torch.Tensor, kept_cnt: torch.Tensor,
              bq: int, bk: int = 64, scale: float | None = None, return_lse: bool = False,
              out: torch.Tensor | None = None, window: int | None = None, row_order: torch.Tensor | None = None):
    """Block-sparse attention from kept-block lists (as written by ``select_mask(kept_lists=True)``).

    With ``window``, the attention runs over the window-transposed token order (the lists index
    its blocks) while q, k, v and the output stay in the original order: the same result as
    ``window_transpose`` of the inputs, ``fwd_lists`` and the inverse transpose of the output.
    ``row_order`` (from ``row_order``) sets the rows' work order; the result is unchanged."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    nqb, nkb = _nblocks(N, bq), _nblocks(N, bk)
    if kept_idx.dtype != torch.int32 or tuple(kept_idx.shape) != (B, H, nqb, nkb) or not kept_idx.is_contiguous():
        raise ValueError(f"kept_idx must be a contiguous int32 [{B}, {H}, {nqb}, {nkb}] tensor")
    if kept_cnt.dtype != torch.int32 or tuple(kept_cnt.shape) != (B, H, nqb) or not kept_cnt.is_contiguous():
        raise ValueError(f"kept_cnt must be a contiguous int32 [{B}, {H}, {nqb}] tensor")
    if kept_idx.device != q.device or kept_cnt.device != q.device:
        raise ValueError("kept lists must be on the device of q")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    if row_order is not None:
        if window is not None:
            raise ValueError("row_order applies to the plain token order only")
        if row_order.dtype != torch.int32 or tuple(row_order.shape) != (B * H * nqb,) or \
                not row_order.is_contiguous() or row_order.device != q.device:
            raise ValueError(f"row_order must be a contiguous int32 [{B * H * nqb}] tensor on the device of q")
        _lib.check(_lib.lib().sparse_attn_fwd_lists_ordered(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype], kept_idx.data_ptr(), kept_cnt.data_ptr(),
            row_order.data_ptr(), B, H, N, d, bq, bk, scale, o.data_ptr(), None if lse is None else lse.data_ptr(),
            _stream(q)))
    elif window is None:
        _lib.check(_lib.lib().sparse_attn_fwd_lists(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype], kept_idx.data_ptr(), kept_cnt.data_ptr(), B,
            H, N, d, bq, bk, scale, o.data_ptr(), None if lse is None else lse.data_ptr(), _stream(q)))
    else:
        _lib.check(_lib.lib().sparse_attn_fwd_lists_window(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype], kept_idx.data_ptr(), kept_cnt.data_ptr(), B,
            H, N, d, bq, bk, int(window), scale, o.data_ptr(), None if lse is None else lse.data_ptr(), _stream(q)))
    return (o, lse) if return_lse else o


def sparse_attention(q, k, v, bq: int, bk: int, k_frac: float, p: float, scale: float | None = None):
    """Pooling, mask selection and sparse attention in sequence; returns (o, mask)."""
    qp, kp = pool_qk(q, k, bq, bk)
    sel = select_mask(qp, kp, k_frac, p, scale)
    return fwd(q, k, v, sel["mask"], bq, bk, scale), sel["mask"]


def pattern_mask(patterns: int, B: int, H: int, N: int, bq: int, bk: int = 64, window: int = 0, band: int = 0,
                 period: int = 0, kept_lists: bool = True, device="cuda", out: dict | None = None):
    """Block mask (and kept lists) of a union of fixed patterns (SA_PAT_* flags)."""
    nqb, nkb = _nblocks(N, bq), _nblocks(N, bk)
    dev = torch.device(device)
    out = {} if out is None else out
    mask = out.get("mask")
    if mask is None:
        mask = out["mask"] = torch.empty((B, H, nqb, nkb), dtype=torch.uint8, device=dev)
    else:
        _check_out(mask, (B, H, nqb, nkb), torch.uint8, dev)
    idx_ptr = cnt_ptr = None
    if kept_lists:
        if out.get("kept_idx") is None:
            out["kept_idx"] = torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=dev)
            out["kept_cnt"] = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
        idx_ptr, cnt_ptr = out["kept_idx"].data_ptr(), out["kept_cnt"].data_ptr()
    _lib.check(_lib.lib().sparse_attn_pattern_mask(int(patterns), int(window), int(band), int(period), B, H, N, bq,
                                                   bk, mask.data_ptr(), idx_ptr, cnt_ptr, _stream(mask)))
    return out


def window_transpose(x: torch.Tensor, window: int, inverse: bool = False, out: torch.Tensor | None = None):
    """Token-axis window transpose of a [B, H, N, d] tensor (the tokens at one position inside
    their window become contiguous; ``inverse`` undoes it)."""
    _check_qkv(x)
    B, H, N, d = x.shape
    o = torch.empty_like(x) if out is None else _check_out(out, x.shape, x.dtype, x.device)
    _lib.check(_lib.lib().sparse_attn_window_transpose(x.data_ptr(), _DTYPES[x.dtype], B, H, N, d, int(window),
                                                       int(bool(inverse)), o.data_ptr(), _stream(x)))
    return o


def squad_masks(B: int, H: int, N: int, window: int, bq: int, bk: int = 64, device="cuda"):
    """Block covers of the two SQuad token patterns as kept lists (the local windows in raster
    order; the runs of N / window in the window-transposed order): the tiles the token-exact
    passes visit, for FLOP accounting and for the block-cover forward of ``fwd_lists``."""
    if window <= 0 or N % window:
        raise ValueError("the window must divide N")
    return (pattern_mask(SA_PAT_LOCAL, B, H, N, bq, bk, window=window, device=device),
            pattern_mask(SA_PAT_LOCAL, B, H, N, bq, bk, window=N // window, device=device))


def squad_fwd(q, k, v, window: int, bq: int, global_pass: bool, scale: float | None = None,
              out: torch.Tensor | None = None, return_lse: bool = False):
    """One token-exact SQuad pass (bf16): the local pass (each token attends to its window of
    ``window`` tokens) or the global pass (each token attends to the tokens at its position
    inside their windows; ``window`` must divide N and N / window be at least 64)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    _lib.check(_lib.lib().sparse_attn_squad_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype], B, H, N, d, bq, int(window),
        _lib.SA_SQUAD_GLOBAL if global_pass else _lib.SA_SQUAD_LOCAL, scale, o.data_ptr(),
        None if lse is None else lse.data_ptr(), _stream(q)))
    return (o, lse) if return_lse else o


def squad_attention(q, k, v, window: int, bq: int, bk: int = 64, scale: float | None = None,
                    return_local: bool = False):
    """The two-pass SQuad operator, token-exact: O_local = the local pass of (Q, K, V), then the
    global pass of (Q, K, O_local). The global pass reads the window-transposed order in place
    when there are at least 64 windows; with fewer it runs as a local pass with windows of
    N / window over transposed copies (the same arithmetic). ``window`` must divide N."""
    if bk != 64:
        raise ValueError("the SQuad passes run on 64-key tiles")
    B, H, N, d = q.shape
    if window <= 0 or N % window:
        raise ValueError("the window must divide N")
    o_local = squad_fwd(q, k, v, window, bq, False, scale)
    if N // window >= 64:
        o = squad_fwd(q, k, o_local, window, bq, True, scale)
    else:
        qt, kt, vt = (window_transpose(t, window) for t in (q, k, o_local))
        o = window_transpose(squad_fwd(qt, kt, vt, N // window, bq, False, scale), window, inverse=True)
    return (o, o_local) if return_local else o


def _workspace(nbytes: int, workspace, device):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace


def bwd_workspace_size(B: int, H: int, N: int, bq: int, bk: int = 64) -> int:
    return int(_lib.lib().sparse_attn_bwd_workspace_size(B, H, N, bq, bk))


def bwd(q, k, v, o, dout, lse, mask, bq: int, bk: int = 64, scale: float | None = None,
        workspace: torch.Tensor | None = None, out: tuple | None = None):
    """(dQ, dK, dV) of the block-sparse attention for the forward's mask, output and LSE (bf16)."""
    _check_qkv(q, k, v, o, dout)
    B, H, N, d = q.shape
    nqb, nkb = _nblocks(N, bq), _nblocks(N, bk)
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (B, H, nqb, nkb) or not mask.is_contiguous():
        raise ValueError(f"mask must be a contiguous uint8 [{B}, {H}, {nqb}, {nkb}] tensor")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 [{B}, {H}, {N}] tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(bwd_workspace_size(B, H, N, bq, bk), workspace, q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if out is None else \
        (_check_out(t, q.shape, q.dtype, q.device) for t in out)
    _lib.check(_lib.lib().sparse_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                          lse.data_ptr(), _DTYPES[q.dtype], mask.data_ptr(), B, H, N, d, bq, bk, scale,
                                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def probe_workspace_size(B: int, H: int, N: int, d: int, bq: int, probes: int) -> int:
    return int(_lib.lib().sparse_attn_probe_workspace_size(B, H, N, d, bq, probes))


def probe_correct(q, k, v, o, bq: int, probes: int, ridge: float, scale: float | None = None,
                  workspace: torch.Tensor | None = None, return_fit: bool = False, rank: int | None = None):
    """Probe-fitted residual correction of the sparse output ``o`` (bf16), in place. ``rank``
    confines the map to that many principal directions of the probe residuals (None: no limit).

    With ``return_fit`` also returns A (float32 ``[B, H, d + 1, d]``) and the exact probe rows
    (float32 ``[B, H, probes * bq, d]``)."""
    _check_qkv(q, k, v, o)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(probe_workspace_size(B, H, N, d, bq, probes), workspace, q.device)
    a = exact = None
    if return_fit:
        a = torch.empty((B, H, d + 1, d), dtype=torch.float32, device=q.device)
        exact = torch.empty((B, H, probes * bq, d), dtype=torch.float32, device=q.device)
    _lib.check(_lib.lib().sparse_attn_probe_correct(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _DTYPES[q.dtype], B, H, N, d, bq, scale, int(probes),
        float(ridge), d if rank is None else int(rank), a.data_ptr() if a is not None else None,
        exact.data_ptr() if exact is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, a, exact) if return_fit else o


def kmeans(x, C: int, iters: int, init: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Lloyd's k-means of the token rows of ``x`` (bf16 ``[B, H, N, d]``) into ``C`` clusters per
    head. Returns a dict with ``centroids`` (float32 ``[B, H, C, d]``), ``labels`` and ``perm``
    (int32 ``[B, H, N]``) and ``offsets`` (int32 ``[B, H, C + 1]``)."""
    _check_qkv(x)
    B, H, N, d = x.shape
    if init is not None and (init.dtype != torch.float32 or tuple(init.shape) != (B, H, C, d)
                             or not init.is_contiguous() or init.device != x.device):
        raise ValueError(f"init must be a contiguous float32 [{B}, {H}, {C}, {d}] tensor on {x.device}")
    workspace = _workspace(int(_lib.lib().sparse_attn_kmeans_workspace_size(B, H, N, d, C)), workspace, x.device)
    out = {"centroids": torch.empty((B, H, C, d), dtype=torch.float32, device=x.device),
           "labels": torch.empty((B, H, N), dtype=torch.int32, device=x.device),
           "perm": torch.empty((B, H, N), dtype=torch.int32, device=x.device),
           "offsets": torch.empty((B, H, C + 1), dtype=torch.int32, device=x.device)}
    _lib.check(_lib.lib().sparse_attn_kmeans(
        x.data_ptr(), _DTYPES[x.dtype], B, H, N, d, int(C), int(iters), init.data_ptr() if init is not None else None,
        out["centroids"].data_ptr(), out["labels"].data_ptr(), out["perm"].data_ptr(), out["offsets"].data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(x)))
    return out


def cluster_select(cq: torch.Tensor, ck: torch.Tensor, k_offsets: torch.Tensor, p: float, scale: float | None = None,
                   return_probs: bool = False):
    """Centroid Top-p: uint8 mask ``[B, H, Cq, Ck]`` (and the float64 masses)."""
    B, H, Cq, d = cq.shape
    Ck = ck.shape[2]
    for t, dt in ((cq, torch.float32), (ck, torch.float32), (k_offsets, torch.int32)):
        if t.dtype != dt or not t.is_contiguous() or t.device != cq.device:
            raise ValueError("cq, ck must be contiguous float32 and k_offsets contiguous int32 on one device")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    mask = torch.empty((B, H, Cq, Ck), dtype=torch.uint8, device=cq.device)
    probs = torch.empty((B, H, Cq, Ck), dtype=torch.float64, device=cq.device) if return_probs else None
    _lib.check(_lib.lib().sparse_attn_cluster_select(
        cq.data_ptr(), ck.data_ptr(), k_offsets.data_ptr(), B, H, Cq, Ck, d, scale, float(p),
        probs.data_ptr() if probs is not None else None, mask.data_ptr(), _stream(cq)))
    return (mask, probs) if return_probs else mask


def permute_rows(x: torch.Tensor, perm: torch.Tensor, inverse: bool = False, out: torch.Tensor | None = None):
    """Gather ``x[..., perm[t'], :]`` into row t' (or scatter row t' to ``perm[t']`` if inverse)."""
    _check_qkv(x)
    B, H, N, d = x.shape
    if perm.dtype != torch.int32 or tuple(perm.shape) != (B, H, N) or not perm.is_contiguous():
        raise ValueError(f"perm must be a contiguous int32 [{B}, {H}, {N}] tensor")
    o = torch.empty_like(x) if out is None else _check_out(out, x.shape, x.dtype, x.device)
    _lib.check(_lib.lib().sparse_attn_permute_rows(x.data_ptr(), _DTYPES[x.dtype], B, H, N, d, perm.data_ptr(),
                                                   1 if inverse else 0, o.data_ptr(), _stream(x)))
    return o


def cluster_fwd(q, k, v, q_offsets, k_offsets, mask, bq: int = 128, scale: float | None = None,
                return_lse: bool = False, workspace: torch.Tensor | None = None, out=None,
                q_perm: torch.Tensor | None = None, k_perm: torch.Tensor | None = None):
    """Attention over variable-size blocks. Q and the output are in the query-permuted order and
    K / V in the key-permuted order, or each in the original token order when its permutation
    (``q_perm`` / ``k_perm``: the clusterings' ``perm``) is given."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    Cq, Ck = q_offsets.shape[-1] - 1, k_offsets.shape[-1] - 1
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (B, H, Cq, Ck) or not mask.is_contiguous():
        raise ValueError(f"mask must be a contiguous uint8 [{B}, {H}, {Cq}, {Ck}] tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace = _workspace(int(_lib.lib().sparse_attn_cluster_fwd_workspace_size(B, H, N, Cq, Ck, bq)), workspace,
                           q.device)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    for name, t in (("q_perm", q_perm), ("k_perm", k_perm)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B, H, N) or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous int32 [{B}, {H}, {N}] tensor on {q.device}")
    _lib.check(_lib.lib().sparse_attn_cluster_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[q.dtype], B, H, N, d, q_offsets.data_ptr(), Cq,
        k_offsets.data_ptr(), Ck, mask.data_ptr(), q_perm.data_ptr() if q_perm is not None else None,
        k_perm.data_ptr() if k_perm is not None else None, bq, scale,
        o.data_ptr(), lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, lse) if return_lse else o


def svg2_attention(q, k, v, Cq: int, Ck: int, iters: int, p: float, bq: int = 128, scale: float | None = None,
                   init_q: torch.Tensor | None = None, init_k: torch.Tensor | None = None, return_info: bool = False):
    """Semantic-aware permutation end to end: k-means of Q and K, centroid Top-p, attention over
    the permuted variable-size blocks, output permuted back to the original token order."""
    kq = kmeans(q, Cq, iters, init=init_q)
    kk = kmeans(k, Ck, iters, init=init_k)
    mask = cluster_select(kq["centroids"], kk["centroids"], kk["offsets"], p, scale)
    o = cluster_fwd(q, k, v, kq["offsets"], kk["offsets"], mask, bq, scale, q_perm=kq["perm"], k_perm=kk["perm"])
    if return_info:
        return o, {"kmeans_q": kq, "kmeans_k": kk, "mask": mask}
    return o
