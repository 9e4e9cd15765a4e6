#!/usr/bin/env python3
"""Throughput of the block-sparse attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in HBM:
    sparse_attn_pool_qk      block mean pooling of Q and K
    sparse_attn_select_mask  pooled softmax, hybrid Top-k U Top-p mask and kept-block lists
    sparse_attn_row_order    the rows' work order (longest kept lists first on short grids)
    sparse_attn_fwd_lists_ordered  block-sparse flash attention over the kept blocks
on the Wan2.1-14B 720p-shaped workload (40 heads x 75600 tokens x 128, bf16, Bq=128, Bk=64,
k_frac=0.03, p=0.9). Throughput is executed TFLOP/s: 4 d sum over kept (query block, key block)
pairs of valid queries x valid keys, divided by the step time.

Prints one JSON line. ``--gpus`` above 1 is refused: the library is a one-GPU kernel library.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X published dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan720p_traffic.json")
WORKLOAD_SHAPES = {"wan720p": "Wan2.1-14B 720p-shaped", "wan480p": "Wan2.1-1.3B 480p-shaped",
                   "stress": "distribution stress (near-uniform and sink-skewed heads),", "tiny": "tiny fp32",
                   "sweep720p": "Wan2.1-14B 720p-shaped"}
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_query_amd", "csrc", f)
                for f in ("attn_fwd.hip", "attn_tiles.h", "sa_common.h")]


def attn_source_digest() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


TRAFFIC_WORKLOAD = "wan720p"  # the workload the committed counters were taken on


def measured_traffic(workload: str):
    """HBM bytes per attention launch and its L2 hit rate, from committed rocprofv3 counters, if
    they were taken on the current kernel source and on this workload."""
    if workload != TRAFFIC_WORKLOAD:
        return None, None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if rec.get("source_sha256") != attn_source_digest():
        return None, None
    return rec.get("bytes_per_launch"), rec.get("l2_hit_rate")


def executed_flops(mask_cpu, n, bq, bk, d):
    import numpy as np
    nqb, nkb = mask_cpu.shape[-2:]
    nq = np.array([min(bq, n - i * bq) for i in range(nqb)], dtype=np.float64)
    nk = np.array([min(bk, n - j * bk) for j in range(nkb)], dtype=np.float64)
    m = mask_cpu.astype(np.float64)
    return float(4 * d * (m * nq[:, None] * nk[None, :]).sum())


def cpu_baseline(w, x, mask_cpu, sample_blocks: int, o_head0=None, lse_head0=None):
    """The float64 oracle on a bounded sample of the same workload, on the host cores.

    With the GPU's output for head 0 (``o_head0`` [B, 1, N, d], ``lse_head0`` [B, 1, N]) it also
    returns the parity of the timed call on that sample: the head's mask against the oracle's
    (mismatches and ties within 1e-6, as the parity tests classify them) and the attention error
    on the sampled query blocks whose mask rows agree."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads, threadpool_limits = 1, None
    h = 0
    q = x["q"][:, h:h + 1].double().numpy()
    k = x["k"][:, h:h + 1].double().numpy()
    v = x["v"][:, h:h + 1].double().numpy()
    nqb = mask_cpu.shape[2]
    scale = 1.0 / math.sqrt(w.head_dim)
    t0 = time.perf_counter()
    mask_o, info = oracle.block_mask(q, k, w.bq, w.bk, w.k_frac, w.p, scale)
    t_mask = time.perf_counter() - t0
    t_mask_1t = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.block_mask(q, k, w.bq, w.bk, w.k_frac, w.p, scale)
            t_mask_1t = time.perf_counter() - t0
    blocks = sorted(set(np.linspace(0, nqb - 1, sample_blocks).round().astype(int).tolist()))
    t0 = time.perf_counter()
    ro, rl = oracle.masked_attention(q, k, v, mask_o, w.bq, w.bk, blocks=[(0, 0, i) for i in blocks])
    t_attn = time.perf_counter() - t0
    sub = np.zeros_like(mask_o)
    sub[0, 0, blocks] = mask_o[0, 0, blocks]
    flops = oracle.executed_flops(sub, w.tokens, w.bq, w.bk, w.head_dim)
    t = t_attn + t_mask * len(blocks) / nqb
    # whole call on all heads: the mask oracle per head, attention scaled by executed FLOPs
    full_flops = executed_flops(mask_cpu, w.tokens, w.bq, w.bk, w.head_dim)
    extrapolated = w.batch * w.heads * t_mask + t_attn * full_flops / flops
    parity = None
    if o_head0 is not None:
        gm = mask_cpu[:, h:h + 1]
        rep = oracle.compare_masks(info["probs"], mask_o, gm, w.k_frac, w.p)
        same = (gm == mask_o).all(axis=-1)[0, 0]
        rows = np.zeros(w.tokens, dtype=bool)
        for i in blocks:
            if same[i]:
                rows[i * w.bq:min(w.tokens, (i + 1) * w.bq)] = True
        go = o_head0[0, 0].double().numpy()[rows]
        err = np.abs(go - ro[0, 0][rows])
        parity = {"head": h, "mask_rows": rep["rows"], "mask_rows_equal": rep["rows_equal"],
                  "mask_ties": rep["ties"], "mask_mismatches": rep["mismatches"],
                  "attn_rows": int(rows.sum()), "attn_max_abs": float(err.max()) if err.size else None,
                  "attn_mean_abs": float(err.mean()) if err.size else None,
                  "bars": {"max_abs": 2e-2, "mean_abs": 5e-3}}
        if lse_head0 is not None:
            gl = lse_head0[0, 0].double().numpy()[rows]
            rr = rl[0, 0][rows]
            fin = np.isfinite(rr)
            parity["lse_max_abs"] = float(np.abs(gl[fin] - rr[fin]).max()) if fin.any() else None
    return parity, {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"head 0 of {w.heads}: float64 mask oracle on all {nqb} query blocks ({t_mask:.2f} s, "
                   f"prorated to the sample), masked-dense attention on {len(blocks)} evenly spaced query "
                   f"blocks ({t_attn:.2f} s); executed FLOPs of those blocks / time"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "seconds": round(t_mask + t_attn + (t_mask_1t or 0.0), 2),
        "mask_oracle_head_s": round(t_mask, 3),
        "mask_oracle_head_s_1thread": None if t_mask_1t is None else round(t_mask_1t, 3),
        "extrapolated_full_call_s": round(extrapolated, 1),
        "extrapolated_note": "extrapolated, not measured: mask oracle time x all heads + sampled attention "
                             "time scaled by executed FLOPs of the whole call",
    }


def pattern_bench(args, sa, w, q, k, v, gen_s):
    """Fixed-pattern workloads on the same kernel. The masks depend on positions only, so they are
    built once before the timed region; a step is the attention work of the pattern."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    frame = w.grid[1] * w.grid[2]
    o = torch.empty_like(q)
    if args.pattern == "squad":
        window = 3 * w.grid[2]  # 3 latent rows: 240 tokens at 720p, about sqrt(N)
        masks = sa.squad_masks(B, H, N, window, w.bq, w.bk, q.device)  # block covers: tile accounting only
        bufs = [torch.empty_like(q) for _ in range(4 if args.squad_materialise else 1)]

        def step(ev):
            ev[0].record()
            sa.squad_fwd(q, k, v, window, w.bq, False, out=bufs[0])   # local pass
            ev[1].record()
            if not args.squad_materialise:  # global pass reading the window-transposed order in place
                sa.squad_fwd(q, k, bufs[0], window, w.bq, True, out=o)
                ev[2].record()
                return
            sa.window_transpose(q, window, out=bufs[1])
            sa.window_transpose(k, window, out=bufs[2])
            sa.window_transpose(bufs[0], window, out=bufs[3])
            ev[2].record()
            sa.squad_fwd(bufs[1], bufs[2], bufs[3], N // window, w.bq, False, out=bufs[0])
            ev[3].record()
            sa.window_transpose(bufs[0], window, inverse=True, out=o)
            ev[4].record()

        mask_list = [m["mask"].cpu().numpy() for m in masks]
        # token-exact operator: each token attends to its window (w keys) and to its position class
        # (N / w keys); the tiles the kernel runs are the block covers of those patterns
        flops = 4.0 * d * B * H * (N * window + N * (N // window))
        params = {"window": window, "global_run": N // window, "operator": "token-exact windows and position classes",
                  "global_pass": "materialised transposes" if args.squad_materialise else "window-order reads"}
        if args.squad_materialise:
            split = lambda e: (e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]),  # noqa: E731
                               e[1].elapsed_time(e[2]) + e[3].elapsed_time(e[4]))
        else:
            split = lambda e: (e[0].elapsed_time(e[2]), 0.0)  # noqa: E731
        metric = "SQuad two-pass (local + global) attention fwd TFLOP/s (token pairs attended)"
    else:
        band, period = 3 * w.grid[2], frame
        m = sa.pattern_mask(sa.SA_PAT_DIAG | sa.SA_PAT_MULTIDIAG | sa.SA_PAT_STRIPE, B, H, N, w.bq, w.bk,
                            band=band, period=period, device=q.device)

        def step(ev):
            ev[0].record()
            sa.fwd_lists(q, k, v, m["kept_idx"], m["kept_cnt"], w.bq, w.bk, out=o)
            ev[1].record()

        mask_list = [m["mask"].cpu().numpy()]
        params = {"band": band, "period": period, "stripe_period": period}
        split = lambda e: (e[0].elapsed_time(e[1]), 0.0)  # noqa: E731
        metric = "Sparse-vDiT pattern (diagonal + per-frame diagonals + frame-start stripes) sparse attention fwd " \
                 "TFLOP/s (executed)"
        flops = None
    tile_flops = sum(executed_flops(mm, N, w.bq, w.bk, d) for mm in mask_list)
    flops = tile_flops if flops is None else flops
    nev = 5 if args.pattern == "squad" else 2  # the squad step without transposes records 3 of them
    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(nev)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for e in evs:
        step(e)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    attn_ms, perm_ms = (float(v) for v in np.array([split(e) for e in evs]).mean(axis=0))
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    return {
        "metric": metric, "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {args.pattern} fixed pattern on the {w.grid[0]}x{w.grid[1]}x{w.grid[2]} "
                               f"latent grid", "batch": B, "heads": H, "tokens": N, "head_dim": d, "bq": w.bq,
                   "bk": w.bk, **params,
                   "kept_block_density": [round(float(mm.mean()), 5) for mm in mask_list],
                   "executed_tflop_per_step": round(flops / 1e12, 4), "tile_tflop_per_step": round(tile_flops / 1e12, 4),
                   "masks": "built once, outside the timed region",
                   "parallelism": "none (1 GPU)"},
        "ms_per_call": {"fwd_lists_total": round(attn_ms, 4), "window_transpose_total": round(perm_ms, 4)},
        "roofline": {"kernel": "attn_fwd_kernel<bf16, 128, 128>", "bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "window_transpose_gbs": None if perm_ms == 0 else round(4 * 2 * B * H * N * d * q.element_size()
                                                                / (perm_ms * 1e-3) / 1e9, 1),
        "input_generation_s": round(gen_s, 1),
    }


def backward_bench(args, sa, w, q, k, v, gen_s):
    """sparse_attn_bwd on the hybrid mask of the workload. Algorithmic FLOPs are 2.5x the forward's
    executed FLOPs (S, dP, dV, dQ, dK at 2 d per kept (query, key) pair); the kernels recompute S
    and dP once more for dQ, which is not credited."""
    import torch
    B, H, N, d = q.shape
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p)
    o, lse = sa.fwd(q, k, v, sel["mask"], w.bq, w.bk, return_lse=True)
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(q.dtype).to(q.device)
    ws = torch.empty(sa.bwd_workspace_size(B, H, N, w.bq, w.bk), dtype=torch.uint8, device=q.device)
    outs = tuple(torch.empty_like(q) for _ in range(3))
    mask_cpu = sel["mask"].cpu().numpy()
    fwd_flops = executed_flops(mask_cpu, N, w.bq, w.bk, d)
    flops = 2.5 * fwd_flops

    def step():
        sa.bwd(q, k, v, o, g, lse, sel["mask"], w.bq, w.bk, workspace=ws, out=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "block-sparse attention backward TFLOP/s (algorithmic: 2.5x forward executed FLOPs)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: backward on the hybrid mask", "batch": B, "heads": H, "tokens": N,
                   "head_dim": d, "bq": w.bq, "bk": w.bk, "k_frac": w.k_frac, "p": w.p,
                   "kept_block_density": round(float(mask_cpu.mean()), 5),
                   "algorithmic_tflop_per_step": round(flops / 1e12, 4), "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "sparse_attn_bwd (delta, dQ, dK/dV kernels)", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "input_generation_s": round(gen_s, 1),
    }


def corrected_bench(args, sa, w, q, k, v, gen_s):
    """The hot path followed by the probe-fitted residual correction (sparse_attn_probe_correct,
    ``--correct`` probes, ridge 1e-3). Executed FLOPs add the probes' dense attention (4 d per
    valid probe query x key) and the applied map (2 d^2 per token) to the sparse attention's. Also
    reports how far the sparse and the corrected outputs are from exact attention on 8 held-out
    query blocks per head (relative L2 error), exact rows from sparse_attn_fwd with those rows'
    masks full."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    nqb, nkb = -(-N // w.bq), -(-N // w.bk)
    P, ridge = args.correct, 1e-3
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p, kept_lists=True)
    o = torch.empty_like(q)
    ws = torch.empty(sa.probe_workspace_size(B, H, N, d, w.bq, P), dtype=torch.uint8, device=q.device)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sa.pool_qk(q, k, w.bq, w.bk, out=(qp, kp))
        sa.select_mask(qp, kp, w.k_frac, w.p, kept_lists=True, out=sel)
        if ev is not None:
            ev[1].record()
        sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, out=o)
        if ev is not None:
            ev[2].record()
        sa.probe_correct(q, k, v, o, w.bq, P, ridge, workspace=ws, rank=args.rank)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mask_cpu = sel["mask"].cpu().numpy()
    full = nqb if N % w.bq == 0 else max(nqb - 1, 1)
    probe_rows = sum(min(w.bq, N - (min(full - 1, int((p + 0.5) * full / P))) * w.bq) for p in range(P))
    probe_flops = 4.0 * d * B * H * probe_rows * N
    apply_flops = 2.0 * d * d * B * H * N
    flops = executed_flops(mask_cpu, N, w.bq, w.bk, d) + probe_flops + apply_flops
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        step(evs[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    mask_ms, attn_ms, corr_ms = (float(x) for x in per.mean(axis=0))

    # held-out quality: exact rows of 8 query blocks per head that are not probes
    held = sorted({min(full - 1, int((j + 0.25) * full / 8)) for j in range(8)} -
                  {min(full - 1, int((p + 0.5) * full / P)) for p in range(P)})
    m_ex = torch.zeros((B, H, nqb, nkb), dtype=torch.uint8, device=q.device)
    m_ex[:, :, held] = 1
    o_ex = sa.fwd(q, k, v, m_ex, w.bq, w.bk)
    o_s = sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk)
    rows = torch.cat([torch.arange(i * w.bq, min(N, (i + 1) * w.bq)) for i in held]).to(q.device)
    ex, sp, co = (t[:, :, rows].float() for t in (o_ex, o_s, o))
    rel = lambda t: float((t - ex).norm() / ex.norm())  # noqa: E731
    by_rank = {}
    for r in args.rank_sweep:  # untimed: the same correction confined to r principal directions
        o_r = o_s.clone()
        sa.probe_correct(q, k, v, o_r, w.bq, P, ridge, workspace=ws, rank=r)
        by_rank[str(r)] = round(rel(o_r[:, :, rows].float()), 5)
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "sparse attention fwd + probe-fitted correction TFLOP/s (executed)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic" + (", smooth values" if args.smooth_v else ""),
        "config": {"workload": f"{w.name}: hybrid mask, then {P} probe blocks per head", "batch": B, "heads": H,
                   "tokens": N, "head_dim": d, "bq": w.bq, "bk": w.bk, "k_frac": w.k_frac, "p": w.p,
                   "probes": P, "ridge": ridge, "rank": d if args.rank is None else args.rank,
                   "kept_block_density": round(float(mask_cpu.mean()), 5),
                   "executed_tflop_per_step": round(flops / 1e12, 4),
                   "probe_dense_tflop": round(probe_flops / 1e12, 4), "apply_tflop": round(apply_flops / 1e12, 4),
                   "parallelism": "none (1 GPU)"},
        "ms_per_call": {"pool_qk+select_mask": round(mask_ms, 4), "fwd_lists": round(attn_ms, 4),
                        "probe_correct": round(corr_ms, 4)},
        "heldout_rel_l2_error": {"query_blocks_per_head": len(held), "sparse": round(rel(sp), 5),
                                 "corrected": round(rel(co), 5), "corrected_by_rank": by_rank},
        "roofline": {"kernel": "attn_fwd_kernel<bf16, 128, 128>", "bound": "mfma",
                     "achieved": round(executed_flops(mask_cpu, N, w.bq, w.bk, d) / (attn_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(executed_flops(mask_cpu, N, w.bq, w.bk, d) / (attn_ms * 1e-3) / 1e12
                                   / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "input_generation_s": round(gen_s, 1),
    }


def svg2_bench(args, sa, w, q, k, v, gen_s):
    """Semantic-aware permutation end to end: k-means of Q (Cq clusters) and K (Ck clusters),
    centroid Top-p, permutation of Q / K / V, attention over the variable-size blocks and the
    inverse permutation of O. Executed FLOPs are 4 d per kept (query, key) pair, counted exactly
    from the clusters (no padding). ``--svg2-warm`` starts each step's k-means from the previous
    step's centroids with one iteration (the centroid cache), otherwise every step starts from
    evenly spaced tokens and runs ``--svg2-iters`` iterations."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    Cq, Ck, p = args.svg2_clusters
    iters = 1 if args.svg2_warm else args.svg2_iters
    cache = {}

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        kq = sa.kmeans(q, Cq, iters, init=cache.get("q"))
        kk = sa.kmeans(k, Ck, iters, init=cache.get("k"))
        if args.svg2_warm:
            cache["q"], cache["k"] = kq["centroids"], kk["centroids"]
        if ev is not None:
            ev[1].record()
        mask = sa.cluster_select(kq["centroids"], kk["centroids"], kk["offsets"], p)
        # Q is read and O written in the original token order through the query permutation; K and
        # V are either permuted into cluster order first or gathered through the key permutation
        if args.svg2_permute_kv:
            kp, vp, k_perm = sa.permute_rows(k, kk["perm"]), sa.permute_rows(v, kk["perm"]), None
        else:
            kp, vp, k_perm = k, v, kk["perm"]
        if ev is not None:
            ev[2].record()
        o = sa.cluster_fwd(q, kp, vp, kq["offsets"], kk["offsets"], mask, w.bq, q_perm=kq["perm"], k_perm=k_perm)
        if ev is not None:
            ev[3].record()
        return o, kq, kk, mask

    if args.svg2_warm:  # fill the cache with a converged cold start, outside the timed region
        kq0, kk0 = sa.kmeans(q, Cq, args.svg2_iters), sa.kmeans(k, Ck, args.svg2_iters)
        cache["q"], cache["k"] = kq0["centroids"], kk0["centroids"]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        o, kq, kk, mask = step(evs[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs]).mean(axis=0)
    nq = np.diff(kq["offsets"].cpu().numpy().astype(np.int64), axis=-1)
    nk = np.diff(kk["offsets"].cpu().numpy().astype(np.int64), axis=-1)
    m = mask.cpu().numpy().astype(np.int64)
    pairs = float(np.einsum("bhi,bhij,bhj->", nq, m, nk))
    kept_keys = np.einsum("bhij,bhj->bhi", m, nk)
    key_tiles = np.ceil(kept_keys / 64.0)
    q_tiles = np.ceil(nq / w.bq)
    tile_flops = 4.0 * d * w.bq * 64 * float((q_tiles * key_tiles).sum())
    flops = 4.0 * d * pairs
    attn_tf = flops / (per[2] * 1e-3) / 1e12
    # sampled quality: 8 positional query blocks per head, exact rows from the dense forward
    nqb, nkb = -(-N // w.bq), -(-N // w.bk)
    full = nqb if N % w.bq == 0 else max(nqb - 1, 1)
    held = sorted({min(full - 1, int((j + 0.25) * full / 8)) for j in range(8)})  # the --correct blocks
    m_ex = torch.zeros((B, H, nqb, nkb), dtype=torch.uint8, device=q.device)
    m_ex[:, :, held] = 1
    o_ex = sa.fwd(q, k, v, m_ex, w.bq, w.bk)
    rows = torch.cat([torch.arange(i * w.bq, min(N, (i + 1) * w.bq)) for i in held]).to(q.device)
    ex, sp = o_ex[:, :, rows].float(), o[:, :, rows].float()
    return {
        "metric": "semantic-aware permutation attention TFLOP/s (executed, whole step)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic" + (", smooth values" if args.smooth_v else ""),
        "config": {"workload": f"{w.name}: k-means permutation, {Cq} query / {Ck} key clusters, p = {p}, "
                               f"{'warm start, 1 iteration' if args.svg2_warm else f'{iters} iterations from evenly spaced tokens'}"
                               f"{', K / V permuted first' if args.svg2_permute_kv else ''}",
                   "batch": B, "heads": H, "tokens": N, "head_dim": d, "bq": w.bq, "query_clusters": Cq,
                   "key_clusters": Ck, "p": p, "kmeans_iters": iters, "kept_pair_density": round(pairs / (B * H * N * N), 5),
                   "executed_tflop_per_step": round(flops / 1e12, 4), "tile_tflop_per_step": round(tile_flops / 1e12, 4),
                   "parallelism": "none (1 GPU)"},
        "ms_per_call": {"kmeans_q+k": round(float(per[0]), 4),
                        ("cluster_select+permute_kv" if args.svg2_permute_kv else "cluster_select"): round(float(per[1]), 4),
                        "cluster_fwd": round(float(per[2]), 4)},
        "cluster_fwd_tflops": round(attn_tf, 2),
        "sampled_rel_l2_error_vs_dense": round(float((sp - ex).norm() / ex.norm()), 5),
        "roofline": {"kernel": "attn_var_kernel<128, 128>", "bound": "mfma", "achieved": round(attn_tf, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
        "input_generation_s": round(gen_s, 1),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=240)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes --steps times (to calibrate "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against a known byte count) and exit")
    ap.add_argument("--pattern", choices=("hybrid", "squad", "vdit"), default="hybrid",
                    help="hybrid: the Top-k U Top-p path (default). squad: fixed two-pass SQuad attention (local "
                         "windows of 240 tokens, then the same-position pass in the window-transposed order). "
                         "vdit: Sparse-vDiT style union of a diagonal band, the band repeated every frame and the "
                         "first key token of every frame")
    ap.add_argument("--backward", action="store_true",
                    help="time the block-sparse backward (sparse_attn_bwd) on the workload's hybrid mask instead "
                         "of the forward path; the mask, O and LSE are computed once before the timed region")
    ap.add_argument("--correct", type=int, default=0, metavar="PROBES",
                    help="time the hot path followed by the probe-fitted residual correction with PROBES probe "
                         "query blocks per head (ridge 1e-3), and report held-out error before and after")
    ap.add_argument("--rank", type=int, default=None,
                    help="--correct: confine the map to RANK principal directions of the probe residuals "
                         "(default: head_dim, no limit)")
    ap.add_argument("--rank-sweep", type=lambda t: [int(x) for x in t.split(",") if x], default=[],
                    help="--correct: also report the held-out error for these comma-separated ranks (untimed)")
    ap.add_argument("--svg2", action="store_true",
                    help="time the semantic-aware permutation path (k-means clusters, centroid Top-p, attention "
                         "over variable-size blocks) instead of the block-mask path")
    ap.add_argument("--svg2-clusters", type=float, nargs=3, default=(128, 256, 0.9), metavar=("CQ", "CK", "P"),
                    help="query clusters, key clusters and Top-p threshold of --svg2 (default 128 256 0.9)")
    ap.add_argument("--svg2-iters", type=int, default=3, help="k-means iterations of --svg2 (default 3)")
    ap.add_argument("--squad-materialise", action="store_true",
                    help="--pattern squad: write window-transposed copies of Q, K and the local output (and "
                         "transpose the result back) instead of reading that order in place")
    ap.add_argument("--svg2-permute-kv", action="store_true",
                    help="--svg2: permute K and V into cluster order first instead of gathering their rows "
                         "through the key permutation")
    ap.add_argument("--svg2-warm", action="store_true",
                    help="with --svg2: start every step from the previous step's centroids, one iteration")
    ap.add_argument("--smooth-v", action="store_true",
                    help="spatially smooth values (a second standardised Gaussian field plus noise) instead of "
                         "i.i.d. ones; for the quality figures of --correct and --svg2")
    ap.add_argument("--sweep-out", default=None,
                    help="also time the attention call on the density sweep and write JSON lines here")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this is a one-GPU kernel library. Heads are "
              f"independent, so several GPUs would each run this same path on their share of heads.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4,
                          "launches": args.steps}))
        return 0
    sys.path.insert(0, ROOT)
    import block_sparse_attention_query_amd as sa
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    x = make_inputs(w, smooth_v=args.smooth_v)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (x["q"], x["k"], x["v"]))
    B, H, N, d = q.shape
    nqb, nkb = -(-N // w.bq), -(-N // w.bk)
    qp = torch.empty((B, H, nqb, d), dtype=torch.float64, device=dev)
    kp = torch.empty((B, H, nkb, d), dtype=torch.float64, device=dev)
    sel = {"probs": torch.empty((B, H, nqb, nkb), dtype=torch.float64, device=dev),
           "mask": torch.empty((B, H, nqb, nkb), dtype=torch.uint8, device=dev),
           "kept_idx": torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=dev),
           "kept_cnt": torch.empty((B, H, nqb), dtype=torch.int32, device=dev)}
    order = torch.empty(B * H * nqb, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    if args.pattern != "hybrid":
        print(json.dumps(pattern_bench(args, sa, w, q, k, v, gen_s)), flush=True)
        return 0
    if args.backward:
        print(json.dumps(backward_bench(args, sa, w, q, k, v, gen_s)), flush=True)
        return 0
    if args.correct:
        print(json.dumps(corrected_bench(args, sa, w, q, k, v, gen_s)), flush=True)
        return 0
    if args.svg2:
        args.svg2_clusters = (int(args.svg2_clusters[0]), int(args.svg2_clusters[1]), float(args.svg2_clusters[2]))
        print(json.dumps(svg2_bench(args, sa, w, q, k, v, gen_s)), flush=True)
        return 0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sa.pool_qk(q, k, w.bq, w.bk, out=(qp, kp))
        if ev is not None:
            ev[1].record()
        sa.select_mask(qp, kp, w.k_frac, w.p, kept_lists=True, out=sel)
        sa.row_order(sel["kept_cnt"], out=order)
        if ev is not None:
            ev[2].record()
        sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, out=o, row_order=order)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mask_cpu = sel["mask"].cpu().numpy()
    flops = executed_flops(mask_cpu, N, w.bq, w.bk, d)
    tile_flops = 4.0 * d * w.bq * w.bk * float(mask_cpu.sum())  # what the kernel runs, padding included
    density = float(mask_cpu.mean())
    # what the hybrid rule kept: Top-k alone keeps k blocks per row, so rows above k are the ones
    # whose Top-p prefix was longer (per group of 8 heads)
    k_blocks = sa.topk_count(w.k_frac, mask_cpu.shape[-1])
    cnt = mask_cpu.sum(-1, dtype=np.int64).reshape(B, H, -1)
    groups = [(h0, min(H, h0 + 8)) for h0 in range(0, H, 8)]
    selection = {"topk_blocks": k_blocks, "kept_per_row_mean": round(float(cnt.mean()), 2),
                 "kept_per_row_max": int(cnt.max()),
                 "rows_topp_longer": round(float((cnt > k_blocks).mean()), 4),
                 "by_head_group": [{"heads": f"{a}-{b - 1}", "kept_per_row_mean": round(float(cnt[:, a:b].mean()), 2),
                                    "rows_topp_longer": round(float((cnt[:, a:b] > k_blocks).mean()), 4)}
                                   for a, b in groups]}

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    pool_ms, select_ms, attn_ms = (float(v) for v in per.mean(axis=0))
    stats = {name: {"median": round(float(np.median(col)), 4), "p10": round(float(np.percentile(col, 10)), 4),
                    "p90": round(float(np.percentile(col, 90)), 4)}
             for name, col in zip(("pool_qk", "select_mask+row_order", "fwd_lists"), per.T)}

    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    alg_bytes = 4 * B * H * N * d * q.element_size()  # Q, K, V read once and O written once
    traffic, l2_hit = measured_traffic(args.workload)
    result = {
        "metric": "sparse attention fwd TFLOP/s (executed) + ms/call at 95% sparsity; % bf16 MFMA peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {WORKLOAD_SHAPES.get(w.name, 'synthetic')} latent grid "
                               f"{w.grid[0]}x{w.grid[1]}x{w.grid[2]}",
                   "batch": B, "heads": H, "tokens": N, "head_dim": d, "bq": w.bq, "bk": w.bk,
                   "k_frac": w.k_frac, "p": w.p, "kept_block_density": round(density, 5),
                   "block_sparsity": round(1 - density, 5), "executed_tflop_per_step": round(flops / 1e12, 4),
                   "parallelism": "none (1 GPU)"},
        "ms_per_call": {"pool_qk": round(pool_ms, 4), "select_mask+row_order": round(select_ms, 4),
                        "fwd_lists": round(attn_ms, 4)},
        "ms_per_call_stats": stats,
        "tile_tflop_per_step": round(tile_flops / 1e12, 4),
        "fwd_tflops": round(attn_tflops, 2),
        "fwd_pct_bf16_peak": round(100 * attn_tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "roofline": {"kernel": "attn_fwd_kernel<bf16, 128, 128>", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_bytes": alg_bytes, "l2_hit_rate": l2_hit},
        "pool_gbs": round(2 * B * H * N * d * q.element_size() / (pool_ms * 1e-3) / 1e9, 1),
        "selection": selection,
        "input_generation_s": round(gen_s, 1),
    }
    if args.sweep_out:
        o_sw = torch.empty_like(q)  # the timed step's output in o stays for the parity stamp below
        with open(args.sweep_out, "w") as f:
            for kf in w.sweep or (1.0, 0.5, 0.25, 0.10, 0.05, 0.03):
                s2 = sa.select_mask(qp, kp, kf, 0.0, kept_lists=True)
                for _ in range(2):
                    sa.fwd_lists(q, k, v, s2["kept_idx"], s2["kept_cnt"], w.bq, w.bk, out=o_sw)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record()
                for _ in range(5):
                    sa.fwd_lists(q, k, v, s2["kept_idx"], s2["kept_cnt"], w.bq, w.bk, out=o_sw)
                b.record()
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / 5
                m2 = s2["mask"].cpu().numpy()
                fl = executed_flops(m2, N, w.bq, w.bk, d)
                rec = {"k_frac": kf, "p": 0.0, "density": float(m2.mean()), "fwd_ms": ms,
                       "fwd_tflops": fl / (ms * 1e-3) / 1e12}
                f.write(json.dumps(rec) + "\n")
                print(json.dumps(rec), file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        # the timed call's output for head 0, with its LSE from one more call on the same lists
        o2, lse = sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, return_lse=True,
                               row_order=order)
        torch.cuda.synchronize()
        same_o = bool(torch.equal(o2, o))
        parity, result["cpu_baseline"] = cpu_baseline(w, x, mask_cpu, args.cpu_sample_blocks,
                                                      o[:, :1].float().cpu(), lse[:, :1].float().cpu())
        parity["lse_call_output_equal"] = same_o
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
