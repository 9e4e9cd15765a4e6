"""GPU parity of the block-sparse attention backward (sparse_attn_bwd) against the float64 oracle
(oracle/backward.py), through the C ABI.

Bar, derived from the arithmetic. Each gradient element is a sum of products whose bf16
operands carry relative errors of at most u = 2^-8 each (round to nearest even): P is recomputed
from the saved LSE, which itself may be off by ln(1 + u) (the forward's row sum adds bf16 values),
and is rounded to bf16 before it multiplies (2u together); dS = P (dP - D) inherits those and is
rounded once more (3u), and D = rowsum(dO * O) reads the bf16-rounded O (u times
e = sum |dO O|, spread to dS by P). The fp32 accumulation adds orders of magnitude less. So
|err| <= 4u times the elementwise scale of masked_attention_bwd_scales (the products over
absolute values plus the D term), for each of dQ, dK, dV: the max bar. The mean bar is u times
the mean scale (rounding errors of independent terms do not all line up).
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
import oracle
from oracle import backward as bw
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_MAX, REL_MEAN = 4 * 2.0 ** -8, 2.0 ** -8


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(torch.bfloat16)


def check_grads(got, ref, scales, label=""):
    for name, a, b, sc in zip(("dQ", "dK", "dV"), got, ref, scales):
        sel = ~np.isnan(b)
        if not sel.any():
            continue
        err = np.abs(f64(a)[sel] - b[sel])
        s = sc[sel]
        print(f"  {label} {name}: max {err.max():.3e} (max err/scale {np.max(err / np.maximum(s, 1e-30)):.2e}), "
              f"mean {err.mean():.3e} (mean err / mean scale {err.mean() / s.mean():.2e}; "
              f"of mean|ref| {err.mean() / max(np.abs(b[sel]).mean(), 1e-30):.2e})", flush=True)
        assert (err <= REL_MAX * s + 1e-7).all() and err.mean() <= REL_MEAN * s.mean(), name


CASES = [  # B, H, N, d, bq, density, seed
    (1, 2, 1024, 64, 64, 0.3, 1),
    (1, 2, 1000, 128, 128, 0.4, 2),
    (2, 1, 777, 64, 128, 0.5, 3),
    (1, 2, 2500, 128, 64, 0.2, 4),
    (1, 1, 130, 128, 128, 1.0, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}bq{c[4]}" for c in CASES])
def test_bwd_random_masks(case):
    B, H, N, d, bq, dens, seed = case
    bk = 64
    q, k, v, g = (_rand((B, H, N, d), seed * 10 + i) for i in range(4))
    nqb, nkb = -(-N // bq), -(-N // bk)
    gen = torch.Generator().manual_seed(seed)
    m = (torch.rand((B, H, nqb, nkb), generator=gen) < dens).to(torch.uint8)
    if nqb > 1:
        m[0, 0, 1] = 0                    # a query block with no kept key block
    if nkb > 2:
        m[0, 0, :, 2] = 0                 # a key block nobody keeps
    m[..., -1, -1] = 1                    # the ragged corner
    qd, kd, vd, gd, md = (t.to(DEV) for t in (q, k, v, g, m))
    o, lse = sa.fwd(qd, kd, vd, md, bq, bk, return_lse=True)
    dq, dk, dv = sa.bwd(qd, kd, vd, o, gd, lse, md, bq, bk)
    torch.cuda.synchronize()
    args = (f64(q), f64(k), f64(v), m.numpy(), f64(g), bq, bk)
    ref = bw.masked_attention_bwd(*args)
    check_grads((dq, dk, dv), ref, bw.masked_attention_bwd_scales(*args), label=str(case))
    mn = m.numpy()
    for b in range(B):
        for h in range(H):
            for i in np.nonzero(mn[b, h].sum(1) == 0)[0]:      # query blocks with no kept key block
                assert (f64(dq)[b, h, i * bq:(i + 1) * bq] == 0).all()
            for j in np.nonzero(mn[b, h].sum(0) == 0)[0]:      # key blocks nobody keeps
                assert (f64(dk)[b, h, j * bk:(j + 1) * bk] == 0).all()
                assert (f64(dv)[b, h, j * bk:(j + 1) * bk] == 0).all()


def test_bwd_is_repeatable():
    B, H, N, d, bq, bk = 1, 2, 1500, 128, 128, 64
    q, k, v, g = (_rand((B, H, N, d), 50 + i).to(DEV) for i in range(4))
    m = (torch.rand((B, H, 12, 24), generator=torch.Generator().manual_seed(3)) < 0.4).to(torch.uint8).to(DEV)
    o, lse = sa.fwd(q, k, v, m, bq, bk, return_lse=True)
    a = sa.bwd(q, k, v, o, g, lse, m, bq, bk)
    b = sa.bwd(q, k, v, o, g, lse, m, bq, bk)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("name,heads,nq,nk", [("stress", [0, 9], 3, 3), ("wan720p", [0, 39], 2, 1)])
def test_bwd_workload_sampled(name, heads, nq, nk):
    """Full-size workloads with the hybrid masks of select_mask; dQ checked on sampled query
    blocks (the first, the ragged last, one in the middle) and dK / dV on sampled key blocks."""
    w = WORKLOADS[name]
    x = make_inputs(w, heads=heads)
    q, k, v = (t.to(DEV) for t in (x["q"], x["k"], x["v"]))
    B, H, N, d = q.shape
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p)
    o, lse = sa.fwd(q, k, v, sel["mask"], w.bq, w.bk, return_lse=True)
    g = _rand((B, H, N, d), 77).to(DEV)
    dq, dk, dv = sa.bwd(q, k, v, o, g, lse, sel["mask"], w.bq, w.bk)
    torch.cuda.synchronize()
    nqb, nkb = -(-N // w.bq), -(-N // w.bk)
    qsel = [(0, h, i) for h in range(H) for i in (0, nqb // 2, nqb - 1)[:nq]]
    ksel = [(0, h, j) for h in range(H) for j in (nkb - 1, nkb // 3, 0)[:nk]]
    args = (f64(x["q"]), f64(x["k"]), f64(x["v"]), sel["mask"].cpu().numpy(), f64(g), w.bq, w.bk)
    ref = bw.masked_attention_bwd(*args, q_blocks=qsel, k_blocks=ksel)
    scales = bw.masked_attention_bwd_scales(*args, q_blocks=qsel, k_blocks=ksel)
    check_grads((dq, dk, dv), ref, scales, label=name)
