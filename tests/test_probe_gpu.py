"""GPU parity of the probe-fitted residual correction (sparse_attn_probe_correct) against the
float64 oracle (oracle/probes.py), through the C ABI.

Three checks per case, each against the oracle on the same inputs:
  exact rows   the dense attention of the probe rows: the attention bar, 2e-2 max / 5e-3 mean abs;
  fit          A against the oracle's fit of the GPU's own sparse and exact probe rows (the same
               float64 normal equations on the same numbers): 1e-5 of max |A| plus 1e-6. With a
               rank, the map is projected on the top eigenvectors of R^T R, which the GPU finds by
               fp32 Jacobi (off-diagonal mass below 1e-12 of the total): eigenvectors then err by
               about 1e-6 of the largest eigenvalue over the eigengap, so the bar adds
               2e-5 max|A_full| / gap (gap = (lambda_r - lambda_r+1) / lambda_1), where the gap
               is at least 1e-3; every case also checks that A has numerical rank <= rank;
  output       the corrected output against the oracle's end-to-end correction (its own exact
               rows and fit) of the GPU's sparse output: the attention bar, since the output is
               attention plus a correction fitted to the exact rows.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
from oracle import probes as pr
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL_MAX, ATOL_MEAN = 2e-2, 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(torch.bfloat16)


def _close(got, want, label):
    err = np.abs(got - want)
    print(f"  {label}: max {err.max():.3e}, mean {err.mean():.3e}", flush=True)
    assert err.max() <= ATOL_MAX and err.mean() <= ATOL_MEAN, label


def _valid_rows(n, bq, probes):
    """Positions, within the GPU's probes * bq exact rows, of the probe rows inside the sequence."""
    blocks = pr.probe_blocks(n, bq, probes)
    return np.concatenate([p * bq + np.arange(min(bq, n - b * bq)) for p, b in enumerate(blocks)])


def _check_rank(a_gpu, os_rows, ex_rows, ridge, rank, label):
    """The projected map against the oracle's, per head, and its numerical rank."""
    d = a_gpu.shape[-1]
    a_full = pr.fit_correction(os_rows, ex_rows, ridge)
    a_same = pr.fit_correction(os_rows, ex_rows, ridge, rank)
    for b in range(a_gpu.shape[0]):
        for h in range(a_gpu.shape[1]):
            r = ex_rows[b, h] - os_rows[b, h]
            lam = np.sort(np.linalg.eigvalsh(r.T @ r))[::-1]
            sv = np.linalg.svd(a_gpu[b, h], compute_uv=False)
            assert sv[rank:].max(initial=0.0) <= 1e-4 * sv[0] + 1e-7, (label, b, h, sv[:rank + 2])
            gap = (lam[rank - 1] - lam[rank]) / lam[0] if rank < d else 1.0
            err = np.abs(a_gpu[b, h] - a_same[b, h]).max()
            print(f"  {label} rank {rank} head ({b},{h}): gap {gap:.2e}, max |A| {np.abs(a_same[b, h]).max():.3e}, "
                  f"max err {err:.3e}", flush=True)
            if gap >= 1e-3:
                assert err <= 1e-5 * np.abs(a_same[b, h]).max() + 2e-5 * np.abs(a_full[b, h]).max() / gap + 1e-6


def run_case(q, k, v, mask, bq, probes, ridge, label, sample_rows=None, rank=None):
    B, H, N, d = q.shape
    qd, kd, vd, md = (t.to(DEV) for t in (q, k, v, mask))
    o_s = sa.fwd(qd, kd, vd, md, bq, 64)
    o_c = o_s.clone()
    _, a, exact = sa.probe_correct(qd, kd, vd, o_c, bq, probes, ridge, return_fit=True, rank=rank)
    torch.cuda.synchronize()
    rows = pr.probe_rows(N, bq, probes)
    valid = _valid_rows(N, bq, probes)
    os64 = f64(o_s)
    ex_ref = pr.exact_rows(f64(q), f64(k), f64(v), rows)
    ex_gpu = f64(exact)[:, :, valid]
    _close(ex_gpu, ex_ref, f"{label} exact rows")
    a_gpu = f64(a)
    if rank is None or rank >= d:
        a_same = pr.fit_correction(os64[:, :, rows], ex_gpu, ridge)
        err = np.abs(a_gpu - a_same).max()
        print(f"  {label} fit: max |A| {np.abs(a_same).max():.3e}, max err {err:.3e}", flush=True)
        assert err <= 1e-5 * np.abs(a_same).max() + 1e-6
    else:
        _check_rank(a_gpu, os64[:, :, rows], ex_gpu, ridge, rank, label)
    a_ref = pr.fit_correction(os64[:, :, rows], ex_ref, ridge, rank)
    sel = slice(None) if sample_rows is None else sample_rows
    want = pr.apply_correction(os64[:, :, sel], a_ref)
    _close(f64(o_c)[:, :, sel], want, f"{label} output")
    # the corrected output, applied with the GPU's own A, within bf16 rounding of the oracle's
    want_same = pr.apply_correction(os64[:, :, sel], a_gpu)
    err = np.abs(f64(o_c)[:, :, sel] - want_same)
    print(f"  {label} apply: max {err.max():.3e}, mean {err.mean():.3e}", flush=True)
    assert err.max() <= 8 * 2.0 ** -9 * max(1.0, np.abs(want_same).max())
    return o_s, o_c, a_gpu, rows, ex_ref


CASES = [  # B, H, N, d, bq, probes, density, seed
    (1, 2, 1024, 64, 64, 2, 0.3, 1),
    (1, 2, 1000, 128, 128, 3, 0.4, 2),
    (2, 1, 777, 64, 128, 1, 0.5, 3),
    (1, 2, 2500, 128, 64, 4, 0.2, 4),
    (1, 1, 100, 128, 128, 2, 1.0, 5),   # one partial block: both probes are block 0, rows past N
    (1, 1, 300, 64, 64, 9, 0.5, 6),     # more probes than full blocks: repeated probes
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}bq{c[4]}P{c[5]}" for c in CASES])
def test_probe_correct_random_masks(case):
    B, H, N, d, bq, probes, dens, seed = case
    q, k, v = (_rand((B, H, N, d), seed * 10 + i) for i in range(3))
    nqb, nkb = -(-N // bq), -(-N // 64)
    m = (torch.rand((B, H, nqb, nkb), generator=torch.Generator().manual_seed(seed)) < dens).to(torch.uint8)
    m[..., torch.arange(nqb), torch.clamp(torch.arange(nqb) * bq // 64, max=nkb - 1)] = 1
    run_case(q, k, v, m, bq, probes, 1e-3, str(case))


@pytest.mark.parametrize("rank", [1, 4, 16, 63])
@pytest.mark.parametrize("case", CASES[:4], ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}bq{c[4]}P{c[5]}" for c in CASES[:4]])
def test_probe_correct_rank(case, rank):
    """The map confined to the top principal directions of the probe residuals."""
    B, H, N, d, bq, probes, dens, seed = case
    q, k, v = (_rand((B, H, N, d), seed * 10 + i) for i in range(3))
    nqb, nkb = -(-N // bq), -(-N // 64)
    m = (torch.rand((B, H, nqb, nkb), generator=torch.Generator().manual_seed(seed)) < dens).to(torch.uint8)
    m[..., torch.arange(nqb), torch.clamp(torch.arange(nqb) * bq // 64, max=nkb - 1)] = 1
    run_case(q, k, v, m, bq, probes, 1e-3, f"{case} rank {rank}", rank=min(rank, d))


def test_probe_correct_planted_low_rank_residual():
    """Values with a strong shared component: the residuals of the dropped keys concentrate in
    a few output directions, so the eigengap is wide and the projected map is compared strictly."""
    B, H, N, d, bq = 1, 2, 2048, 128, 128
    q, k = (_rand((B, H, N, d), 300 + i) for i in range(2))
    g = torch.Generator().manual_seed(303)
    basis = torch.randn(3, d, generator=g)
    v = torch.randn(B, H, N, 3, generator=g) @ basis + 0.05 * torch.randn(B, H, N, d, generator=g)
    v = v / v.std()  # unit scale, as the attention bar assumes
    v = v.to(torch.bfloat16)
    m = (torch.rand((B, H, N // bq, N // 64), generator=g) < 0.15).to(torch.uint8)
    m[..., torch.arange(N // bq), torch.arange(N // bq) * 2] = 1
    run_case(q, k, v, m, bq, 2, 1e-3, "planted rank 3", rank=3)


def test_probe_correct_exact_mask_is_identity():
    """A full mask makes the sparse output exact: the residual is rounding only and the
    correction changes the output by a few bf16 units at most."""
    B, H, N, d, bq = 1, 2, 640, 128, 128
    q, k, v = (_rand((B, H, N, d), 90 + i) for i in range(3))
    m = torch.ones((B, H, N // bq, N // 64), dtype=torch.uint8)
    o_s, o_c, a, _, _ = run_case(q, k, v, m, bq, 2, 1e-3, "dense mask")
    assert np.abs(a).max() < 0.05
    assert (o_c - o_s).abs().max().item() <= 4 * 2.0 ** -8 * o_s.abs().max().item()


def test_probe_correct_is_repeatable():
    B, H, N, d, bq = 1, 2, 1500, 128, 128
    q, k, v = (_rand((B, H, N, d), 50 + i).to(DEV) for i in range(3))
    m = (torch.rand((B, H, 12, 24), generator=torch.Generator().manual_seed(3)) < 0.4).to(torch.uint8).to(DEV)
    o = sa.fwd(q, k, v, m, bq, 64)
    a, b = o.clone(), o.clone()
    sa.probe_correct(q, k, v, a, bq, 2, 1e-3)
    sa.probe_correct(q, k, v, b, bq, 2, 1e-3)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,heads", [("wan720p", [0, 39]), ("stress", [0, 9])])
def test_probe_correct_workload_sampled(name, heads):
    """Full-size workloads with the hybrid masks of select_mask and two probes: exact rows and
    the fit in full, the corrected output on sampled rows (the first and last query blocks, one
    in the middle)."""
    w = WORKLOADS[name]
    x = make_inputs(w, heads=heads)
    q, k, v = x["q"], x["k"], x["v"]
    N = q.shape[2]
    qd, kd = q.to(DEV), k.to(DEV)
    qp, kp = sa.pool_qk(qd, kd, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p)
    nqb = -(-N // w.bq)
    sample = np.concatenate([np.arange(b * w.bq, min(N, (b + 1) * w.bq)) for b in (0, nqb // 2, nqb - 1)])
    o_s, o_c, _, rows, ex_ref = run_case(q, k, v, sel["mask"].cpu(), w.bq, 2, 1e-3, name, sample_rows=sample)
    # and with the map confined to the top two principal directions of the residuals
    run_case(q, k, v, sel["mask"].cpu(), w.bq, 2, 1e-3, f"{name} rank 2", sample_rows=sample, rank=2)
    # on the probe rows the correction moves the output towards the exact rows
    e_before = ((f64(o_s)[:, :, rows] - ex_ref) ** 2).sum()
    e_after = ((f64(o_c)[:, :, rows] - ex_ref) ** 2).sum()
    print(f"  {name}: probe-row squared error {e_before:.4e} -> {e_after:.4e}", flush=True)
    assert e_after < e_before
