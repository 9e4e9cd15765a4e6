"""GPU parity of the semantic-aware permutation path (k-means, centroid Top-p, row permutation,
attention over variable-size blocks) against the float64 oracle (oracle/svg2.py), through the C
ABI. Every step is checked on the GPU's own inputs to that step:

  assignment   each label is a nearest centroid up to the rounding of the kernel's distances (the
               token in bf16 against the centroid split into two bf16 parts, fp32 sums): its
               float64 distance is within 1e-4 (|x|^2 + max |mu|^2) of the minimum;
  permutation  bit-exact: the stable sort of the GPU labels, and its offsets;
  update       the float64 mean of each cluster's tokens, rounded to fp32: 1e-6 relative;
  select       masses within 1e-12 relative, masks bit-exact except rows tied within 1e-6;
  permute      bit-exact row moves;
  attention    the attention bar, 2e-2 max / 5e-3 mean abs, in the original token order, and the
               forward's LSE bar, 1e-3 + log(1 + 2^-8).
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
import oracle
from oracle import svg2
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL_MAX, ATOL_MEAN = 2e-2, 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(torch.bfloat16)


def _smooth(shape, seed):
    """Tokens with clusters: a few random directions plus noise, so that k-means has structure."""
    g = torch.Generator().manual_seed(seed)
    B, H, N, d = shape
    centers = torch.randn(B, H, 12, d, generator=g) * 2.0
    pick = torch.randint(0, 12, (B, H, N), generator=g)
    x = torch.gather(centers, 2, pick[..., None].expand(B, H, N, d)) + 0.7 * torch.randn(B, H, N, d, generator=g)
    return x.to(torch.bfloat16)


def check_assignment(x, mu, labels):
    x, mu = f64(x), np.asarray(mu, np.float64)
    dist = (mu * mu).sum(-1)[:, :, None, :] - 2.0 * np.einsum("bhnd,bhcd->bhnc", x, mu)
    got = np.take_along_axis(dist, labels[..., None].astype(np.int64), -1)[..., 0]
    tol = 1e-4 * ((x * x).sum(-1) + (mu * mu).sum(-1).max(-1, keepdims=True))
    gap = got - dist.min(-1)
    exact = (labels == svg2.kmeans_assign(x, mu)).mean()
    print(f"  assignment: max gap/tol {np.max(gap / tol):.2e}, equal to the float64 argmin {exact:.4%}", flush=True)
    assert (gap <= tol).all()


def check_kmeans_step(x, C, init):
    """One GPU iteration from `init` (None: evenly spaced tokens) against the oracle's steps."""
    xd = x.to(DEV)
    init_t = None if init is None else torch.as_tensor(init, dtype=torch.float32).contiguous().to(DEV)
    out = sa.kmeans(xd, C, 1, init=init_t)
    torch.cuda.synchronize()
    mu0 = svg2.init_centroids(f64(x), C) if init is None else np.asarray(init, np.float64)
    labels = out["labels"].cpu().numpy()
    check_assignment(x, mu0, labels)
    perm, off = svg2.cluster_permutation(labels, C)
    np.testing.assert_array_equal(out["perm"].cpu().numpy(), perm)
    np.testing.assert_array_equal(out["offsets"].cpu().numpy(), off)
    want = svg2.kmeans_update(f64(x), labels, mu0)
    got = f64(out["centroids"])
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    return out


@pytest.mark.parametrize("B,H,N,d,C,seed", [(1, 2, 1000, 64, 16, 1), (1, 2, 777, 128, 40, 2), (2, 1, 3000, 128, 300, 3),
                                            (1, 1, 70, 64, 70, 4), (1, 1, 513, 128, 1, 5)])
def test_kmeans_steps(B, H, N, d, C, seed):
    x = _smooth((B, H, N, d), seed)
    out = check_kmeans_step(x, C, None)
    out2 = check_kmeans_step(x, C, f64(out["centroids"]))  # a warm start from the first iteration
    # several iterations in one call equal the same iterations one call at a time
    many = sa.kmeans(x.to(DEV), C, 3)
    one = sa.kmeans(x.to(DEV), C, 1)
    for _ in range(2):
        one = sa.kmeans(x.to(DEV), C, 1, init=one["centroids"])
    torch.cuda.synchronize()
    for key in ("labels", "perm", "offsets", "centroids"):
        assert torch.equal(many[key], one[key]), key
    del out2


def test_kmeans_is_repeatable():
    x = _smooth((1, 2, 2000, 128), 9).to(DEV)
    a, b = sa.kmeans(x, 100, 4), sa.kmeans(x, 100, 4)
    torch.cuda.synchronize()
    assert all(torch.equal(a[k], b[k]) for k in a)


def _select_check(cq, ck, off, p, label):
    mask, probs = sa.cluster_select(cq, ck, off, p, return_probs=True)
    torch.cuda.synchronize()
    sizes = np.diff(off.cpu().numpy().astype(np.int64), axis=-1)
    d = cq.shape[-1]
    want_m, want_p = svg2.cluster_select(f64(cq), f64(ck), sizes, 1.0 / np.sqrt(d), p)
    got_p = probs.cpu().numpy()
    np.testing.assert_allclose(got_p, want_p, rtol=1e-12, atol=1e-300)
    rep = oracle.compare_masks(want_p, want_m, mask.cpu().numpy(), 1.0 / want_p.shape[-1], p)
    print(f"  {label}: rows {rep['rows']}, equal {rep['rows_equal']}, ties {rep['ties']}, "
          f"mismatches {rep['mismatches']}, kept {mask.float().mean().item():.4f}", flush=True)
    assert rep["mismatches"] == 0
    return mask


@pytest.mark.parametrize("p", [0.0, 0.5, 0.9, 1.0])
def test_cluster_select(p):
    q, k = _smooth((1, 2, 3000, 128), 11), _smooth((1, 2, 3000, 128), 12)
    kq, kk = sa.kmeans(q.to(DEV), 50, 3), sa.kmeans(k.to(DEV), 200, 3)
    _select_check(kq["centroids"], kk["centroids"], kk["offsets"], p, f"p={p}")


def test_cluster_select_skips_empty_clusters():
    cq = torch.randn(1, 1, 5, 64).to(DEV)
    ck = torch.randn(1, 1, 9, 64).to(DEV)
    off = torch.tensor([[[0, 10, 10, 25, 25, 25, 40, 41, 60, 64]]], dtype=torch.int32).to(DEV)
    mask = _select_check(cq, ck, off, 1.0, "empty clusters")
    assert mask[..., [1, 3, 4]].sum().item() == 0


def test_permute_rows_round_trip():
    x = _rand((2, 3, 500, 64), 21).to(DEV)
    perm = torch.stack([torch.stack([torch.randperm(500, generator=torch.Generator().manual_seed(b * 3 + h))
                                     for h in range(3)]) for b in range(2)]).to(torch.int32).to(DEV)
    y = sa.permute_rows(x, perm)
    z = sa.permute_rows(y, perm, inverse=True)
    torch.cuda.synchronize()
    want = torch.gather(x.cpu(), 2, perm.cpu().long()[..., None].expand(-1, -1, -1, 64))
    assert torch.equal(y.cpu(), want)
    assert torch.equal(z, x)
    xf = torch.randn(1, 1, 77, 128).to(DEV)
    pf = torch.randperm(77).to(torch.int32)[None, None].to(DEV)
    assert torch.equal(sa.permute_rows(sa.permute_rows(xf, pf), pf, inverse=True), xf)


def check_cluster_attention(q, k, v, Cq, Ck, p, bq, label, mask_fn=None, sample=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    kq, kk = sa.kmeans(qd, Cq, 3), sa.kmeans(kd, Ck, 3)
    mask = sa.cluster_select(kq["centroids"], kk["centroids"], kk["offsets"], p)
    if mask_fn is not None:
        mask = mask_fn(mask)
    qp, kp, vp = sa.permute_rows(qd, kq["perm"]), sa.permute_rows(kd, kk["perm"]), sa.permute_rows(vd, kk["perm"])
    op, lsep = sa.cluster_fwd(qp, kp, vp, kq["offsets"], kk["offsets"], mask, bq, return_lse=True)
    o = sa.permute_rows(op, kq["perm"], inverse=True)
    lse = torch.empty_like(lsep)
    lse.scatter_(2, kq["perm"].long(), lsep)
    # reading Q / K / V and writing O / LSE through the permutations changes addressing only
    o2, lse2 = sa.cluster_fwd(qd, kp, vp, kq["offsets"], kk["offsets"], mask, bq, return_lse=True, q_perm=kq["perm"])
    o3, lse3 = sa.cluster_fwd(qd, kd, vd, kq["offsets"], kk["offsets"], mask, bq, return_lse=True, q_perm=kq["perm"],
                              k_perm=kk["perm"])
    o4 = sa.cluster_fwd(qp, kd, vd, kq["offsets"], kk["offsets"], mask, bq, k_perm=kk["perm"])
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse), "q_perm path differs from the permuted path"
    assert torch.equal(o3, o) and torch.equal(lse3, lse), "q_perm + k_perm path differs from the permuted path"
    assert torch.equal(o4, op), "k_perm path differs from the permuted path"
    lq, lk = kq["labels"].cpu().numpy(), kk["labels"].cpu().numpy()
    m = mask.cpu().numpy()
    want, wlse = svg2.cluster_attention(f64(q), f64(k), f64(v), lq, lk, m, clusters=sample)
    sel = ~np.isnan(want[..., 0])
    err = np.abs(f64(o)[sel] - want[sel])
    print(f"  {label}: kept pairs {m.mean():.4f}, max {err.max():.3e}, mean {err.mean():.3e}", flush=True)
    assert err.max() <= ATOL_MAX and err.mean() <= ATOL_MEAN
    g_lse, w_lse = f64(lse)[sel], wlse[sel]
    fin = np.isfinite(w_lse)
    assert (np.isfinite(g_lse) == fin).all()
    # the forward's LSE bar: the row sum adds the bf16-rounded weights the product uses
    assert np.abs(g_lse[fin] - w_lse[fin]).max() <= 1e-3 + np.log1p(2.0 ** -8)
    return o, mask, kq, kk


CASES = [  # B, H, N, d, Cq, Ck, p, bq, seed
    (1, 2, 1000, 64, 8, 40, 0.7, 64, 1),      # key clusters smaller than a key tile
    (1, 2, 1500, 128, 5, 6, 0.5, 128, 2),     # clusters larger than a query tile
    (2, 1, 2500, 128, 30, 250, 0.9, 128, 3),
    (1, 1, 333, 128, 333, 17, 0.6, 64, 4),    # one query per cluster
    (1, 2, 2048, 64, 20, 100, 1.0, 128, 5),   # every cluster with mass kept
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[2]}d{c[3]}Cq{c[4]}Ck{c[5]}p{c[6]}bq{c[7]}" for c in CASES])
def test_cluster_attention(case):
    B, H, N, d, Cq, Ck, p, bq, seed = case
    q, k = _smooth((B, H, N, d), seed * 10), _smooth((B, H, N, d), seed * 10 + 1)
    v = _rand((B, H, N, d), seed * 10 + 2)
    check_cluster_attention(q, k, v, Cq, Ck, p, bq, str(case))


def test_cluster_attention_empty_rows():
    """A query cluster with no kept key cluster gets O = 0 and LSE = -inf."""
    q, k, v = _smooth((1, 1, 800, 64), 31), _smooth((1, 1, 800, 64), 32), _rand((1, 1, 800, 64), 33)

    def drop(mask):
        mask = mask.clone()
        mask[0, 0, 1] = 0
        return mask
    o, mask, kq, _ = check_cluster_attention(q, k, v, 6, 20, 0.8, 64, "empty row", mask_fn=drop)
    rows = (kq["labels"][0, 0] == 1).cpu()
    assert rows.any() and (o[0, 0].cpu()[rows] == 0).all()


def test_svg2_attention_matches_steps():
    q, k, v = _smooth((1, 2, 1200, 128), 41), _smooth((1, 2, 1200, 128), 42), _rand((1, 2, 1200, 128), 43)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, info = sa.svg2_attention(qd, kd, vd, 10, 60, 3, 0.9, return_info=True)
    torch.cuda.synchronize()
    want, _ = svg2.cluster_attention(f64(q), f64(k), f64(v), info["kmeans_q"]["labels"].cpu().numpy(),
                                     info["kmeans_k"]["labels"].cpu().numpy(), info["mask"].cpu().numpy())
    err = np.abs(f64(o) - want)
    assert err.max() <= ATOL_MAX and err.mean() <= ATOL_MEAN


@pytest.mark.parametrize("name,heads", [("wan720p", [0, 39]), ("stress", [0, 9])])
def test_svg2_workload_sampled(name, heads):
    """Full-size workloads: 128 query and 256 key clusters, 3 iterations, p = 0.9; the attention
    checked on three query clusters per head (the first, a middle one, the last)."""
    w = WORKLOADS[name]
    x = make_inputs(w, heads=heads)
    q, k, v = x["q"], x["k"], x["v"]
    H = q.shape[1]
    sample = [(0, h, i) for h in range(H) for i in (0, 64, 127)]
    check_cluster_attention(q, k, v, 128, 256, 0.9, 128, name, sample=sample)
