"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Bars (stated for this method): pooled vectors and pooled probabilities agree to float64
rounding; masks agree bit for bit except rows the oracle classes as ties within 1e-6 of a
threshold (counted and printed, never mismatches); attention outputs are within 2e-2 max abs
and 5e-3 mean abs of the oracle. Small shapes cover several tiles and ragged tails; the
workload shapes run at full size with attention checked on sampled query blocks.
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
import oracle
from workloads import WORKLOADS, make_inputs, torch_dtype

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN = 2e-2, 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rand_qkv(B, H, N, d, dtype, seed, qk_scale=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (qk_scale * torch.randn(B, H, N, d, generator=g)).to(dtype)
    k = (qk_scale * torch.randn(B, H, N, d, generator=g)).to(dtype)
    v = torch.randn(B, H, N, d, generator=g).to(dtype)
    return q, k, v


# B, H, N, d, bq, bk, dtype, k_frac, p, seed
SMALL = [
    (1, 2, 1024, 64, 64, 64, torch.float32, 0.25, 0.6, 1),
    (1, 3, 1000, 128, 128, 64, torch.bfloat16, 0.2, 0.7, 2),
    (2, 2, 777, 64, 64, 64, torch.bfloat16, 0.3, 0.5, 3),
    (1, 2, 1100, 128, 64, 64, torch.float32, 0.1, 0.9, 4),
    (1, 2, 2500, 128, 128, 64, torch.bfloat16, 0.05, 0.9, 5),
    (1, 1, 100, 128, 128, 64, torch.bfloat16, 0.5, 0.5, 6),
    (1, 1, 1, 64, 64, 64, torch.float32, 0.0, 0.3, 7),
]
IDS = [f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}bq{c[4]}bk{c[5]}-{str(c[6])[6:]}" for c in SMALL]


def check_pool(q, k, bq, bk):
    qp, kp = sa.pool_qk(q, k, bq, bk)
    np.testing.assert_allclose(f64(qp), oracle.pool_blocks(f64(q), bq), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f64(kp), oracle.pool_blocks(f64(k), bk), rtol=1e-12, atol=1e-15)
    return qp, kp


def check_select(q, k, qp, kp, bq, bk, k_frac, p, lists=True):
    d = q.shape[-1]
    sel = sa.select_mask(qp, kp, k_frac, p, kept_lists=lists)
    ref_mask, info = oracle.block_mask(f64(q), f64(k), bq, bk, k_frac, p, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(f64(sel["probs"]), info["probs"], rtol=0, atol=1e-13)
    gm = sel["mask"].cpu().numpy()
    rep = oracle.compare_masks(info["probs"], ref_mask, gm, k_frac, p)
    print(f"  mask rows={rep['rows']} equal={rep['rows_equal']} ties={rep['ties']} "
          f"mismatches={rep['mismatches']} density={gm.mean():.4f}", flush=True)
    assert rep["mismatches"] == 0, rep["mismatch_rows"][:10]
    if lists:
        cnt = sel["kept_cnt"].cpu().numpy()
        idx = sel["kept_idx"].cpu().numpy()
        np.testing.assert_array_equal(cnt, gm.sum(-1))
        flat_m, flat_i, flat_c = gm.reshape(-1, gm.shape[-1]), idx.reshape(-1, idx.shape[-1]), cnt.reshape(-1)
        for r in range(flat_m.shape[0]):
            np.testing.assert_array_equal(flat_i[r, :flat_c[r]], np.nonzero(flat_m[r])[0])
    check_no_probs(qp, kp, k_frac, p, sel, lists)
    return sel, ref_mask, info


def check_no_probs(qp, kp, k_frac, p, sel, lists, scale=None):
    """Without the probabilities output the call gives the same mask and lists bit for bit."""
    s2 = sa.select_mask(qp, kp, k_frac, p, scale, kept_lists=lists, probs=False)
    assert "probs" not in s2
    assert torch.equal(s2["mask"], sel["mask"])
    if lists:
        assert torch.equal(s2["kept_cnt"], sel["kept_cnt"])
        m = sel["mask"].reshape(-1, sel["mask"].shape[-1])
        i1 = sel["kept_idx"].reshape(m.shape)
        i2 = s2["kept_idx"].reshape(m.shape)
        c = sel["kept_cnt"].reshape(-1)
        cols = torch.arange(m.shape[-1], device=m.device)[None, :]
        used = cols < c[:, None]  # entries past each row's count are unwritten
        assert torch.equal(torch.where(used, i1, 0), torch.where(used, i2, 0))


def fp32_bounds(q, k, v, n_keys):
    """Forward-error bounds of the fp32 path (fp32 matrix products, fp32 softmax, nothing rounded
    to bf16). With u = 2^-24 and g(n) = n u / (1 - n u):
      each logit scale * q.k carries at most dS = scale * g(d) * max|q| * max|k| (Cauchy-Schwarz
      on the sum of |q_i k_i|), plus the rounding of the exp2-domain scaling (|S| u, covered by the
      1e-5 slack);
      O moves by at most 2 dS max|V| through the softmax weights, and its two fp32 sums over n
      keys (numerator and denominator) by at most 2 g(n) max|V|;
      LSE moves by at most dS + g(n)."""
    qd, kd, vd = f64(q), f64(k), f64(v)
    d = qd.shape[-1]
    u = 2.0 ** -24
    g = lambda n: n * u / (1 - n * u)  # noqa: E731
    ds = g(d) * np.linalg.norm(qd, axis=-1).max() * np.linalg.norm(kd, axis=-1).max() / math.sqrt(d)
    vmax = np.abs(vd).max()
    return 2 * ds * vmax + 2 * g(n_keys) * vmax + 1e-5, ds + g(n_keys) + 1e-5


def check_attention(q, k, v, mask, bq, bk, blocks=None, lse_tol=None):
    o, lse = sa.fwd(q, k, v, mask, bq, bk, return_lse=True)
    mref = mask.cpu().numpy()
    ro, rl = oracle.masked_attention(f64(q), f64(k), f64(v), mref, bq, bk, blocks=blocks)
    sel = ~np.isnan(rl)
    go, gl = f64(o), f64(lse)
    err = np.abs(go[sel] - ro[sel])
    finite = np.isfinite(rl) & sel
    assert np.array_equal(np.isneginf(gl[sel]), np.isneginf(rl[sel]))
    lse_err = np.abs(gl[finite] - rl[finite]) if finite.any() else np.zeros(1)
    print(f"  attention rows={int(sel.sum())} max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
          f"lse_max={lse_err.max():.3e}", flush=True)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN
    if q.dtype == torch.float32:
        o_bound, lse_bound = fp32_bounds(q, k, v, q.shape[-2])
        assert err.max() <= o_bound, (err.max(), o_bound)
        assert lse_err.max() <= (lse_bound if lse_tol is None else lse_tol), (lse_err.max(), lse_bound)
    elif finite.any():
        # bf16 inputs reach the MFMA exactly, but the row sum l adds the bf16-rounded probabilities
        # that also multiply V (unit roundoff 2^-8 each), so LSE = m + ln l may be off by up to
        # ln(1 + 2^-8)
        tol = (1e-3 + math.log1p(2.0 ** -8)) if lse_tol is None else lse_tol
        assert np.all(lse_err <= tol)
    return o, lse


@pytest.mark.parametrize("case", SMALL, ids=IDS)
def test_small_end_to_end(case):
    B, H, N, d, bq, bk, dt, k_frac, p, seed = case
    print(f"case {case}", flush=True)
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, dt, seed))
    qp, kp = check_pool(q, k, bq, bk)
    sel, _, _ = check_select(q, k, qp, kp, bq, bk, k_frac, p)
    check_attention(q, k, v, sel["mask"], bq, bk)


@pytest.mark.parametrize("case", SMALL[:5], ids=IDS[:5])
def test_dense_mask_is_full_attention(case):
    B, H, N, d, bq, bk, dt, _, _, seed = case
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, dt, seed + 100))
    mask = torch.ones((B, H, -(-N // bq), -(-N // bk)), dtype=torch.uint8, device=DEV)
    check_attention(q, k, v, mask, bq, bk)


@pytest.mark.parametrize("case", SMALL[:5], ids=IDS[:5])
def test_random_masks(case):
    B, H, N, d, bq, bk, dt, _, _, seed = case
    # logits of scale 2 (|S| up to ~40): bf16 inputs enter the MFMA exactly, fp32 inputs run on
    # the fp32 matrix instruction
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, dt, seed + 200, qk_scale=2.0))
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, -(-N // bq), -(-N // bk))
    m = (torch.rand(shape, generator=g) < 0.3).to(torch.uint8)
    m[..., 0, :] = 0                  # first query block: no key block (empty row)
    m[..., -1, :] = 0
    m[..., -1, -1] = 1                # last query block: only the ragged last key block
    check_attention(q, k, v, m.to(DEV), bq, bk)


def test_empty_mask_gives_zero_and_neg_inf():
    q, k, v = (t.to(DEV) for t in rand_qkv(1, 2, 300, 128, torch.bfloat16, 9))
    m = torch.zeros((1, 2, 3, 5), dtype=torch.uint8, device=DEV)
    o, lse = sa.fwd(q, k, v, m, 128, 64, return_lse=True)
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()


def test_uniform_rows_keep_lowest_indices():
    # identical keys: every pooled probability is 1/nKB exactly, ties break to lower indices
    N, d = 1024, 64
    q = torch.randn(1, 1, N, d).to(DEV)
    k = torch.randn(1, 1, 1, d).expand(1, 1, N, d).contiguous().to(DEV)
    qp, kp = sa.pool_qk(q, k, 64, 64)
    sel = sa.select_mask(qp, kp, 0.25, 0.6)
    assert torch.all(sel["probs"] == 1.0 / 16).item()
    m = sel["mask"].cpu().numpy()[0, 0]
    assert (m[:, :10] == 1).all() and (m[:, 10:] == 0).all()
    check_no_probs(qp, kp, 0.25, 0.6, sel, False)


def test_repeatable_bitwise():
    q, k, v = (t.to(DEV) for t in rand_qkv(1, 4, 3000, 128, torch.bfloat16, 11))
    o1, m1 = sa.sparse_attention(q, k, v, 128, 64, 0.1, 0.8)
    o2, m2 = sa.sparse_attention(q, k, v, 128, 64, 0.1, 0.8)
    assert torch.equal(m1, m2) and torch.equal(o1, o2)


# ------------------------------------------------------------------------------ workloads

_CACHE = {}


def workload_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        w = WORKLOADS[name]
        x = make_inputs(w)
        _CACHE[name] = (w, x, tuple(t.to(DEV) for t in (x["q"], x["k"], x["v"])))
    return _CACHE[name]


def sample_blocks(w, x, heads, per_head_random=5, seed=0):
    """First block, ragged last block, the blocks holding boosted keys, and a few random ones."""
    nqb = -(-w.tokens // w.bq)
    rng = np.random.default_rng(seed)
    out = []
    for b in range(w.batch):
        for h in heads:
            blk = {0, nqb - 1}
            blk |= {s // w.bq for s in x["sinks"][(b, h)]}
            blk |= set(rng.choice(nqb, size=min(per_head_random, nqb), replace=False).tolist())
            out += [(b, h, i) for i in sorted(blk)]
    return out


@pytest.mark.parametrize("name,heads", [("tiny", None), ("stress", [0, 5, 8, 15]), ("wan480p", [0, 6, 11]),
                                        ("wan720p", [0, 13, 27, 39])])
def test_workload(name, heads):
    w, x, (q, k, v) = workload_inputs(name)
    print(f"workload {name}: {tuple(q.shape)} {q.dtype} k_frac={w.k_frac} p={w.p}", flush=True)
    qp, kp = check_pool(q, k, w.bq, w.bk)
    sel, _, _ = check_select(q, k, qp, kp, w.bq, w.bk, w.k_frac, w.p, lists=(name != "wan720p"))
    blocks = None if heads is None else sample_blocks(w, x, heads)
    check_attention(q, k, v, sel["mask"], w.bq, w.bk, blocks=blocks)


@pytest.mark.parametrize("k_frac", [1.0, 0.5, 0.25, 0.10, 0.05, 0.03])
def test_density_sweep(k_frac):
    w, x, (q, k, v) = workload_inputs("wan720p")
    w = WORKLOADS["sweep720p"]
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, k_frac, 0.0)
    m = sel["mask"]
    want = oracle.topk_count(k_frac, m.shape[-1])
    assert torch.all(m.sum(-1, dtype=torch.int64) == want).item()
    check_no_probs(qp, kp, k_frac, 0.0, sel, False)  # Top-k alone (p = 0) on the probs-free kernel
    check_attention(q, k, v, m, w.bq, w.bk, blocks=sample_blocks(w, x, [3, 30], per_head_random=2, seed=1))


def test_lists_path_matches_mask_path():
    """fwd_lists (the call the benchmark times) on the kept lists of select_mask gives the same
    bits as fwd on the mask, on the full 720p-shaped workload."""
    w, x, (q, k, v) = workload_inputs("wan720p")
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p, kept_lists=True)
    o1, l1 = sa.fwd(q, k, v, sel["mask"], w.bq, w.bk, return_lse=True)
    o2, l2 = sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_lists_out_of_range_entries_are_clamped(dt):
    """Entries outside [0, nKB) and counts above nKB are clamped: the call completes, reads
    nothing outside K and V, and rows whose entries are all valid are unaffected."""
    B, H, N, d, bq, bk = 1, 2, 1000, 128, 128, 64
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, dt, 11))
    nqb, nkb = -(-N // bq), -(-N // bk)
    idx = torch.arange(nkb, dtype=torch.int32).repeat(B, H, nqb, 1)
    cnt = torch.full((B, H, nqb), nkb, dtype=torch.int32)
    idx[0, 0, 1, :3] = torch.tensor([-7, 1 << 20, nkb], dtype=torch.int32)
    cnt[0, 1, 2] = 1 << 20
    cnt[0, 1, 3] = -4
    o = sa.fwd_lists(q, k, v, idx.to(DEV), cnt.to(DEV), bq, bk)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    full = torch.ones((B, H, nqb, nkb), dtype=torch.uint8, device=DEV)
    ref = sa.fwd(q, k, v, full, bq, bk)
    good = torch.ones((H, nqb), dtype=torch.bool)
    good[0, 1] = False
    good[1, 3] = False
    rows = good.repeat_interleave(bq, dim=1)[:, :N]
    assert torch.equal(o[0][rows.to(DEV)], ref[0][rows.to(DEV)])
    assert torch.equal(o[0, 1, 3 * bq:4 * bq], torch.zeros_like(o[0, 1, 3 * bq:4 * bq]))  # count -4 -> empty row


@pytest.mark.parametrize("H,nqb,nkb,d", [(7, 40, 300, 128), (3, 17, 1182, 64), (9, 33, 77, 128)])
def test_select_without_probs_on_uneven_groups(H, nqb, nkb, d):
    """The probs-free kernel takes 16 query-block rows per workgroup and hands the (head, group)
    items to the XCDs in contiguous ranges: item counts that are not a multiple of 8 (21, 6, 27)
    and a ragged last group must still select every row exactly once, as the two-kernel path and
    the oracle do."""
    g = torch.Generator().manual_seed(H * 1000 + nqb)
    base = torch.randn(1, H, 1, d, generator=g, dtype=torch.float64)
    qp = base + 0.5 * torch.randn(1, H, nqb, d, generator=g, dtype=torch.float64)
    kp = 0.4 * torch.randn(1, H, nkb, d, generator=g, dtype=torch.float64) + 0.6 * base
    qp, kp = qp.to(DEV), kp.to(DEV)
    scale = 1.0 / math.sqrt(d)
    sel = sa.select_mask(qp, kp, 0.05, 0.9, scale, kept_lists=True)
    probs = oracle.pooled_probabilities(f64(qp), f64(kp), scale)
    ref, _ = oracle.select_mask(probs, 0.05, 0.9)
    rep = oracle.compare_masks(probs, ref, sel["mask"].cpu().numpy(), 0.05, 0.9)
    assert rep["mismatches"] == 0, rep["mismatch_rows"][:10]
    check_no_probs(qp, kp, 0.05, 0.9, sel, True, scale)


@pytest.mark.parametrize("nkb,k_frac,p", [(1280, 0.03, 0.9), (1281, 0.03, 0.9), (2048, 0.03, 0.9),
                                          (2049, 0.03, 0.9), (3000, 0.1, 0.5),
                                          (8192, 0.01, 0.95)])
def test_select_long_rows(nkb, k_frac, p):
    """Rows of 2048 key blocks (the last size taken by one wave per row) and of 2049-8192 (one
    workgroup per row), on synthetic pooled vectors with a smooth key profile plus sinks."""
    B, H, nqb, d = 1, 2, 5, 64
    g = torch.Generator().manual_seed(nkb)
    base = torch.randn(B, H, 1, d, generator=g, dtype=torch.float64)
    qp = base + 0.5 * torch.randn(B, H, nqb, d, generator=g, dtype=torch.float64)
    t = torch.linspace(0, 6.283, nkb, dtype=torch.float64)
    kp = 0.3 * torch.randn(B, H, nkb, d, generator=g, dtype=torch.float64) \
        + torch.sin(t)[None, None, :, None] * base
    kp[..., ::997, :] *= 4.0  # a few sinks
    qp, kp = qp.to(DEV), kp.to(DEV)
    scale = 1.0 / math.sqrt(d)
    sel = sa.select_mask(qp, kp, k_frac, p, scale, kept_lists=True)
    probs = oracle.pooled_probabilities(f64(qp), f64(kp), scale)
    ref, _ = oracle.select_mask(probs, k_frac, p)
    np.testing.assert_allclose(f64(sel["probs"]), probs, rtol=0, atol=1e-13)
    gm = sel["mask"].cpu().numpy()
    rep = oracle.compare_masks(probs, ref, gm, k_frac, p)
    print(f"  nkb={nkb} rows={rep['rows']} equal={rep['rows_equal']} ties={rep['ties']} "
          f"mismatches={rep['mismatches']} kept/row={gm.sum(-1).mean():.1f}", flush=True)
    assert rep["mismatches"] == 0, rep["mismatch_rows"]
    cnt = sel["kept_cnt"].cpu().numpy().reshape(-1)
    idx = sel["kept_idx"].cpu().numpy().reshape(-1, nkb)
    flat = gm.reshape(-1, nkb)
    np.testing.assert_array_equal(cnt, flat.sum(-1))
    for r in range(flat.shape[0]):
        np.testing.assert_array_equal(idx[r, :cnt[r]], np.nonzero(flat[r])[0])
    if nkb <= sa.SELECT_FUSED_NKB:
        check_no_probs(qp, kp, k_frac, p, sel, True, scale)
    else:
        with pytest.raises(sa.SparseAttnError):
            sa.select_mask(qp, kp, k_frac, p, scale, kept_lists=True, probs=False)
