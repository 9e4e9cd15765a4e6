"""GPU parity of the fixed-pattern masks, the window transpose and the two-pass SQuad attention
against the float64 oracle (oracle/patterns.py), through the C ABI."""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
import oracle
from oracle import patterns as pt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN = 2e-2, 5e-3

# (patterns, window, band, period)
PATTERNS = [
    (pt.LOCAL, 240, 0, 0),
    (pt.LOCAL, 100, 0, 0),
    (pt.GLOBAL, 240, 0, 0),
    (pt.GLOBAL, 37, 0, 0),
    (pt.DIAG, 0, 0, 0),
    (pt.DIAG, 0, 130, 0),
    (pt.MULTIDIAG, 0, 50, 700),
    (pt.MULTIDIAG, 0, 0, 333),
    (pt.STRIPE, 0, 0, 300),
    (pt.DIAG | pt.MULTIDIAG | pt.STRIPE, 0, 80, 1000),
    (pt.LOCAL | pt.GLOBAL, 250, 0, 0),
]


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("n,bq,bk", [(3000, 128, 64), (2500, 64, 64), (1000, 128, 128), (77, 64, 64)])
@pytest.mark.parametrize("pat", PATTERNS, ids=[f"p{p[0]}w{p[1]}b{p[2]}P{p[3]}" for p in PATTERNS])
def test_pattern_mask_matches_brute_force(n, bq, bk, pat):
    kinds, window, band, period = pat
    sel = sa.pattern_mask(kinds, 1, 2, n, bq, bk, window=window, band=band, period=period, device=DEV)
    ref = pt.pattern_block_mask(kinds, n, bq, bk, window=window, band=band, period=period)
    gm = sel["mask"].cpu().numpy()
    assert (gm == ref[None, None]).all()
    cnt, idx = sel["kept_cnt"].cpu().numpy(), sel["kept_idx"].cpu().numpy()
    for h in range(2):
        for i in range(ref.shape[0]):
            np.testing.assert_array_equal(idx[0, h, i, :cnt[0, h, i]], np.nonzero(ref[i])[0])


@pytest.mark.parametrize("pat", [(pt.LOCAL, 240, 0, 0), (pt.GLOBAL, 240, 0, 0),
                                 (pt.DIAG | pt.MULTIDIAG | pt.STRIPE, 0, 240, 3600)])
def test_pattern_mask_720p_rows(pat):
    """The 720p token count (21 x 45 x 80), sampled query blocks checked by brute force."""
    kinds, window, band, period = pat
    n, bq, bk = 75600, 128, 64
    sel = sa.pattern_mask(kinds, 1, 1, n, bq, bk, window=window, band=band, period=period, device=DEV,
                          kept_lists=False)
    rows = [0, 1, 17, 295, 296, 589, 590]
    ref = pt.pattern_block_mask(kinds, n, bq, bk, window=window, band=band, period=period, rows=rows)
    gm = sel["mask"].cpu().numpy()[0, 0]
    np.testing.assert_array_equal(gm[rows], ref[rows])
    print(f"  pattern {kinds}: density {gm.mean():.4f}", flush=True)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,w", [(2048, 64), (1000, 40), (75600, 240)])
def test_window_transpose_is_the_permutation(dt, n, w):
    g = torch.Generator().manual_seed(n)
    x = torch.randn(1, 2, n, 64, generator=g).to(dt).to(DEV)
    y = sa.window_transpose(x, w)
    perm = torch.from_numpy(pt.window_transpose(n, w)).to(DEV)
    assert torch.equal(y, x[:, :, perm])
    assert torch.equal(sa.window_transpose(y, w, inverse=True), x)


def _random_lists(B, H, nqb, nkb, density, g):
    """Kept lists (ascending) of a random block mask; query block 0 of head 0 keeps nothing."""
    m = torch.rand(B, H, nqb, nkb, generator=g) < density
    m[0, 0, 0] = False
    idx = torch.zeros(B, H, nqb, nkb, dtype=torch.int32)
    cnt = m.sum(-1).to(torch.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                kept = torch.nonzero(m[b, h, i]).flatten()
                idx[b, h, i, :kept.numel()] = kept.to(torch.int32)
    return idx.to(DEV), cnt.to(DEV)


@pytest.mark.parametrize("n,w,d,bq", [(4096, 32, 128, 128), (3000, 40, 128, 64), (4160, 65, 64, 128),
                                      (6400, 100, 64, 64), (75600, 240, 128, 128)])
def test_window_order_fwd_is_the_transposed_fwd(n, w, d, bq):
    """fwd_lists(window=w) reads the window-transposed order in place; it must give, bit for bit,
    the O and LSE of transposing Q, K, V, running fwd_lists and transposing back."""
    bk, H = 64, (1 if n > 10000 else 2)
    g = torch.Generator().manual_seed(n + w)
    q, k, v = (torch.randn(1, H, n, d, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    if n > 10000:
        _, mg = sa.squad_masks(1, H, n, w, bq, bk, DEV)
        idx, cnt = mg["kept_idx"], mg["kept_cnt"]
    else:
        idx, cnt = _random_lists(1, H, (n + bq - 1) // bq, (n + bk - 1) // bk, 0.3, g)
    o, lse = sa.fwd_lists(q, k, v, idx, cnt, bq, bk, return_lse=True, window=w)
    qt, kt, vt = (sa.window_transpose(t, w) for t in (q, k, v))
    ot, lt = sa.fwd_lists(qt, kt, vt, idx, cnt, bq, bk, return_lse=True)
    perm = torch.from_numpy(pt.window_transpose(n, w)).to(DEV)
    ref_lse = torch.empty_like(lt)
    ref_lse[:, :, perm] = lt
    assert torch.equal(o, sa.window_transpose(ot, w, inverse=True))
    assert torch.equal(lse, ref_lse)


@pytest.mark.parametrize("n,w,d,bq", [(2048, 64, 64, 128), (2048, 256, 128, 64), (1920, 240, 128, 128),
                                      (4096, 32, 128, 128), (3000, 40, 64, 64), (4800, 75, 128, 128),
                                      (3000, 120, 128, 64), (75600, 240, 128, 128)])
def test_squad_attention_matches_oracle(n, w, d, bq):
    """Token-exact SQuad ([SQ] "手法"): windows and position classes that do not align with the
    64- or 128-token blocks, so the kernel's tiles hold tokens of several windows. At 75 600
    tokens (the 720p grid, w = 240) the local pass is compared everywhere and the global pass on
    sampled positions (every token of each sampled position class)."""
    bk = 64
    H = 1 if n > 10000 else 2
    g = torch.Generator().manual_seed(w)
    q, k, v = (torch.randn(1, H, n, d, generator=g).to(torch.bfloat16) for _ in range(3))
    o, o_local = sa.squad_attention(q.to(DEV), k.to(DEV), v.to(DEV), w, bq, bk, return_local=True)
    positions = None if n <= 10000 else [0, 1, 63, 64, 127, 128, 200, w - 1]
    ro, rl, _, _ = pt.squad_attention(f64(q), f64(k), f64(v), w, 1.0 / math.sqrt(d), positions)
    el = np.abs(f64(o_local) - rl)
    rows = ~np.isnan(ro[0, 0, :, 0])
    e = np.abs(f64(o)[:, :, rows] - ro[:, :, rows])
    print(f"  squad n={n} w={w}: local max {el.max():.3e} mean {el.mean():.3e}; "
          f"global max {e.max():.3e} mean {e.mean():.3e} on {int(rows.sum())} rows", flush=True)
    assert el.max() <= O_MAX and el.mean() <= O_MEAN
    # the global pass reads the bf16-rounded local output as its values (relative 2^-9 each)
    assert e.max() <= O_MAX and e.mean() <= O_MEAN


@pytest.mark.parametrize("n,w,d,bq", [(4800, 75, 128, 128), (6400, 100, 64, 64), (75600, 240, 128, 128)])
def test_squad_global_in_place_is_the_transposed_local_pass(n, w, d, bq):
    """The global pass read in place equals, bit for bit, the local pass with windows of n / w over
    window-transposed copies of Q, K and V, transposed back (O and LSE)."""
    H = 1 if n > 10000 else 2
    g = torch.Generator().manual_seed(n - w)
    q, k, v = (torch.randn(1, H, n, d, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    o, lse = sa.squad_fwd(q, k, v, w, bq, True, return_lse=True)
    qt, kt, vt = (sa.window_transpose(t, w) for t in (q, k, v))
    ot, lt = sa.squad_fwd(qt, kt, vt, n // w, bq, False, return_lse=True)
    perm = torch.from_numpy(pt.window_transpose(n, w)).to(DEV)
    ref_lse = torch.empty_like(lt)
    ref_lse[:, :, perm] = lt
    assert torch.equal(o, sa.window_transpose(ot, w, inverse=True))
    assert torch.equal(lse, ref_lse)


def test_squad_lse_matches_oracle():
    """LSE of both passes against the oracle, within the bf16 rounding of P (ln(1 + 2^-8))."""
    n, w, d, bq = 7680, 120, 128, 64   # 64 windows: the global pass runs in place
    g = torch.Generator().manual_seed(21)
    q, k, v = (torch.randn(1, 2, n, d, generator=g).to(torch.bfloat16) for _ in range(3))
    ol, ll = sa.squad_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w, bq, False, return_lse=True)
    _, lg = sa.squad_fwd(q.to(DEV), k.to(DEV), ol, w, bq, True, return_lse=True)
    _, rl, rlse, rlse_l = pt.squad_attention(f64(q), f64(k), f64(v), w, 1.0 / math.sqrt(d))
    assert np.all(np.abs(f64(ll) - rlse_l) <= 1e-3 + math.log1p(2.0 ** -8))
    assert np.all(np.abs(f64(lg) - rlse) <= 1e-3 + math.log1p(2.0 ** -8))


def test_vdit_pattern_attention_matches_oracle():
    """Sparse-vDiT style union (diagonal band, the same band every `period` tokens, and the first
    key token of each period) through sparse_attn_fwd."""
    n, d, bq, bk = 3000, 128, 128, 64
    kinds, band, period = pt.DIAG | pt.MULTIDIAG | pt.STRIPE, 100, 1000
    g = torch.Generator().manual_seed(9)
    q, k, v = (torch.randn(1, 2, n, d, generator=g).to(torch.bfloat16) for _ in range(3))
    m = sa.pattern_mask(kinds, 1, 2, n, bq, bk, band=band, period=period, device=DEV, kept_lists=False)["mask"]
    o, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), m, bq, bk, return_lse=True)
    ref_m = pt.pattern_block_mask(kinds, n, bq, bk, band=band, period=period)
    ro, rl = oracle.masked_attention(f64(q), f64(k), f64(v), np.broadcast_to(ref_m, (1, 2) + ref_m.shape), bq, bk)
    e = np.abs(f64(o) - ro)
    assert e.max() <= O_MAX and e.mean() <= O_MEAN
    assert np.all(np.abs(f64(lse) - rl) <= 1e-3 + math.log1p(2.0 ** -8))
