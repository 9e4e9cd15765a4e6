"""CPU pins of the fixed-pattern oracle (oracle/patterns.py): closed forms of the block covers,
the token-exact SQuad passes against torch float64 attention with dense token masks and closed
forms, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle
from oracle import patterns as pt


def _interval_distance(a0, a1, b0, b1):
    return max(0, b0 - a1, a0 - b1)


@pytest.mark.parametrize("n,bq,bk", [(1024, 128, 64), (1000, 128, 64), (777, 64, 64)])
def test_local_window_equal_to_query_block(n, bq, bk):
    """local(w = bq) with bk | bq: query block i keeps exactly the key blocks inside it."""
    m = pt.pattern_block_mask(pt.LOCAL, n, bq, bk, window=bq)
    nqb, nkb = m.shape
    want = np.zeros_like(m)
    for i in range(nqb):
        want[i, (i * bq) // bk: min(nkb, ((i + 1) * bq + bk - 1) // bk)] = 1
    np.testing.assert_array_equal(m, want)


@pytest.mark.parametrize("band", [0, 1, 63, 64, 65, 200])
def test_diagonal_is_interval_distance(band):
    n, bq, bk = 1000, 128, 64
    m = pt.pattern_block_mask(pt.DIAG, n, bq, bk, band=band)
    for i in range(m.shape[0]):
        for j in range(m.shape[1]):
            d = _interval_distance(i * bq, min(n, (i + 1) * bq) - 1, j * bk, min(n, (j + 1) * bk) - 1)
            assert m[i, j] == (d <= band), (i, j, band)


def test_stripe_columns():
    n, bq, bk, period = 1000, 128, 64, 300
    m = pt.pattern_block_mask(pt.STRIPE, n, bq, bk, period=period)
    cols = sorted({u // bk for u in range(0, n, period)})
    want = np.zeros(m.shape[1], dtype=np.uint8)
    want[cols] = 1
    assert (m == want[None, :]).all()


def test_multidiagonal_long_period_is_diagonal():
    n, bq, bk = 700, 64, 64
    a = pt.pattern_block_mask(pt.MULTIDIAG, n, bq, bk, band=70, period=2 * n)
    b = pt.pattern_block_mask(pt.DIAG, n, bq, bk, band=70)
    np.testing.assert_array_equal(a, b)


def test_multidiagonal_repeats_every_period():
    """With period a multiple of both block sizes, the mask is invariant under shifting both
    block indices by one period."""
    n, bq, bk, period = 2048, 128, 64, 512
    m = pt.pattern_block_mask(pt.MULTIDIAG, n, bq, bk, band=40, period=period)
    sq, sk = period // bq, period // bk
    np.testing.assert_array_equal(m[sq:, sk:], m[:-sq, :-sk])


def test_union_is_or_of_parts():
    n, bq, bk = 900, 128, 64
    kw = dict(window=200, band=30, period=300)
    parts = [pt.pattern_block_mask(k, n, bq, bk, **kw) for k in (pt.LOCAL, pt.DIAG, pt.STRIPE)]
    allm = pt.pattern_block_mask(pt.LOCAL | pt.DIAG | pt.STRIPE, n, bq, bk, **kw)
    np.testing.assert_array_equal(allm, parts[0] | parts[1] | parts[2])


def test_window_transpose_groups_positions():
    n, w = 96, 12
    perm = pt.window_transpose(n, w)
    assert sorted(perm.tolist()) == list(range(n))
    nw = n // w
    for s in range(n):
        assert perm[s] % w == s // nw and perm[s] // w == s % nw


def _sdpa_token_mask(q, k, v, keep, scale):
    """torch float64 scaled_dot_product_attention with a dense boolean token mask, and the LSE of
    the masked scores (an implementation independent of the oracle's)."""
    import torch
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = torch.from_numpy(keep)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    s = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    return o.numpy(), lse.numpy()


def _squad_by_sdpa(q, k, v, w, scale):
    n = q.shape[-2]
    t = np.arange(n)
    local = pt.token_pattern(pt.LOCAL, t[:, None], t[None, :], window=w)
    glob = pt.token_pattern(pt.GLOBAL, t[:, None], t[None, :], window=w)
    ol, ll = _sdpa_token_mask(q, k, v, local, scale)
    og, lg = _sdpa_token_mask(q, k, ol, glob, scale)
    return og, ol, lg, ll


# (n, w): windows that divide n, that do not (a last window of 1 token at 1000 / 37), that are not
# multiples of any block size, and the degenerate w = 1 and w = n
SQUAD_CASES = [(1000, 37), (333, 50), (768, 48), (240, 240), (96, 1), (130, 64)]


@pytest.mark.parametrize("n,w", SQUAD_CASES)
def test_squad_matches_token_mask_sdpa(n, w):
    """Both passes equal softmax attention with the dense token masks of [SQ] "手法": the local
    pass with floor(t / w) == floor(u / w), the global pass with t mod w == u mod w over the local
    output as values."""
    rng = np.random.default_rng(n + w)
    d = 16
    q, k, v = (rng.standard_normal((1, 2, n, d)) for _ in range(3))
    scale = 0.4
    o, o_local, lse, lse_local = pt.squad_attention(q, k, v, w, scale)
    ro, rl, rlse, rlse_l = _squad_by_sdpa(q, k, v, w, scale)
    np.testing.assert_allclose(o_local, rl, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_local, rlse_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


def test_squad_degenerate_windows_are_dense_attention():
    """w = 1: every token is its own window, so O_local = V exactly and the global pass, where all
    tokens share position 0, is dense attention over V. w = N: the local pass is dense attention
    and every token is alone at its position, so O = O_local."""
    rng = np.random.default_rng(11)
    n, d = 200, 8
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    dense, dl = _sdpa_token_mask(q, k, v, np.ones((n, n), dtype=bool), 0.5)
    o, o_local, _, _ = pt.squad_attention(q, k, v, 1, 0.5)
    assert np.array_equal(o_local, v)
    np.testing.assert_allclose(o, dense, rtol=0, atol=1e-12)
    o, o_local, lse, _ = pt.squad_attention(q, k, v, n, 0.5)
    np.testing.assert_allclose(o_local, dense, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(o, o_local)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,w", [(960, 40), (75600 // 105, 24)])
def test_squad_global_is_local_in_window_transposed_order(n, w):
    """Permuting tokens and permuting the outputs back leaves attention unchanged ([SVG2] "2. 手法"
    A): the global pass equals the local pass with windows of n / w in the window-transposed
    order, the form the GPU path runs when w divides n."""
    rng = np.random.default_rng(w)
    d = 8
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    og, lg = pt.squad_global(q, k, v, w, 0.3)
    perm = pt.window_transpose(n, w)
    op, lp = pt.squad_local(q[..., perm, :], k[..., perm, :], v[..., perm, :], n // w, 0.3)
    np.testing.assert_allclose(og[..., perm, :], op, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lg[..., perm], lp, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,w", [(100, 7), (96, 12), (75600, 240), (50, 64)])
def test_squad_pairs(n, w):
    if n <= 200:
        t = np.arange(n)
        want = int(pt.token_pattern(pt.LOCAL, t[:, None], t[None, :], window=w).sum()
                   + pt.token_pattern(pt.GLOBAL, t[:, None], t[None, :], window=w).sum())
        assert pt.squad_pairs(n, w) == want
    if n % w == 0:
        assert pt.squad_pairs(n, w) == n * w + n * n // w


def test_squad_sampled_positions_equal_full():
    rng = np.random.default_rng(3)
    n, w, d = 500, 23, 8
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    o, _, _, _ = pt.squad_attention(q, k, v, w, 0.3)
    pos = [0, 5, 22]
    os_, _, _, _ = pt.squad_attention(q, k, v, w, 0.3, positions=pos)
    rows = np.concatenate([np.arange(r, n, w) for r in pos])
    np.testing.assert_array_equal(os_[..., rows, :], o[..., rows, :])
    others = np.setdiff1d(np.arange(n), rows)
    assert np.isnan(os_[..., others, :]).all()


def test_squad_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(7)
    n, w, d, scale = 1000, 37, 8, 0.4
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    ro, rl, _, _ = _squad_by_sdpa(q, k, v, w, scale)

    def err():
        o, _, _, _ = pt.squad_attention(q, k, v, w, scale)
        return np.abs(o - ro).max()

    assert err() < 1e-12
    # the global pass reading V instead of the local output
    real_global = pt.squad_global
    monkeypatch.setattr(pt, "squad_global", lambda q_, k_, v_, w_, s_, p_=None: real_global(q_, k_, v, w_, s_, p_))
    assert err() > 1e-3
    monkeypatch.undo()
    # the block cover of the windows (64-token blocks) instead of the token windows
    real_local = pt.squad_local

    def block_cover_local(q_, k_, v_, w_, s_, windows=None):
        m = pt.pattern_block_mask(pt.LOCAL, n, 64, 64, window=w_)
        return oracle.masked_attention(q_, k_, v_, m[None, None], 64, 64, s_)
    monkeypatch.setattr(pt, "squad_local", block_cover_local)
    assert err() > 1e-3
    monkeypatch.setattr(pt, "squad_local", real_local)
    # same position taken as same window index in the global pass
    real_attend = pt._attend_set
    monkeypatch.setattr(pt, "squad_global",
                        lambda q_, k_, v_, w_, s_, p_=None: real_local(q_, k_, v_, -(-n // w_), s_))
    assert err() > 1e-3
    monkeypatch.undo()
    # a dropped softmax scale
    monkeypatch.setattr(pt, "_attend_set", lambda a, b, c, s_: real_attend(a, b, c, 1.0))
    assert err() > 1e-3


def test_planted_mistakes_are_caught(monkeypatch):
    # a transpose that forgets to regroup the positions breaks the transposed-order equivalence
    rng = np.random.default_rng(7)
    n, w = 96, 12
    q, k, v = (rng.standard_normal((1, 1, n, 8)) for _ in range(3))
    og, _ = pt.squad_global(q, k, v, w, 0.3)
    perm = np.arange(n)
    op, _ = pt.squad_local(q[..., perm, :], k[..., perm, :], v[..., perm, :], n // w, 0.3)
    assert np.abs(og[..., perm, :] - op).max() > 1e-3
    # a strict band comparison in the diagonal pattern
    real = pt.token_pattern
    monkeypatch.setattr(pt, "token_pattern",
                        lambda kinds, t, u, window=0, band=0, period=0: real(kinds, t, u, window, band - 1, period))
    bad = pt.pattern_block_mask(pt.DIAG, 1000, 128, 64, band=65)
    monkeypatch.undo()
    good = pt.pattern_block_mask(pt.DIAG, 1000, 128, 64, band=65)
    assert (bad != good).any()


def test_block_helpers_shared_definitions():
    assert pt.block_sizes is oracle.block_sizes
