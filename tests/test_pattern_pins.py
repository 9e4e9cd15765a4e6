"""CPU pins of the fixed-pattern oracle (oracle/patterns.py): closed forms of the block covers,
direct per-window / per-residue attention for the two SQuad passes, and planted mistakes that
the pins must catch."""

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


def _dense_softmax_attention(q, k, v, keep, scale):
    s = (q @ k.T) * scale
    s = np.where(keep, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v


def test_squad_passes_match_direct_token_attention():
    """Block-aligned windows, so the local block cover is the token window and the local pass is
    softmax attention inside each w-token window; the global pass, in the window-transposed order,
    is the block cover recomputed by hand."""
    rng = np.random.default_rng(5)
    n, d, w, bq, bk = 1024, 16, 128, 64, 64   # n / w = 8 tokens per position group
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    scale = 0.25
    o, o_local = pt.squad_attention(q, k, v, w, bq, bk, scale)
    t = np.arange(n)
    want_local = _dense_softmax_attention(q[0, 0], k[0, 0], v[0, 0], (t[:, None] // w) == (t[None, :] // w), scale)
    np.testing.assert_allclose(o_local[0, 0], want_local, rtol=0, atol=1e-12)
    # global pass: the n / w = 8 tokens of one position group are only 8 apart in the transposed
    # order, so the block cover (64-token blocks) keeps whole groups together with other groups;
    # the pin is therefore the block-cover definition, recomputed here by hand
    perm = pt.window_transpose(n, w)
    groups = (np.arange(n) // (n // w))
    keep_perm = (groups[:, None] // (bq // (n // w))) == (groups[None, :] // (bk // (n // w)))
    gp = _dense_softmax_attention(q[0, 0][perm], k[0, 0][perm], want_local[perm], keep_perm, scale)
    want = np.empty_like(gp)
    want[perm] = gp
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-12)


def test_squad_global_pass_is_same_position_attention_when_groups_fill_blocks():
    """When n / w equals the block size, each transposed block is exactly one position group, so
    the global pass is softmax attention among the tokens with the same position in their window."""
    rng = np.random.default_rng(6)
    n, d, bq = 64 * 8, 8, 64
    w = n // bq                                # n / w = 64 = block size
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    o, o_local = pt.squad_attention(q, k, v, w, bq, bq, 0.3)
    t = np.arange(n)
    want = _dense_softmax_attention(q[0, 0], k[0, 0], o_local[0, 0], (t[:, None] % w) == (t[None, :] % w), 0.3)
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(7)
    n, d, bq = 64 * 8, 8, 64
    w = n // bq
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    o_ok, o_local = pt.squad_attention(q, k, v, w, bq, bq, 0.3)
    # a transpose that forgets to regroup the positions
    monkeypatch.setattr(pt, "window_transpose", lambda n_, w_: np.arange(n_))
    o_bad, _ = pt.squad_attention(q, k, v, w, bq, bq, 0.3)
    assert np.abs(o_bad - o_ok).max() > 1e-3
    monkeypatch.undo()
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
