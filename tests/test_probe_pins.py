"""CPU pins of the probe-fitted residual correction oracle (oracle/probes.py): closed forms,
recovery of an exactly affine residual, the ridge normal equations against a least-squares
routine, the subspace property, and planted mistakes."""

import math

import numpy as np
import pytest

import oracle
from oracle import probes as pr


def test_probe_positions():
    np.testing.assert_array_equal(pr.probe_blocks(75600, 128, 2), [147, 442])   # 590 full blocks
    np.testing.assert_array_equal(pr.probe_blocks(1024, 64, 4), [2, 6, 10, 14])
    assert pr.probe_blocks(100, 128, 3).tolist() == [0, 0, 0]                    # one partial block
    rows = pr.probe_rows(1000, 128, 2)                                           # 7 full blocks of 8
    assert rows.tolist() == list(range(128, 256)) + list(range(640, 768))


def test_exact_rows_are_dense_attention():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 2, 96, 8)) for _ in range(3))
    rows = np.array([5, 40, 95])
    got = pr.exact_rows(q, k, v, rows, 0.4)
    full, _ = oracle.masked_attention(q, k, v, np.ones((1, 2, 3, 3), np.uint8), 32, 32, 0.4)
    np.testing.assert_allclose(got, full[:, :, rows], atol=1e-13)


def test_zero_residual_gives_zero_correction():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal((1, 1, 50, 6))
    a = pr.fit_correction(xs, xs, 1e-3)
    assert np.abs(a).max() == 0.0
    o = rng.standard_normal((1, 1, 80, 6))
    np.testing.assert_array_equal(pr.apply_correction(o, a), o)


def test_affine_residual_is_recovered():
    """O_e = O_s + O_s A0 + b0 exactly: with a vanishing ridge the fit returns [A0; b0]."""
    rng = np.random.default_rng(3)
    xs = rng.standard_normal((2, 1, 200, 5))
    a0 = 0.1 * rng.standard_normal((2, 1, 6, 5))
    xe = xs + xs @ a0[:, :, :-1] + a0[:, :, -1:]
    a = pr.fit_correction(xs, xe, 1e-14)
    np.testing.assert_allclose(a, a0, atol=1e-9)
    o = rng.standard_normal((2, 1, 30, 5))
    np.testing.assert_allclose(pr.apply_correction(o, a), o + o @ a0[:, :, :-1] + a0[:, :, -1:], atol=1e-9)


def test_ridge_matches_least_squares_routine():
    """The normal equations with mu I equal lstsq on the system stacked with sqrt(mu) I."""
    rng = np.random.default_rng(4)
    xs = rng.standard_normal((1, 1, 40, 7))
    xe = xs + 0.2 * rng.standard_normal((1, 1, 40, 7))
    a = pr.fit_correction(xs, xe, 0.05)
    x = np.concatenate([xs[0, 0], np.ones((40, 1))], axis=1)
    mu = 0.05 * np.trace(x.T @ x) / 8
    big = np.concatenate([x, math.sqrt(mu) * np.eye(8)], axis=0)
    rhs = np.concatenate([xe[0, 0] - xs[0, 0], np.zeros((8, 7))], axis=0)
    want, *_ = np.linalg.lstsq(big, rhs, rcond=None)
    np.testing.assert_allclose(a[0, 0], want, atol=1e-12)


def test_correction_lies_in_the_residual_row_space():
    rng = np.random.default_rng(5)
    xs = rng.standard_normal((1, 1, 60, 8))
    basis = rng.standard_normal((2, 8))                  # residuals span a 2-d output subspace
    xe = xs + rng.standard_normal((1, 1, 60, 2)) @ basis
    a = pr.fit_correction(xs, xe, 1e-3)
    proj = np.linalg.pinv(basis) @ basis                 # projector on the residual row space
    np.testing.assert_allclose(a[0, 0] @ proj, a[0, 0], atol=1e-10)


def test_correction_reduces_probe_error():
    """On the probe rows themselves the fit cannot increase the squared error (ridge >= 0)."""
    rng = np.random.default_rng(6)
    b, h, n, d = 1, 2, 512, 16
    q, k, v = (rng.standard_normal((b, h, n, d)) for _ in range(3))
    mask = (rng.random((b, h, 8, 8)) < 0.3).astype(np.uint8)
    mask[..., np.arange(8), np.arange(8)] = 1
    os_, _ = oracle.masked_attention(q, k, v, mask, 64, 64)
    oc, a, rows, oe = pr.probe_corrected(q, k, v, os_, 64, 2, 1e-3)
    assert ((oc[:, :, rows] - oe) ** 2).sum() < ((os_[:, :, rows] - oe) ** 2).sum()


_REAL_FIT = pr.fit_correction


def _fit_without_bias(xs, xe, ridge):
    a = _REAL_FIT(xs, xe, ridge)
    a[:, :, -1] = 0.0
    return a


def _fit_residual_sign_flipped(xs, xe, ridge):
    return _REAL_FIT(xe, xs, ridge)


@pytest.mark.parametrize("mutant", [_fit_without_bias, _fit_residual_sign_flipped])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(pr, "fit_correction", mutant)
    with pytest.raises(AssertionError):
        test_affine_residual_is_recovered()


def _rank_case(seed, m=200, d=12, k=5, noise=0.05):
    """Probe rows whose residual has k dominant directions (singular values 8..4) plus noise."""
    rng = np.random.default_rng(seed)
    xs = rng.standard_normal((1, 1, m, d))
    u = np.linalg.qr(rng.standard_normal((m, k)))[0]
    w = np.linalg.qr(rng.standard_normal((d, k)))[0]
    r = u @ np.diag(np.linspace(8, 4, k)) @ w.T + noise * rng.standard_normal((m, d))
    return xs, xs + r[None, None], r


def test_full_rank_is_the_unprojected_fit():
    xs, xe, _ = _rank_case(11)
    d = xs.shape[-1]
    np.testing.assert_allclose(pr.fit_correction(xs, xe, 1e-3, rank=d), pr.fit_correction(xs, xe, 1e-3),
                               rtol=0, atol=1e-13)


def test_exactly_low_rank_residual_is_left_unchanged():
    """A residual of exact rank k: the unprojected map's rows already lie in its row space, so
    any rank >= k reproduces it."""
    xs, xe, _ = _rank_case(12, noise=0.0)
    full = pr.fit_correction(xs, xe, 1e-3)
    for r in (5, 7, 11):
        np.testing.assert_allclose(pr.fit_correction(xs, xe, 1e-3, rank=r), full, rtol=0, atol=1e-11)
    assert np.abs(pr.fit_correction(xs, xe, 1e-3, rank=3) - full).max() > 1e-3


def test_correction_rows_lie_in_top_singular_subspace():
    """Every correction row [O, 1] A lies in the span of the top-r right singular vectors of R,
    computed here by the SVD of R (a different routine from the oracle's eigendecomposition of
    R^T R), and the captured energy |R V_r|^2 is the sum of the r largest squared singular values
    (Eckart-Young)."""
    xs, xe, r = _rank_case(13)
    _, sv, wt = np.linalg.svd(r)
    for rank in (1, 3, 5):
        a = pr.fit_correction(xs, xe, 1e-3, rank=rank)
        basis = wt[:rank].T
        rows = np.concatenate([xs[0, 0], np.ones((xs.shape[2], 1))], axis=1) @ a[0, 0]
        np.testing.assert_allclose(rows - rows @ basis @ basis.T, 0.0, atol=1e-10)
        vr = pr.residual_subspace(r, rank)
        np.testing.assert_allclose(np.linalg.norm(r @ vr) ** 2, (sv[:rank] ** 2).sum(), rtol=1e-12)
        np.testing.assert_allclose(vr.T @ vr, np.eye(rank), atol=1e-12)


def test_rank_one_residual_closed_form():
    """R = u w^T: the subspace is the line of w, and with rank 1 the map is A_full w w^T / |w|^2."""
    rng = np.random.default_rng(14)
    m, d = 80, 6
    xs = rng.standard_normal((1, 1, m, d))
    u, w = rng.standard_normal(m), rng.standard_normal(d)
    xe = xs + np.outer(u, w)[None, None]
    full = pr.fit_correction(xs, xe, 1e-3)
    np.testing.assert_allclose(pr.fit_correction(xs, xe, 1e-3, rank=1), full @ np.outer(w, w) / (w @ w), atol=1e-12)


def _subspace_smallest(r, rank):
    evals, evecs = np.linalg.eigh(np.asarray(r, dtype=np.float64).T @ np.asarray(r, dtype=np.float64))
    return evecs[:, :rank]


_REAL_FIT_R = pr.fit_correction


def _fit_projection_dropped(xs, xe, ridge, rank=None):
    return _REAL_FIT_R(xs, xe, ridge, None)


@pytest.mark.parametrize("mutant", ["smallest", "dropped"])
def test_subspace_planted_mistakes_are_caught(monkeypatch, mutant):
    if mutant == "smallest":
        monkeypatch.setattr(pr, "residual_subspace", _subspace_smallest)
    else:
        monkeypatch.setattr(pr, "fit_correction", _fit_projection_dropped)
    with pytest.raises(AssertionError):
        test_correction_rows_lie_in_top_singular_subspace()
