"""CPU pins of the semantic-aware permutation oracle (oracle/svg2.py): brute-force distances,
Lloyd's monotone objective, exact recovery of separated clusters, stability of the permutation,
closed forms of the size-weighted centroid probabilities, reductions to the pinned block-sparse
oracle and to dense attention, permutation equivalence, and planted mistakes."""

import math

import numpy as np
import pytest

import oracle
from oracle import svg2


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_init_is_evenly_spaced_tokens():
    x = np.arange(10.0)[None, None, :, None] * np.ones((1, 1, 10, 3))
    mu = svg2.init_centroids(x, 4)
    assert mu[0, 0, :, 0].tolist() == [1.0, 3.0, 6.0, 8.0]      # floor((2c + 1) 10 / 8)


def test_assign_is_brute_force_nearest_centroid():
    x = _rand((2, 2, 40, 5), 1)
    mu = _rand((2, 2, 7, 5), 2)
    got = svg2.kmeans_assign(x, mu)
    for b in range(2):
        for h in range(2):
            for t in range(40):
                d2 = [float(np.sum((x[b, h, t] - mu[b, h, c]) ** 2)) for c in range(7)]
                assert got[b, h, t] == int(np.argmin(d2))


def test_assign_tie_goes_to_lower_index():
    x = np.zeros((1, 1, 1, 2))
    mu = np.array([[[[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]]]])      # all at distance 1
    assert svg2.kmeans_assign(x, mu)[0, 0, 0] == 0


def test_update_is_mean_and_empty_cluster_stays():
    x = np.array([[[[0.0, 0.0], [2.0, 4.0], [10.0, 10.0]]]])
    labels = np.array([[[0, 0, 2]]])
    prev = np.array([[[[9.0, 9.0], [5.0, -5.0], [0.0, 0.0]]]])
    mu = svg2.kmeans_update(x, labels, prev)
    np.testing.assert_array_equal(mu[0, 0], [[1.0, 2.0], [5.0, -5.0], [10.0, 10.0]])


def test_lloyd_objective_never_increases():
    x = _rand((1, 2, 300, 6), 3)
    mu = svg2.init_centroids(x, 9)
    prev = math.inf
    for _ in range(6):
        labels = svg2.kmeans_assign(x, mu)
        obj = svg2.kmeans_objective(x, mu, labels)
        assert obj <= prev + 1e-9
        mu = svg2.kmeans_update(x, labels, mu)
        assert svg2.kmeans_objective(x, mu, labels) <= obj + 1e-9
        prev = svg2.kmeans_objective(x, mu, labels)


def test_separated_clusters_are_recovered():
    """Four tight blobs of 25 tokens each, contiguous in token order: the evenly spaced start
    takes one token from each blob, so one iteration finds the partition and the means."""
    rng = np.random.default_rng(4)
    centers = 100.0 * np.eye(4)
    x = np.concatenate([c + 0.01 * rng.standard_normal((25, 4)) for c in centers])[None, None]
    mu, labels = svg2.kmeans(x, 4, 2)
    assert labels[0, 0].tolist() == sum([[c] * 25 for c in range(4)], [])
    for c in range(4):
        np.testing.assert_allclose(mu[0, 0, c], x[0, 0, 25 * c:25 * (c + 1)].mean(0), atol=1e-12)


def test_permutation_is_stable_with_offsets():
    labels = np.array([[[2, 0, 2, 1, 0, 2]]])
    perm, off = svg2.cluster_permutation(labels, 4)
    assert perm[0, 0].tolist() == [1, 4, 3, 0, 2, 5]
    assert off[0, 0].tolist() == [0, 2, 3, 6, 6]


def test_size_weighted_probabilities_closed_form():
    cq = np.zeros((1, 1, 1, 3))
    ck = np.zeros((1, 1, 3, 3))
    ck[0, 0, 2] = [1.0, 0.0, 0.0]
    cq[0, 0, 0] = [2.0, 0.0, 0.0]
    p = svg2.cluster_probabilities(cq, ck, np.array([[[3, 1, 2]]]), 0.5)
    w = np.array([3.0, 1.0, 2.0 * math.e])                          # n_j exp(S_ij), S = 0, 0, 1
    np.testing.assert_allclose(p[0, 0, 0], w / w.sum(), rtol=1e-14)
    p0 = svg2.cluster_probabilities(cq, ck, np.array([[[3, 0, 2]]]), 0.5)
    assert p0[0, 0, 0, 1] == 0.0


def test_select_with_equal_sizes_is_the_block_select():
    """With equal cluster sizes the weights are the plain softmax of the centroid scores, so the
    selection is the pinned hybrid block selection with a Top-k of one."""
    cq, ck = _rand((1, 2, 6, 8), 5), _rand((1, 2, 20, 8), 6)
    scale = 0.3
    for p in (0.0, 0.3, 0.8, 1.0):
        mask, probs = svg2.cluster_select(cq, ck, np.full((1, 2, 20), 7), scale, p)
        want, _ = oracle.select_mask(oracle.pooled_probabilities(cq, ck, scale), 1.0 / 20, p)
        np.testing.assert_array_equal(mask, want)
        np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=1e-14)


def test_select_keeps_at_least_one_and_skips_empty():
    cq, ck = _rand((1, 1, 3, 4), 7), _rand((1, 1, 5, 4), 8)
    sizes = np.array([[[4, 0, 4, 4, 4]]])
    mask, _ = svg2.cluster_select(cq, ck, sizes, 1.0, 0.0)
    assert (mask.sum(-1) == 1).all()
    mask, _ = svg2.cluster_select(cq, ck, sizes, 1.0, 1.0)
    assert (mask[..., 1] == 0).all() and (mask.sum(-1) >= 1).all()


def test_contiguous_clusters_reduce_to_block_sparse_attention():
    """Labels t // bq and t // bk make clusters the positional blocks: the result is the pinned
    block-sparse oracle's."""
    q, k, v = (_rand((1, 2, 200, 8), s) for s in (9, 10, 11))
    bq, bk = 64, 32
    n = 200
    lq = np.broadcast_to(np.arange(n) // bq, (1, 2, n))
    lk = np.broadcast_to(np.arange(n) // bk, (1, 2, n))
    mask = (np.random.default_rng(12).random((1, 2, 4, 7)) < 0.5).astype(np.uint8)
    got, lse = svg2.cluster_attention(q, k, v, lq, lk, mask, 0.4)
    want, wlse = oracle.masked_attention(q, k, v, mask, bq, bk, 0.4)
    np.testing.assert_allclose(got, want, atol=1e-13)
    np.testing.assert_allclose(lse, wlse, atol=1e-13)


def test_all_pairs_kept_is_dense_attention():
    q, k, v = (_rand((1, 1, 50, 4), s) for s in (13, 14, 15))
    lq = np.random.default_rng(16).integers(0, 5, (1, 1, 50))
    lk = np.random.default_rng(17).integers(0, 3, (1, 1, 50))
    got, _ = svg2.cluster_attention(q, k, v, lq, lk, np.ones((1, 1, 5, 3), np.uint8), 0.5)
    s = 0.5 * q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(1, keepdims=True))
    want = (p / p.sum(1, keepdims=True)) @ v[0, 0]
    for i in range(5):
        rows = lq[0, 0] == i
        np.testing.assert_allclose(got[0, 0, rows], want[rows], atol=1e-13)


def test_permutation_equivalence():
    """Attention computed on the permuted tokens with contiguous clusters, then scattered back,
    equals attention in the original order (the page's mathematical equivalence)."""
    rng = np.random.default_rng(18)
    q, k, v = (_rand((1, 1, 120, 6), s) for s in (19, 20, 21))
    lq, lk = rng.integers(0, 4, (1, 1, 120)), rng.integers(0, 6, (1, 1, 120))
    mask = (rng.random((1, 1, 4, 6)) < 0.5).astype(np.uint8)
    mask[..., 0] = 1
    direct, _ = svg2.cluster_attention(q, k, v, lq, lk, mask, 0.3)
    pq, _ = svg2.cluster_permutation(lq, 4)
    pk, _ = svg2.cluster_permutation(lk, 6)
    qp, kp, vp = q[:, :, pq[0, 0]], k[:, :, pk[0, 0]], v[:, :, pk[0, 0]]
    out_p, _ = svg2.cluster_attention(qp, kp, vp, lq[:, :, pq[0, 0]], lk[:, :, pk[0, 0]], mask, 0.3)
    back = np.empty_like(out_p)
    back[:, :, pq[0, 0]] = out_p
    np.testing.assert_allclose(back, direct, atol=1e-13)


_REAL_PROBS = svg2.cluster_probabilities
_REAL_ASSIGN = svg2.kmeans_assign


def _probs_unweighted(cq, ck, sizes, scale):
    return _REAL_PROBS(cq, ck, np.where(np.asarray(sizes) > 0, 1, 0), scale)


def _assign_farthest(x, mu):
    return _REAL_ASSIGN(-np.asarray(x, dtype=np.float64), mu)


@pytest.mark.parametrize("mutant,target,test", [
    (_probs_unweighted, "cluster_probabilities", test_size_weighted_probabilities_closed_form),
    (_assign_farthest, "kmeans_assign", test_assign_is_brute_force_nearest_centroid),
])
def test_planted_mistakes_are_caught(monkeypatch, mutant, target, test):
    monkeypatch.setattr(svg2, target, mutant)
    with pytest.raises(AssertionError):
        test()
