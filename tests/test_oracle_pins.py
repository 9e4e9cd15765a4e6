"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each ``check_*`` helper uses the oracle's functions at call time, so the mutation tests at the
end can swap in a plausible mistake and show that the matching pin catches it.

Cited pages: [SA2] "SpargeAttention2とは？…" (ai-papers.net); [SVG2] "Sparse VideoGen2 …"
(gist.science); [SPR] "Partition the Support, Reconstruct the Residual …" (physicalainews.jp).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_qkv(seed, b, h, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((b, h, n, d)), scale * rng.standard_normal((b, h, n, d)),
            rng.standard_normal((b, h, n, d)))


def _sdpa(q, k, v, keep_tokens=None):
    """torch's scaled_dot_product_attention in float64 on the CPU (default scale 1/sqrt(d))."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    am = None if keep_tokens is None else torch.from_numpy(keep_tokens)
    with torch.no_grad():
        return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am).numpy()


# ------------------------------------------------------------------ pooling ([SVG2] 1. 問題定義)

def check_pool_closed_form():
    # Token t carries the value t in every channel: the mean of a block of consecutive tokens is
    # the midpoint of its index range, and the partial last block averages its valid tokens only.
    n, d, bsz = 150, 3, 64
    x = np.broadcast_to(np.arange(n, dtype=np.float64)[None, None, :, None], (1, 2, n, d)).copy()
    got = oracle.pool_blocks(x, bsz)
    want = np.array([(0 + 63) / 2, (64 + 127) / 2, (128 + 149) / 2])
    assert got.shape == (1, 2, 3, d)
    np.testing.assert_array_equal(got[0, 1, :, 2], want)
    # constant rows pool to that constant
    c = np.full((1, 1, 70, 4), 3.25)
    np.testing.assert_array_equal(oracle.pool_blocks(c, 32), np.full((1, 1, 3, 4), 3.25))


def test_pool_closed_form():
    check_pool_closed_form()


def test_block_sizes():
    assert oracle.num_blocks(75600, 128) == 591 and oracle.num_blocks(75600, 64) == 1182
    assert oracle.block_sizes(75600, 128)[-1] == 80 and oracle.block_sizes(75600, 64)[-1] == 16
    assert oracle.block_sizes(32760, 128)[-1] == 120 and oracle.block_sizes(32760, 64)[-1] == 56


# ------------------------------------------------------------------ pooled probabilities

def check_pooled_two_block_logistic():
    # One query block against two key blocks with scores s and 0: the softmax of two entries is
    # the logistic function, p0 = 1 / (1 + exp(-s)), with s = scale * <qbar, kbar_0>.
    d = 4
    qp = np.array([[[[1.0, 2.0, 0.0, -1.0]]]])
    kp = np.array([[[[0.5, 1.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0]]]])
    scale = 1 / math.sqrt(d)
    s = scale * (0.5 + 2.0 + 0.0 - 2.0)
    got = oracle.pooled_probabilities(qp, kp, scale)
    assert got.shape == (1, 1, 1, 2)
    assert abs(got[0, 0, 0, 0] - 1 / (1 + math.exp(-s))) < 1e-15
    # A 3 x 5 case: rows are query blocks and sum to one over the key axis.
    rng = np.random.default_rng(3)
    qp = rng.standard_normal((1, 1, 3, d))
    kp = rng.standard_normal((1, 1, 5, d))
    p = oracle.pooled_probabilities(qp, kp, scale)
    assert p.shape == (1, 1, 3, 5)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-15)
    # agrees with torch.softmax on the same logits
    ref = torch.softmax(torch.from_numpy(scale * qp[0, 0] @ kp[0, 0].T), dim=-1).numpy()
    np.testing.assert_allclose(p[0, 0], ref, rtol=1e-14, atol=1e-16)


def test_pooled_two_block_logistic():
    check_pooled_two_block_logistic()


# ------------------------------------------------------------------ selection ([SA2], [SVG2] B)

def test_topk_counts_of_the_workloads():
    # ceil of the kept fraction, hand-computed for the workload shapes
    assert oracle.topk_count(0.25, 16) == 4
    assert oracle.topk_count(0.03, 512) == 16
    assert oracle.topk_count(0.05, 256) == 13
    assert oracle.topk_count(0.03, 1182) == 36
    assert [oracle.topk_count(f, 1182) for f in (1.0, 0.5, 0.25, 0.10, 0.05, 0.03)] == [1182, 591, 296, 119, 60, 36]
    assert oracle.topk_count(0.0, 1182) == 0


def _row_check(probs, k_frac, p, expect):
    probs = np.asarray(probs, dtype=np.float64)
    k = oracle.topk_count(k_frac, probs.size)
    mask, order, m_star, L = oracle.select_row(probs, k, p)
    assert k == expect["k"]
    assert m_star == expect["m_star"]
    assert L == expect["L"]
    assert sorted(np.nonzero(mask)[0].tolist()) == expect["kept"]


def check_golden_rows():
    g = _load("fig2_uniform_row.json")
    nkb = g["nkb"]
    # identical pooled keys -> exactly uniform probabilities
    qp = np.random.default_rng(0).standard_normal((1, 1, 1, 8))
    kp = np.broadcast_to(np.random.default_rng(1).standard_normal((1, 1, 1, 8)), (1, 1, nkb, 8)).copy()
    probs = oracle.pooled_probabilities(qp, kp, 0.3)[0, 0, 0]
    assert np.all(probs == 1.0 / nkb)
    _row_check(probs, g["k_frac"], g["p"], g["expect"])
    topk_only, _, _, _ = oracle.select_row(probs, oracle.topk_count(g["k_frac"], nkb), 0.0)
    assert np.nonzero(topk_only)[0].tolist() == g["expect"]["topk_alone_kept"]
    g = _load("fig3_skewed_row.json")
    _row_check(g["probs"], g["k_frac"], g["p"], g["expect"])
    for row in _load("hand_rows.json")["rows"]:
        _row_check(row["probs"], row["k_frac"], row["p"], row["expect"])


def test_golden_rows():
    check_golden_rows()


def _subsets(n):
    for r in range(n + 1):
        yield from itertools.combinations(range(n), r)


def check_bruteforce_selection(seed=0, trials=40):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        nkb = int(rng.integers(2, 11))
        logits = 2.5 * rng.standard_normal(nkb)
        probs = np.exp(logits - logits.max())
        probs /= probs.sum()
        k_frac = float(rng.choice([0.0, 0.1, 0.25, 0.5, 1.0]))
        p = float(rng.choice([0.0, 0.3, 0.6, 0.9, 0.97]))
        k = oracle.topk_count(k_frac, nkb)
        mask, _, m_star, L = oracle.select_row(probs, k, p)
        kept = set(np.nonzero(mask)[0].tolist())
        # Top-k alone: the k-subset of largest mass (unique: random probabilities have no ties)
        best_k = max(itertools.combinations(range(nkb), k), key=lambda s: probs[list(s)].sum())
        # Top-p alone: minimum cardinality of any subset whose mass reaches p
        if p <= 0:
            m_bf = 0
        else:
            m_bf = min(len(s) for s in _subsets(nkb) if probs[list(s)].sum() >= p - 1e-12)
        assert m_star == m_bf, (t, m_star, m_bf)
        best_p = max(itertools.combinations(range(nkb), m_bf), key=lambda s: probs[list(s)].sum())
        # union rule
        assert kept >= set(best_k) | set(best_p)
        assert len(kept) == L == max(k, m_bf)


def test_bruteforce_selection():
    check_bruteforce_selection()


def check_token_limit(seed=5):
    # With one token per block the block mask is p's token-level rule on the exact attention
    # probabilities of each query ([SA2] Top-k/Top-p definitions, stated per token).
    n, d = 10, 8
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    for k_frac, p in ((0.2, 0.6), (0.0, 0.8), (0.5, 0.0), (0.3, 0.95)):
        mask, info = oracle.block_mask(q, k, 1, 1, k_frac, p)
        attn = torch.softmax(torch.from_numpy(q[0, 0] @ k[0, 0].T / math.sqrt(d)), dim=-1).numpy()
        kk = math.ceil(k_frac * n - 1e-9)
        for t in range(n):
            pr = attn[t]
            topk = set(np.argsort(-pr)[:kk].tolist())
            m_bf = 0 if p <= 0 else min(len(s) for s in _subsets(n) if pr[list(s)].sum() >= p - 1e-12)
            topp = set(max(itertools.combinations(range(n), m_bf), key=lambda s: pr[list(s)].sum()))
            assert set(np.nonzero(mask[0, 0, t])[0].tolist()) == topk | topp


def test_token_limit():
    check_token_limit()


# ------------------------------------------------------------------ attention

def check_full_attention_is_sdpa():
    # All blocks kept (k_frac = 1): block-sparse attention is dense softmax attention.
    q, k, v = _rand_qkv(11, 1, 2, 200, 16)
    o, lse, mask, _ = oracle.sparse_attention(q, k, v, 64, 32, 1.0, 0.0)
    assert mask.all()
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(q @ np.swapaxes(k, -1, -2) / 4.0), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_full_attention_is_sdpa():
    check_full_attention_is_sdpa()


def check_masked_attention_is_sdpa_with_mask():
    # A random block mask expanded to tokens and handed to torch's attention as a boolean mask.
    n, d, bq, bk = 200, 16, 64, 32
    q, k, v = _rand_qkv(12, 1, 2, n, d)
    nqb, nkb = oracle.num_blocks(n, bq), oracle.num_blocks(n, bk)
    rng = np.random.default_rng(13)
    mask = (rng.random((1, 2, nqb, nkb)) < 0.4).astype(np.uint8)
    mask[..., 0] = 1  # every row keeps something (torch yields NaN for an empty row)
    o, _ = oracle.masked_attention(q, k, v, mask, bq, bk)
    tok = np.repeat(np.repeat(mask.astype(bool), bq, axis=2)[:, :, :n], bk, axis=3)[:, :, :, :n]
    np.testing.assert_allclose(o, _sdpa(q, k, v, tok), rtol=0, atol=1e-12)


def test_masked_attention_is_sdpa_with_mask():
    check_masked_attention_is_sdpa_with_mask()


def check_zero_query_closed_form():
    # Q = 0 makes every score 0: each query averages the V rows of its kept keys, and
    # LSE = log(number of kept keys). The partial last key block contributes only its valid keys.
    n, d, bq, bk = 150, 8, 64, 32        # key blocks of 32, 32, 32, 32, 22
    _, k, v = _rand_qkv(14, 1, 1, n, d)
    q = np.zeros_like(k)
    mask = np.zeros((1, 1, 3, 5), dtype=np.uint8)
    mask[0, 0, 0, [0, 4]] = 1
    mask[0, 0, 1, [4]] = 1
    mask[0, 0, 2, [1, 2]] = 1
    o, lse = oracle.masked_attention(q, k, v, mask, bq, bk)
    np.testing.assert_allclose(o[0, 0, 0], np.r_[v[0, 0, 0:32], v[0, 0, 128:150]].mean(0), atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 70], v[0, 0, 128:150].mean(0), atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 149], v[0, 0, 32:96].mean(0), atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(54)) < 1e-14
    assert abs(lse[0, 0, 64] - math.log(22)) < 1e-14
    assert abs(lse[0, 0, 140] - math.log(64)) < 1e-14


def test_zero_query_closed_form():
    check_zero_query_closed_form()


def test_row_stochastic_and_linear_in_v():
    q, k, v = _rand_qkv(15, 1, 2, 130, 8)
    mask, _ = oracle.block_mask(q, k, 64, 32, 0.25, 0.5)
    o1, _ = oracle.masked_attention(q, k, np.ones_like(v), mask, 64, 32)
    np.testing.assert_allclose(o1, 1.0, atol=1e-14)
    v2 = np.random.default_rng(16).standard_normal(v.shape)
    oa, _ = oracle.masked_attention(q, k, v, mask, 64, 32)
    ob, _ = oracle.masked_attention(q, k, v2, mask, 64, 32)
    oc, _ = oracle.masked_attention(q, k, 2 * v - 3 * v2, mask, 64, 32)
    np.testing.assert_allclose(oc, 2 * oa - 3 * ob, atol=1e-12)


def test_empty_rows():
    q, k, v = _rand_qkv(17, 1, 1, 96, 8)
    o, lse, mask, _ = oracle.sparse_attention(q, k, v, 32, 32, 0.0, 0.0)
    assert not mask.any()
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def check_block_permutation_equivalence():
    # [SVG2] "2. 手法" A: consistently permuting tokens leaves attention unchanged up to the
    # inverse permutation. Here whole blocks move: key blocks of K, V and mask columns together,
    # query blocks of Q and mask rows together.
    n, d, bq, bk = 256, 8, 64, 32
    q, k, v = _rand_qkv(18, 1, 1, n, d)
    rng = np.random.default_rng(19)
    mask = (rng.random((1, 1, 4, 8)) < 0.5).astype(np.uint8)
    mask[..., 3] = 1
    o, _ = oracle.masked_attention(q, k, v, mask, bq, bk)
    pk = rng.permutation(8)
    tok = (pk[:, None] * bk + np.arange(bk)[None]).reshape(-1)
    o2, _ = oracle.masked_attention(q, k[:, :, tok], v[:, :, tok], mask[..., pk], bq, bk)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    pq = rng.permutation(4)
    tq = (pq[:, None] * bq + np.arange(bq)[None]).reshape(-1)
    o3, _ = oracle.masked_attention(q[:, :, tq], k, v, mask[:, :, pq], bq, bk)
    np.testing.assert_allclose(o3, o[:, :, tq], atol=1e-13)
    # the pooled probabilities follow the same permutation of key blocks
    p1 = oracle.pooled_probabilities(oracle.pool_blocks(q, bq), oracle.pool_blocks(k, bk), 0.3)
    p2 = oracle.pooled_probabilities(oracle.pool_blocks(q, bq), oracle.pool_blocks(k[:, :, tok], bk), 0.3)
    np.testing.assert_allclose(p2, p1[..., pk], rtol=1e-13)


def test_block_permutation_equivalence():
    check_block_permutation_equivalence()


def test_executed_flops():
    n, d = 150, 8
    full = np.ones((1, 1, 3, 5), dtype=np.uint8)
    assert oracle.executed_flops(full, n, 64, 32, d) == 4 * d * n * n
    one = np.zeros_like(full)
    one[0, 0, 2, 4] = 1                     # 22 valid queries x 22 valid keys
    assert oracle.executed_flops(one, n, 64, 32, d) == 4 * d * 22 * 22


# ------------------------------------------------------------------ comparing masks with ties

def test_compare_masks_classifies_ties_and_mismatches():
    probs = np.array([[0.3, 0.2, 0.2 + 5e-7, 0.1, 0.1, 0.1 - 5e-7]])
    probs = probs / probs.sum()
    ref, _ = oracle.select_mask(probs, 0.34, 0.0)      # k = 3 -> {0, 2, 1}
    assert ref[0].tolist() == [1, 1, 1, 0, 0, 0]
    r = oracle.compare_masks(probs, ref, ref, 0.34, 0.0)
    assert r["rows_equal"] == 1 and r["ties"] == 0 and r["mismatches"] == 0
    # swapping two probabilities 1e-6 apart at the boundary is a tie ...
    alt = ref.copy()
    probs2 = np.array([[0.3, 0.2, 0.1, 0.1 + 4e-7, 0.2, 0.1]])
    probs2 /= probs2.sum()
    ref2, _ = oracle.select_mask(probs2, 0.6, 0.0)     # k = 4: keeps 0, 1, 4, 3 (0.1+4e-7 beats 0.1)
    assert ref2[0].tolist() == [1, 1, 0, 1, 1, 0]
    alt2 = ref2.copy()
    alt2[0, 3], alt2[0, 2] = 0, 1
    r = oracle.compare_masks(probs2, ref2, alt2, 0.6, 0.0)
    assert r["ties"] == 1 and r["mismatches"] == 0
    # ... dropping a clear winner is a mismatch
    alt[0, 0], alt[0, 3] = 0, 1
    r = oracle.compare_masks(probs, ref, alt, 0.34, 0.0)
    assert r["mismatches"] == 1
    # a running sum within 1e-6 of p may stop one block later: tie
    probs3 = np.array([[0.5, 0.25 - 2e-7, 0.25 + 2e-7]])
    ref3, info = oracle.select_mask(probs3, 0.0, 0.75)
    assert ref3[0].tolist() == [1, 0, 1] and info["m_star"][0] == 2
    longer = np.ones_like(ref3)
    r = oracle.compare_masks(probs3, ref3, longer, 0.0, 0.75)
    assert r["ties"] == 1 and r["mismatches"] == 0
    assert oracle.ambiguous_rows(probs3, 0.0, 0.75).tolist() == [0]


# ------------------------------------------------------------------ the pins catch planted mistakes

def _mutant_pool_divides_by_block_size(x, bsz):
    x = np.asarray(x, dtype=np.float64)
    b, h, n, d = x.shape
    nb = oracle.num_blocks(n, bsz)
    out = np.zeros((b, h, nb, d))
    for i in range(nb):
        out[:, :, i] = x[:, :, i * bsz:(i + 1) * bsz].sum(2) / bsz
    return out


def _mutant_softmax_wrong_axis(q_pool, k_pool, scale):
    s = scale * np.matmul(q_pool, np.swapaxes(k_pool, -1, -2))
    e = np.exp(s - s.max(axis=-2, keepdims=True))
    return e / e.sum(axis=-2, keepdims=True)


def _mutant_topp_strict(sorted_probs, p):
    if p <= 0:
        return 0
    c = np.cumsum(sorted_probs)
    hit = np.nonzero(c > p)[0]
    return int(hit[0]) + 1 if hit.size else len(sorted_probs)


def _mutant_order_high_index_first(prob_row):
    j = np.arange(prob_row.shape[0])
    return np.lexsort((-j, -prob_row))


def _mutant_attend_no_scale(q_blk, k_all, v_all, key_keep, scale):
    return orc.__dict__["_orig_attend_block"](q_blk, k_all, v_all, key_keep, 1.0)


def _mutant_attend_keeps_dropped(q_blk, k_all, v_all, key_keep, scale):
    return orc.__dict__["_orig_attend_block"](q_blk, k_all, v_all, np.ones_like(key_keep), scale)


@pytest.mark.parametrize("target,mutant,check", [
    ("pool_blocks", _mutant_pool_divides_by_block_size, check_pool_closed_form),
    ("pooled_probabilities", _mutant_softmax_wrong_axis, check_pooled_two_block_logistic),
    ("topp_count", _mutant_topp_strict, check_golden_rows),
    ("row_order", _mutant_order_high_index_first, check_golden_rows),
    ("attend_block", _mutant_attend_no_scale, check_full_attention_is_sdpa),
    ("attend_block", _mutant_attend_keeps_dropped, check_masked_attention_is_sdpa_with_mask),
])
def test_pins_catch_planted_mistakes(monkeypatch, target, mutant, check):
    monkeypatch.setitem(orc.__dict__, "_orig_attend_block", orc.attend_block)
    monkeypatch.setattr(orc, target, mutant)
    monkeypatch.setattr(oracle, target, mutant, raising=False)
    with pytest.raises(AssertionError):
        check()
