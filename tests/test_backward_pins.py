"""CPU pins of the backward oracle (oracle/backward.py): torch float64 autograd of masked scaled
dot-product attention, central finite differences, zero-gradient special cases, and planted
mistakes that the pins must catch."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw


def _inputs(b, h, n, d, seed):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((b, h, n, d)) for _ in range(4))


def _token_mask(mask, n, bq, bk):
    return np.repeat(np.repeat(mask.astype(bool), bq, axis=-2), bk, axis=-1)[..., :n, :n]


def _torch_grads(q, k, v, g, mask, bq, bk, scale):
    """Autograd of torch's float64 scaled_dot_product_attention with the token-level mask; rows
    with no kept key are dropped from the loss (their output is defined as 0)."""
    n = q.shape[-2]
    tm = torch.from_numpy(_token_mask(mask, n, bq, bk))
    live = tm.any(-1, keepdim=True)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    safe = tm | ~live                      # keep the softmax finite on dead rows, then zero them
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=safe, scale=scale)
    o = torch.where(live, o, torch.zeros_like(o))
    (o * torch.from_numpy(g)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("n,d,bq,bk,density,seed", [(96, 8, 16, 8, 0.4, 1), (130, 16, 32, 16, 0.6, 2),
                                                     (64, 4, 64, 64, 1.0, 3), (75, 8, 16, 16, 0.3, 4)])
def test_matches_torch_autograd(n, d, bq, bk, density, seed):
    q, k, v, g = _inputs(2, 2, n, d, seed)
    rng = np.random.default_rng(seed + 10)
    mask = (rng.random((2, 2, oracle.num_blocks(n, bq), oracle.num_blocks(n, bk))) < density).astype(np.uint8)
    mask[0, 0, 0] = 0                      # an empty row
    scale = 1.0 / math.sqrt(d)
    got = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk, scale)
    want = _torch_grads(q, k, v, g, mask, bq, bk, scale)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


def test_finite_differences():
    n, d, bq, bk = 24, 4, 8, 8
    q, k, v, g = _inputs(1, 1, n, d, 7)
    mask = np.array([[[[1, 0, 1], [0, 1, 1], [1, 1, 0]]]], dtype=np.uint8)
    scale = 0.7

    def loss(q_, k_, v_):
        o, _ = oracle.masked_attention(q_, k_, v_, mask, bq, bk, scale)
        return float((o * g).sum())

    dq, dk, dv = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk, scale)
    eps = 1e-6
    rng = np.random.default_rng(8)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if name == "q" else q, xp if name == "k" else k, xp if name == "v" else v]
            args_m = [xm if name == "q" else q, xm if name == "k" else k, xm if name == "v" else v]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_zero_gradient_cases():
    n, d, bq, bk = 64, 8, 16, 16
    q, k, v, g = _inputs(1, 1, n, d, 9)
    mask = np.zeros((1, 1, 4, 4), dtype=np.uint8)
    mask[0, 0, 1, [0, 2]] = 1
    dq, dk, dv = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk)
    assert (dq[0, 0, :16] == 0).all() and (dq[0, 0, 32:] == 0).all()      # blocks with empty rows
    assert (dk[0, 0, 16:32] == 0).all() and (dv[0, 0, 48:] == 0).all()    # key blocks nobody keeps
    # V = constant: softmax rows sum to one, so dS sums to zero per row, dQ and dK vanish
    dq, dk, _ = bw.masked_attention_bwd(q, k, np.ones_like(v), np.ones((1, 1, 4, 4), np.uint8),
                                        g, bq, bk)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


def check_against_autograd():
    n, d, bq, bk = 48, 8, 16, 16
    q, k, v, g = _inputs(1, 1, n, d, 11)
    mask = np.array([[[[1, 0, 1], [1, 1, 0], [0, 1, 1]]]], dtype=np.uint8)
    scale = 1.0 / math.sqrt(d)
    got = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk, scale)
    want = _torch_grads(q, k, v, g, mask, bq, bk, scale)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


def _mutant(kind):
    """The backward with one plausible mistake planted."""
    def f(q, k, v, mask, dout, bq, bk, scale=None):
        q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        b_, h_, n, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for i in range(oracle.num_blocks(n, bq)):
            keep = np.repeat(np.asarray(mask[0, 0, i], dtype=bool), bk)[:n]
            if not keep.any():
                continue
            lo, hi = i * bq, min(n, (i + 1) * bq)
            s = scale * (q[0, 0, lo:hi] @ k[0, 0].T)
            s[:, ~keep] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            g = dout[0, 0, lo:hi]
            dv[0, 0] += p.T @ g
            dp = g @ v[0, 0].T
            if kind == "no_rowsum":
                ds = p * dp
            else:
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[0, 0, lo:hi] = (1.0 if kind == "dq_unscaled" else scale) * (ds @ k[0, 0])
            dk[0, 0] += scale * ((ds.T @ q[0, 0, lo:hi]) if kind != "dk_from_dp" else (dp.T @ q[0, 0, lo:hi]))
        return dq, dk, dv
    return f


@pytest.mark.parametrize("kind", ["no_rowsum", "dq_unscaled", "dk_from_dp"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    check_against_autograd()
    monkeypatch.setattr(bw, "masked_attention_bwd", _mutant(kind))
    with pytest.raises(AssertionError):
        check_against_autograd()


def test_sampled_blocks_equal_full():
    n, d, bq, bk = 130, 8, 32, 16
    q, k, v, g = _inputs(1, 2, n, d, 21)
    rng = np.random.default_rng(22)
    mask = (rng.random((1, 2, oracle.num_blocks(n, bq), oracle.num_blocks(n, bk))) < 0.5).astype(np.uint8)
    full = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk)
    qs, ks = [(0, 1, 2), (0, 0, 4)], [(0, 0, 3), (0, 1, 8), (0, 1, 0)]
    part = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk, q_blocks=qs, k_blocks=ks)
    for (b, h, i) in qs:
        np.testing.assert_allclose(part[0][b, h, i * bq:(i + 1) * bq], full[0][b, h, i * bq:(i + 1) * bq], atol=1e-13)
    for (b, h, j) in ks:
        for t in (1, 2):
            np.testing.assert_allclose(part[t][b, h, j * bk:(j + 1) * bk], full[t][b, h, j * bk:(j + 1) * bk],
                                       atol=1e-13)
    assert np.isnan(part[0][0, 0, 0]).all() and np.isnan(part[1][0, 0, 0]).all()


def test_error_scales_bound_the_gradients():
    """|x . y| <= |x| . |y| termwise: each scale is at least the magnitude of its gradient."""
    n, d, bq, bk = 96, 8, 32, 16
    q, k, v, g = _inputs(1, 2, n, d, 31)
    rng = np.random.default_rng(32)
    mask = (rng.random((1, 2, 3, 6)) < 0.6).astype(np.uint8)
    grads = bw.masked_attention_bwd(q, k, v, mask, g, bq, bk)
    scales = bw.masked_attention_bwd_scales(q, k, v, mask, g, bq, bk)
    for a, s in zip(grads, scales):
        assert (np.abs(a) <= s + 1e-12).all()
    part = bw.masked_attention_bwd_scales(q, k, v, mask, g, bq, bk, q_blocks=[(0, 1, 1)], k_blocks=[(0, 0, 2)])
    np.testing.assert_allclose(part[0][0, 1, 32:64], scales[0][0, 1, 32:64], atol=1e-13)
    np.testing.assert_allclose(part[1][0, 0, 32:48], scales[1][0, 0, 32:48], atol=1e-13)


def test_error_scales_closed_form_one_key():
    """One query attending to one key: P = 1 and O = V, so dP = D = dO.V and dS = 0. The gradients
    are dQ = dK = 0 and dV = dO; the scales reduce exactly to the D-spread term for dQ and dK,
    scale * e |K| and scale * e |Q| with e = sum_c |dO_c V_c|, and to |dO| for dV. Equality pins
    the scale function from both sides: a dropped D term gives zero, a doubled term twice the
    value."""
    rng = np.random.default_rng(41)
    d, sc = 8, 0.3
    q, k, v, g = (rng.standard_normal((1, 1, 1, d)) for _ in range(4))
    mask = np.ones((1, 1, 1, 1), dtype=np.uint8)
    dq, dk, dv = bw.masked_attention_bwd(q, k, v, mask, g, 1, 1, sc)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv, g, rtol=0, atol=1e-15)
    sq, sk, sv = bw.masked_attention_bwd_scales(q, k, v, mask, g, 1, 1, sc)
    e = np.abs(g * v).sum()
    np.testing.assert_allclose(sq, sc * e * np.abs(k), rtol=1e-14, atol=0)
    np.testing.assert_allclose(sk, sc * e * np.abs(q), rtol=1e-14, atol=0)
    np.testing.assert_allclose(sv, np.abs(g), rtol=1e-14, atol=0)


def test_error_scales_closed_form_two_tied_keys():
    """Two identical queries (same dO) and two identical keys: for each query P = (1/2, 1/2),
    O = (V_1 + V_2) / 2, dP_u = dO.V_u, D = (dP_1 + dP_2) / 2, so |dS_1| = |dS_2| = |dP_1 - dP_2| / 4.
    With e = sum_c |dO_c O_c|: scale(dQ_t) = scale (|dS_1| + e / 2) (|K_1| + |K_2|) for each query,
    and over the two queries scale(dK_u) = 2 scale (|dS_1| + e / 2) |Q| and scale(dV_u) = |dO|."""
    rng = np.random.default_rng(42)
    d, sc = 6, 0.7
    q0, k1, g0 = (rng.standard_normal(d) for _ in range(3))
    q = np.stack([q0, q0])[None, None]
    k = np.stack([k1, k1])[None, None]
    g = np.stack([g0, g0])[None, None]
    v = rng.standard_normal((1, 1, 2, d))
    mask = np.ones((1, 1, 1, 1), dtype=np.uint8)
    sq, sk, sv = bw.masked_attention_bwd_scales(q, k, v, mask, g, 2, 2, sc)
    dp = v[0, 0] @ g0
    ds1 = abs(dp[0] - dp[1]) / 4
    e = np.abs(g0 * (v[0, 0, 0] + v[0, 0, 1]) / 2).sum()
    np.testing.assert_allclose(sq[0, 0], np.stack([sc * (ds1 + e / 2) * 2 * np.abs(k1)] * 2), rtol=1e-13, atol=0)
    np.testing.assert_allclose(sk[0, 0], np.stack([2 * sc * (ds1 + e / 2) * np.abs(q0)] * 2), rtol=1e-13, atol=0)
    np.testing.assert_allclose(sv[0, 0], np.stack([np.abs(g0)] * 2), rtol=1e-13, atol=0)
