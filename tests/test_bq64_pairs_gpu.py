"""GPU checks of the forward on 64-query blocks, which for d = 128 runs them two at a time on the
4-wave kernel over the union of the pair's kept lists (through the C ABI; d = 64 keeps the one-row
kernel, for which the same properties hold trivially).

A row's result must not depend on its partner's list: each wave scores the blocks its own row does
not keep at -inf, which adds exactly nothing. So changing only the partner rows' lists must leave
a row's output and LSE bit for bit unchanged. The cases cover disjoint, identical and nested
lists, empty rows on either side, a partner row past the end (an odd number of 64-query blocks),
a ragged last key block kept by one row only, and both head dimensions; each call is also checked
against the float64 oracle. Above the union's size limit (4096 key blocks) the one-row kernel
runs instead; one case checks it on sampled query blocks.
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN = 2e-2, 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rand_qkv(B, H, N, d, seed, qk_scale=2.0):
    g = torch.Generator().manual_seed(seed)
    q = (qk_scale * torch.randn(B, H, N, d, generator=g)).to(torch.bfloat16)
    k = (qk_scale * torch.randn(B, H, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    return q, k, v


def lists_of(mask):
    m = mask.cpu()
    nkb = m.shape[-1]
    cnt = m.sum(-1, dtype=torch.int32)
    order = torch.argsort((1 - m.to(torch.int64)) * nkb + torch.arange(nkb), dim=-1, stable=True).to(torch.int32)
    return order.contiguous().to(DEV), cnt.contiguous().to(DEV)


def run(q, k, v, mask):
    idx, cnt = lists_of(mask)
    o, lse = sa.fwd_lists(q, k, v, idx, cnt, 64, 64, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def check_oracle(q, k, v, mask, o, lse, blocks=None):
    ro, rl = oracle.masked_attention(f64(q), f64(k), f64(v), mask.numpy(), 64, 64, blocks=blocks)
    sel = ~np.isnan(rl)
    go, gl = f64(o), f64(lse)
    err = np.abs(go[sel] - ro[sel])
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, (err.max(), err.mean())
    assert np.array_equal(np.isneginf(gl[sel]), np.isneginf(rl[sel]))
    fin = np.isfinite(rl) & sel
    if fin.any():
        assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-3 + math.log1p(2.0 ** -8))


def rows_of(mask, even):
    """Token rows of the 64-query blocks of the given parity."""
    n = mask.shape[2]
    return [i for i in range(n) if (i % 2 == 0) == even]


def token_rows(blocks, N):
    r = torch.zeros(N, dtype=torch.bool)
    for i in blocks:
        r[i * 64:min(N, (i + 1) * 64)] = True
    return r


# B, H, N, d, density, seed
CASES = [
    (1, 2, 1000, 128, 0.3, 1),   # 16 blocks of 64: 8 whole pairs, ragged key tail
    (1, 2, 1050, 128, 0.4, 2),   # 17 blocks: the last pair has no partner row
    (2, 1, 777, 64, 0.5, 3),
    (1, 3, 2500, 128, 0.1, 4),
    (1, 1, 64, 64, 1.0, 5),      # one block, no partner
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}" for c in CASES])
def test_partner_list_does_not_change_a_row(case):
    B, H, N, d, dens, seed = case
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, seed))
    nqb, nkb = -(-N // 64), -(-N // 64)
    g = torch.Generator().manual_seed(seed)
    m1 = (torch.rand((B, H, nqb, nkb), generator=g) < dens).to(torch.uint8)
    if nqb > 3:
        m1[..., 0, :] = 0                      # empty row with a non-empty partner
        m1[..., 2, :] = m1[..., 3, :]          # identical lists
        m1[..., 1, -1] = 1                     # the ragged last key block kept by one row only
        m1[..., 0, -1] = 0
    o1, l1 = run(q, k, v, m1)
    check_oracle(q.cpu(), k.cpu(), v.cpu(), m1, o1, l1)
    for even in (True, False):
        # change the partners of the rows of one parity: new random lists, disjoint where possible
        m2 = m1.clone()
        other = rows_of(m1, not even)
        m2[..., other, :] = 1 - m1[..., other, :]
        o2, l2 = run(q, k, v, m2)
        keep = token_rows(rows_of(m1, even), N).to(DEV)
        assert torch.equal(o1[:, :, keep], o2[:, :, keep]) and torch.equal(l1[:, :, keep], l2[:, :, keep])
        check_oracle(q.cpu(), k.cpu(), v.cpu(), m2, o2, l2)


def test_all_partner_rows_empty():
    B, H, N, d = 1, 2, 1280, 128
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, 11))
    g = torch.Generator().manual_seed(11)
    m = (torch.rand((B, H, 20, 20), generator=g) < 0.3).to(torch.uint8)
    m[..., 1::2, :] = 0
    o, lse = run(q, k, v, m)
    empty = token_rows(range(1, 20, 2), N).to(DEV)
    assert torch.all(o[:, :, empty] == 0).item() and torch.all(torch.isneginf(lse[:, :, empty])).item()
    check_oracle(q.cpu(), k.cpu(), v.cpu(), m, o, lse)


def test_above_union_limit_runs_one_row_kernel():
    """4097 key blocks: above the paired walk's limit, the one-row kernel serves 64-query blocks."""
    B, H, d = 1, 1, 128
    N = 4097 * 64 - 13
    q, k, v = (t.to(DEV) for t in rand_qkv(B, H, N, d, 12, qk_scale=1.0))
    nqb = nkb = -(-N // 64)
    g = torch.Generator().manual_seed(12)
    m = torch.zeros((B, H, nqb, nkb), dtype=torch.uint8)
    cols = torch.randint(0, nkb, (nqb, 6), generator=g)
    m[0, 0].scatter_(1, cols, 1)
    m[0, 0, :, nkb - 1] = 1
    m[0, 0, torch.arange(nqb), torch.arange(nqb)] = 1
    o, lse = run(q, k, v, m)
    blocks = [(0, 0, i) for i in (0, 1, 2, 1000, 2047, nqb - 2, nqb - 1)]
    check_oracle(q.cpu(), k.cpu(), v.cpu(), m, o, lse, blocks=blocks)
