"""GPU checks of the rows' work order (sparse_attn_row_order) and of the ordered forward
(sparse_attn_fwd_lists_ordered), through the C ABI.

The order is scheduling only, so the checks are exact: it is a permutation of the rows; on
short grids (fewer than 8192 rows) workgroup 8 l + x takes the row of rank l among the rows
that XCD x walks by default, ranked by descending kept count with ties in default order; on
long grids it is the default order; and the ordered forward equals the plain one bit for bit.
The default order is restated here from its definition: XCD x takes chunks x, x + 8, ... of 128
consecutive rows, rows outside whole chunks split into one piece per XCD, and the rows past
the eight equal shares in place."""

import numpy as np
import pytest
import torch

import block_sparse_attention_query_amd as sa
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def default_row(w, n, chunk=128):
    per = n // 8
    if w >= per * 8:
        return w
    x, l = w % 8, w // 8
    full = per // chunk
    c, off = divmod(l, chunk)
    if c < full:
        return (c * 8 + x) * chunk + off
    return full * 8 * chunk + x * (per - full * chunk) + off


@pytest.mark.parametrize("rows", [3, 8, 100, 1000, 3072, 8191, 8192, 23640])
def test_row_order_is_longest_first_per_xcd(rows):
    g = torch.Generator().manual_seed(rows)
    cnt = torch.randint(0, 40, (1, 1, rows), generator=g, dtype=torch.int32)
    order = sa.row_order(cnt.to(DEV)).cpu().numpy()
    torch.cuda.synchronize()
    assert sorted(order.tolist()) == list(range(rows))
    default = [default_row(w, rows) for w in range(rows)]
    c = cnt.numpy().reshape(-1)
    if rows >= 8192:
        assert order.tolist() == default
        return
    per = rows // 8
    for x in range(8):
        ws = list(range(x, per * 8, 8))
        rows_x = [default[w] for w in ws]
        pos = {r: i for i, r in enumerate(rows_x)}
        want = sorted(rows_x, key=lambda r: (-int(c[r]), pos[r]))
        assert [int(order[w]) for w in ws] == want, x
    assert order[per * 8:].tolist() == list(range(per * 8, rows))


@pytest.mark.parametrize("name,heads", [("wan480p", None), ("stress", [0, 9]), ("tiny", None)])
def test_fwd_lists_ordered_matches_plain(name, heads):
    w = WORKLOADS[name]
    x = make_inputs(w, heads=heads)
    q, k, v = (t.to(DEV) for t in (x["q"], x["k"], x["v"]))
    qp, kp = sa.pool_qk(q, k, w.bq, w.bk)
    sel = sa.select_mask(qp, kp, w.k_frac, w.p, kept_lists=True)
    order = sa.row_order(sel["kept_cnt"])
    o1, l1 = sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, return_lse=True)
    o2, l2 = sa.fwd_lists(q, k, v, sel["kept_idx"], sel["kept_cnt"], w.bq, w.bk, return_lse=True, row_order=order)
    torch.cuda.synchronize()
    rows = sel["kept_cnt"].numel()
    print(f"  {name}: {rows} rows, longest first: {rows < 8192}", flush=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
