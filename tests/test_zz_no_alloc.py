"""GPU check of sparse_attn_fwd_noalloc, the forward entry point that allocates nothing (its kept
lists live in the library's scratch array): two calls in a row through the C ABI, the second on
a smaller input, each bit-identical to sparse_attn_fwd with a caller workspace."""

import pytest
import torch

import block_sparse_attention_query_amd as sa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(B, H, N, d, bq, dt, density, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, d, generator=g, device=DEV).to(dt) for _ in range(3))
    nqb, nkb = -(-N // bq), -(-N // 64)
    m = (torch.rand(B, H, nqb, nkb, generator=g, device=DEV) < density).to(torch.uint8)
    m[..., 0, :] = 0      # an empty row
    m[..., -1, -1] = 1    # the ragged last key block
    return q, k, v, m


def test_noalloc_matches_fwd_on_two_calls():
    # 40 heads of the 720p grid (75 600 tokens): 2.8 MB of lists per head, so the 32 MiB scratch
    # takes the heads in four groups; then 3 heads of 1000 fp32 tokens, over the first call's lists
    cases = [(1, 40, 75600, 128, 128, torch.bfloat16, 0.05, 1), (1, 3, 1000, 64, 64, torch.float32, 0.3, 2)]
    inputs = [_case(*c) for c in cases]
    outs = []
    for (B, H, N, d, bq, dt, _, _), (q, k, v, m) in zip(cases, inputs):
        print(f"noalloc B={B} H={H} N={N} d={d} bq={bq} {dt}", flush=True)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        sa.fwd_noalloc(q, k, v, m, bq, 64, out=o, lse=lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for (B, H, N, d, bq, dt, _, _), (q, k, v, m), (o, lse) in zip(cases, inputs, outs):
        ro, rl = sa.fwd(q, k, v, m, bq, 64, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ro), (N, (o.float() - ro.float()).abs().max().item())
        assert torch.equal(lse, rl)
