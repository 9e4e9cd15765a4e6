"""Host-side checks of the C ABI (no GPU): the library loads, exports every declared symbol,
and rejects invalid arguments with the documented codes before touching the GPU."""

import ctypes
import math
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_lib_module():
    """The ctypes table (_lib.py) loaded by path, without the package's torch binding, so these
    tests also run under a preloaded sanitizer runtime."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "sa_abi_lib", os.path.join(ROOT, "block_sparse_attention_query_amd", "_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_lib = _load_lib_module()
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsparse_attn.so not built")

# Fake device addresses: never dereferenced because every call below fails validation first.
P = 1 << 20      # 256-byte aligned
P_ODD = P + 8    # not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 25
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.SIGNATURES) == names


def test_error_strings():
    lib = _lib.lib()
    assert lib.sparse_attn_error_string(0) == b"ok"
    for c in (-1, -2, -3):
        assert lib.sparse_attn_error_string(c)
    assert lib.sparse_attn_error_string(17) == b"unknown error code"


def test_topk_count_matches_oracle_rule():
    lib = _lib.lib()
    for nkb in (1, 7, 16, 256, 512, 1182, 8192):
        for k_frac in (0.0, 0.01, 0.03, 0.05, 0.1, 0.25, 0.3, 1 / 3, 0.5, 0.6, 0.9, 0.999, 1.0):
            assert lib.sparse_attn_topk_count(k_frac, nkb) == oracle.topk_count(k_frac, nkb), (k_frac, nkb)
    assert lib.sparse_attn_topk_count(-0.1, 10) == -1
    assert lib.sparse_attn_topk_count(1.5, 10) == -1
    assert lib.sparse_attn_topk_count(float("nan"), 10) == -1


def test_workspace_size():
    lib = _lib.lib()
    rows, nkb = 40 * 591, 1182
    want = math.ceil(rows * nkb * 4 / 256) * 256 + math.ceil(rows * 4 / 256) * 256
    assert lib.sparse_attn_fwd_workspace_size(1, 40, 75600, 128, 64) == want
    assert lib.sparse_attn_fwd_workspace_size(0, 40, 75600, 128, 64) == 0


def _pool(**kw):
    a = dict(q=P, k=P, dtype=0, B=1, H=2, N=1024, d=64, Bq=64, Bk=64, qp=P, kp=P, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_pool_qk(*a.values())


def _select(**kw):
    a = dict(qp=P, kp=P, B=1, H=2, nqb=16, nkb=16, d=64, scale=0.125, k_frac=0.25, p=0.6, probs=P, mask=P,
             idx=None, cnt=None, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_select_mask(*a.values())


def _fwd(**kw):
    ws = _lib.lib().sparse_attn_fwd_workspace_size(1, 2, 1024, 64, 64)
    a = dict(q=P, k=P, v=P, dtype=0, mask=P, B=1, H=2, N=1024, d=64, Bq=64, Bk=64, scale=0.125, o=P, lse=None,
             ws=P, ws_bytes=ws, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kp=None), -1), (dict(N=0), -1), (dict(B=-1), -1),
    (dict(d=96), -2), (dict(Bq=32), -2), (dict(Bk=256), -2), (dict(dtype=5), -2), (dict(q=P_ODD), -1),
    (dict(B=300, H=300), -2),
])
def test_pool_rejects(kw, code):
    assert _pool(**kw) == code
    assert _lib.lib().sparse_attn_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(qp=None), -1), (dict(mask=None), -1), (dict(probs=None, nkb=1281), -1), (dict(idx=P), -1), (dict(cnt=P), -1),
    (dict(nkb=0), -1), (dict(d=32), -2), (dict(nkb=8193), -2), (dict(k_frac=-0.01), -1), (dict(k_frac=1.01), -1),
    (dict(p=float("nan")), -1), (dict(p=1.5), -1), (dict(scale=0.0), -1), (dict(scale=float("inf")), -1),
])
def test_select_rejects(kw, code):
    assert _select(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), -1), (dict(mask=None), -1), (dict(ws=None), -1), (dict(o=None), -1), (dict(N=-5), -1),
    (dict(d=80), -2), (dict(Bk=128), -2), (dict(Bq=256), -2), (dict(dtype=2), -2), (dict(ws_bytes=100), -1),
    (dict(ws=P + 16), -1), (dict(o=P_ODD), -1), (dict(scale=-1.0), -1),
])
def test_fwd_rejects(kw, code):
    assert _fwd(**kw) == code


def _fwd_lists(**kw):
    a = dict(q=P, k=P, v=P, dtype=0, idx=P, cnt=P, B=1, H=2, N=1024, d=64, Bq=64, Bk=64, scale=0.125, o=P,
             lse=None, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_fwd_lists(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), -1), (dict(cnt=None), -1), (dict(q=None), -1), (dict(d=48), -2), (dict(Bk=32), -2),
    (dict(k=P_ODD), -1), (dict(scale=float("nan")), -1), (dict(H=0), -1),
])
def test_fwd_lists_rejects(kw, code):
    assert _fwd_lists(**kw) == code


def _row_order(**kw):
    a = dict(cnt=P, B=1, H=2, nqb=16, order=P, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_row_order(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(cnt=None), -1), (dict(order=None), -1), (dict(B=0), -1), (dict(H=-1), -1), (dict(nqb=0), -1),
    (dict(B=1 << 16, H=1 << 16, nqb=2), -2),
])
def test_row_order_rejects(kw, code):
    assert _row_order(**kw) == code


def _fwd_lists_ordered(**kw):
    a = dict(q=P, k=P, v=P, dtype=0, idx=P, cnt=P, order=P, B=1, H=2, N=1024, d=64, Bq=64, Bk=64, scale=0.125, o=P,
             lse=None, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_fwd_lists_ordered(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(order=None), -1), (dict(idx=None), -1), (dict(cnt=None), -1), (dict(v=None), -1), (dict(d=48), -2),
    (dict(Bq=32), -2), (dict(o=P_ODD), -1), (dict(scale=0.0), -1),
])
def test_fwd_lists_ordered_rejects(kw, code):
    assert _fwd_lists_ordered(**kw) == code


def _fwd_lists_window(**kw):
    a = dict(q=P, k=P, v=P, dtype=0, idx=P, cnt=P, B=1, H=2, N=6400, d=128, Bq=128, Bk=64, window=100, scale=0.125,
             o=P, lse=None, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_fwd_lists_window(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), -1), (dict(cnt=None), -1), (dict(o=None), -1), (dict(d=48), -2), (dict(Bk=128), -2),
    (dict(dtype=1), -2), (dict(window=0), -1), (dict(window=-100), -1), (dict(window=99), -1),
    (dict(window=130), -1), (dict(window=128), -2), (dict(window=200), -2), (dict(H=0), -1),
    (dict(N=20_000_000, window=200), -2),
])
def test_fwd_lists_window_rejects(kw, code):
    assert _fwd_lists_window(**kw) == code


def _fwd_noalloc(**kw):
    a = dict(q=P, k=P, v=P, dtype=0, mask=P, B=1, H=2, N=1000, d=128, Bq=128, Bk=64, scale=0.125, o=P, lse=None,
             stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_fwd_noalloc(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), -1), (dict(q=None), -1), (dict(o=P_ODD), -1), (dict(d=48), -2), (dict(Bq=32), -2),
    (dict(Bk=128), -2), (dict(dtype=2), -2), (dict(scale=-1.0), -1), (dict(N=0), -1),
    # one head's lists (4096 x 8192 int32 = 128 MiB) exceed the 32 MiB scratch: rejected before any HIP call
    (dict(N=524288), -2),
])
def test_fwd_noalloc_rejects(kw, code):
    assert _fwd_noalloc(**kw) == code


def test_fwd_noalloc_names_the_scratch_limit():
    assert _fwd_noalloc(N=300000) == -2
    msg = _lib.lib().sparse_attn_last_error().decode()
    assert "scratch" in msg and str(_lib.SA_NOALLOC_SCRATCH_BYTES) in msg


def _squad(**kw):
    a = dict(q=P, k=P, v=P, dtype=0, B=1, H=2, N=6400, d=128, Bq=128, window=100, pass_=1, scale=0.125, o=P,
             lse=None, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_squad_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(v=P_ODD), -1), (dict(dtype=1), -2), (dict(d=48), -2),
    (dict(Bq=32), -2), (dict(scale=0.0), -1), (dict(pass_=2), -1), (dict(pass_=-1), -1), (dict(window=0), -1),
    (dict(window=6401), -1), (dict(window=99), -1), (dict(window=128), -2), (dict(N=20_000_000, window=200), -2),
    (dict(H=0), -1),
])
def test_squad_fwd_rejects(kw, code):
    assert _squad(**kw) == code


def test_squad_local_pass_takes_any_window():
    """The local pass has no divisibility or run-count condition: the same bad-alignment check
    is what fails first."""
    assert _squad(pass_=0, window=99, o=P_ODD) == -1
    assert "aligned" in _lib.lib().sparse_attn_last_error().decode()


def test_last_error_names_the_problem():
    assert _fwd(ws_bytes=100) == -1
    msg = _lib.lib().sparse_attn_last_error().decode()
    assert "workspace" in msg and "100" in msg
    with pytest.raises(_lib.SparseAttnError) as ei:
        _lib.check(_fwd(d=80))
    assert ei.value.code == -2 and "80" in str(ei.value)


def _pattern(**kw):
    a = dict(patterns=1, window=128, band=0, period=0, B=1, H=2, N=1024, Bq=128, Bk=64, mask=P, idx=None, cnt=None,
             stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_pattern_mask(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), -1), (dict(idx=P), -1), (dict(cnt=P), -1), (dict(N=0), -1), (dict(patterns=0), -1),
    (dict(patterns=32), -1), (dict(window=0), -1), (dict(patterns=4, band=-1), -1), (dict(patterns=8, band=3), -1),
    (dict(patterns=16, period=-2), -1), (dict(Bq=32), -2), (dict(Bk=256), -2), (dict(N=64 * 8193), -2),
])
def test_pattern_mask_rejects(kw, code):
    assert _pattern(**kw) == code


def _wt(**kw):
    a = dict(x=P, dtype=0, B=1, H=2, N=1024, d=64, window=128, inverse=0, out=P + 4096, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_window_transpose(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(out=None), -1), (dict(window=0), -1), (dict(window=100), -1), (dict(out=P), -1),
    (dict(x=P_ODD), -1), (dict(d=96), -2), (dict(dtype=3), -2),
])
def test_window_transpose_rejects(kw, code):
    assert _wt(**kw) == code


def _bwd(**kw):
    ws = _lib.lib().sparse_attn_bwd_workspace_size(1, 2, 1024, 64, 64)
    a = dict(q=P, k=P, v=P, o=P, g=P, lse=P, dtype=0, mask=P, B=1, H=2, N=1024, d=64, Bq=64, Bk=64, scale=0.125,
             dq=P, dk=P, dv=P, ws=P, ws_bytes=ws, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_bwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), -1), (dict(g=None), -1), (dict(lse=None), -1), (dict(mask=None), -1), (dict(dk=None), -1),
    (dict(ws=None), -1), (dict(ws_bytes=64), -1), (dict(ws=P + 16), -1), (dict(dv=P_ODD), -1), (dict(dtype=1), -2),
    (dict(d=32), -2), (dict(Bk=128), -2), (dict(scale=0.0), -1),
])
def test_bwd_rejects(kw, code):
    assert _bwd(**kw) == code


def test_bwd_workspace_size():
    lib = _lib.lib()
    bh, n, bq = 2, 1000, 128
    nqb, nkb = 8, 16
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = al(bh * nqb * nkb * 4) + al(bh * nqb * 4) + al(bh * nkb * nqb * 4) + al(bh * nkb * 4) + \
        al(bh * nkb * nqb) + 2 * al(bh * nqb * bq * 4)
    assert lib.sparse_attn_bwd_workspace_size(1, 2, n, bq, 64) == want
    assert lib.sparse_attn_bwd_workspace_size(1, 2, n, 96, 64) == 0


def _probe(**kw):
    ws = _lib.lib().sparse_attn_probe_workspace_size(1, 2, 1024, 64, 64, 2)
    a = dict(q=P, k=P, v=P, o=P, dtype=0, B=1, H=2, N=1024, d=64, Bq=64, scale=0.125, probes=2, ridge=1e-3,
             rank=8, a_out=None, exact_out=None, ws=P, ws_bytes=ws, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_probe_correct(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), -1), (dict(q=None), -1), (dict(ws=None), -1), (dict(ws_bytes=64), -1), (dict(ws=P + 16), -1),
    (dict(o=P_ODD), -1), (dict(a_out=P_ODD), -1), (dict(exact_out=P_ODD), -1), (dict(probes=0), -1),
    (dict(probes=1025), -1), (dict(ridge=0.0), -1), (dict(ridge=float("nan")), -1), (dict(scale=-1.0), -1),
    (dict(dtype=1), -2), (dict(d=96), -2), (dict(Bq=32), -2), (dict(N=0), -1), (dict(rank=0), -1),
    (dict(rank=-3), -1),
])
def test_probe_correct_rejects(kw, code):
    assert _probe(**kw) == code


def test_probe_workspace_size():
    """Partial outputs of S key-block ranges (S minimises rounds of 512 workgroups times key
    blocks per range, at most 24 ranges, at least 4 key blocks per range), the exact probe rows,
    Z^T Z = [X | R]^T [X | R] in float64 (its last d rows only with a rank below d), the factor
    (rows padded to blocks of 8 plus the n reciprocals of its diagonal, an even count of float64),
    A, A^T in bf16 and the bias row."""
    lib = _lib.lib()
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    bh, n, d, bq, probes = 2, 1000, 128, 128, 3
    nkb = 16
    smax = max(1, min(24, nkb // 4))
    costs = [(-(-(bh * probes * S) // 512)) * (-(-nkb // S)) for S in range(1, smax + 1)]
    s = 1 + costs.index(min(costs))
    units = bh * probes * s
    m = d + 1
    fac = (m * (-(-m // 8) * 8) + m + 1) // 2 * 2
    want = al(units * bq * d * 4) + al(units * bq * 8) + al(bh * probes * bq * d * 4) + \
        al(bh * (2 * d + 1) * (2 * d + 1) * 8) + al(bh * fac * 8) + al(bh * m * d * 4) + al(bh * d * d * 2) + \
        al(bh * d * 4)
    assert lib.sparse_attn_probe_workspace_size(1, 2, n, d, bq, probes) == want
    assert lib.sparse_attn_probe_workspace_size(1, 2, n, 96, bq, probes) == 0
    assert lib.sparse_attn_probe_workspace_size(1, 2, n, d, bq, 0) == 0


def _km(**kw):
    ws = _lib.lib().sparse_attn_kmeans_workspace_size(1, 2, 1000, 64, 16)
    a = dict(x=P, dtype=0, B=1, H=2, N=1000, d=64, C=16, iters=2, init=None, cen=P, labels=P, perm=P, off=P, ws=P,
             ws_bytes=ws, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_kmeans(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(cen=None), -1), (dict(perm=None), -1), (dict(ws=None), -1), (dict(ws_bytes=64), -1),
    (dict(ws=P + 16), -1), (dict(x=P_ODD), -1), (dict(C=0), -1), (dict(C=1001), -1), (dict(iters=0), -1),
    (dict(dtype=1), -2), (dict(d=96), -2),
])
def test_kmeans_rejects(kw, code):
    assert _km(**kw) == code


def test_kmeans_rejects_too_many_clusters():
    assert _km(N=5000, C=1025, ws_bytes=1 << 30) == -2


def _csel(**kw):
    a = dict(cq=P, ck=P, off=P, B=1, H=2, Cq=8, Ck=40, d=64, scale=0.125, p=0.9, probs=None, mask=P, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_cluster_select(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), -1), (dict(off=None), -1), (dict(mask=None), -1), (dict(Cq=0), -1), (dict(p=1.5), -1),
    (dict(p=-0.1), -1), (dict(scale=0.0), -1), (dict(d=32), -2), (dict(Ck=1025), -2),
])
def test_cluster_select_rejects(kw, code):
    assert _csel(**kw) == code


def _perm(**kw):
    a = dict(x=P, dtype=0, B=1, H=2, N=1000, d=64, perm=P + 4096, inverse=0, out=P + 8192, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_permute_rows(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(perm=None), -1), (dict(out=P), -1), (dict(out=P_ODD), -1), (dict(d=96), -2),
    (dict(dtype=4), -2),
])
def test_permute_rows_rejects(kw, code):
    assert _perm(**kw) == code


def _cfwd(**kw):
    ws = _lib.lib().sparse_attn_cluster_fwd_workspace_size(1, 2, 1000, 8, 40, 128)
    a = dict(q=P, k=P, v=P, dtype=0, B=1, H=2, N=1000, d=64, qo=P, Cq=8, ko=P, Ck=40, mask=P, q_perm=None, k_perm=None,
             Bq=128, scale=0.125, o=P, lse=None, ws=P, ws_bytes=ws, stream=None)
    a.update(kw)
    return _lib.lib().sparse_attn_cluster_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(qo=None), -1), (dict(mask=None), -1), (dict(ws=None), -1), (dict(ws_bytes=64), -1), (dict(o=None), -1),
    (dict(Cq=0), -1), (dict(Ck=1001), -1), (dict(dtype=1), -2), (dict(Bq=32), -2), (dict(scale=-1.0), -1),
    (dict(N=20_000_000, d=128), -2),
])
def test_cluster_fwd_rejects(kw, code):
    assert _cfwd(**kw) == code


def test_cluster_workspace_sizes():
    lib = _lib.lib()
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    bh, n, d, c = 2, 1000, 64, 40
    cp, nch = 64, 4
    assert lib.sparse_attn_kmeans_workspace_size(1, 2, n, d, c) == \
        2 * al(bh * cp * d * 2) + al(bh * cp * 4) + al(bh * n * 4) + al(bh * nch * c * 4) + al(bh * cp * 4)
    mt = 8 + 8
    assert lib.sparse_attn_cluster_fwd_workspace_size(1, 2, n, 8, 40, 128) == \
        al(bh * mt * 16) + al(bh * 4) + al(bh * 8 * 40 * 4) + al(bh * 8 * 4)
    assert lib.sparse_attn_kmeans_workspace_size(1, 2, n, 96, c) == 0
    assert lib.sparse_attn_cluster_fwd_workspace_size(1, 2, n, 8, 40, 96) == 0


def test_select_fused_limit_matches_header():
    """The binding's limit for leaving out the probabilities is the header's, and the call names it
    when a longer row comes without them."""
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "sparse_attn.h")).read()
    assert int(re.search(r"#define SA_SELECT_FUSED_NKB (\d+)", hdr).group(1)) == _lib.SA_SELECT_FUSED_NKB
    assert _select(probs=None, nkb=_lib.SA_SELECT_FUSED_NKB + 1) == -1
    msg = _lib.lib().sparse_attn_last_error().decode()
    assert "probs" in msg and str(_lib.SA_SELECT_FUSED_NKB) in msg
