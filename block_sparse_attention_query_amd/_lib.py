"""ctypes loader for libsparse_attn.so (built in-tree by ``build.py``)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_attn.so")
# The host tests can point this module at another build of the same ABI (the sanitizer build).
LIB_PATH = os.environ.get("SA_LIB_PATH", LIB_PATH)

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_HIP = -3
SA_BF16 = 0
SA_F32 = 1
SA_PAT_LOCAL, SA_PAT_GLOBAL, SA_PAT_DIAG, SA_PAT_MULTIDIAG, SA_PAT_STRIPE = 1, 2, 4, 8, 16
SA_SELECT_FUSED_NKB = 1280  # longest rows whose selection may leave out the probabilities
SA_SQUAD_LOCAL, SA_SQUAD_GLOBAL = 0, 1
SA_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/sparse_attn.h declares, with (restype, argtypes).
_vp, _i, _d, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
SIGNATURES = {
    "sparse_attn_pool_qk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "sparse_attn_select_mask": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _d, _d, _d, _vp, _vp, _vp, _vp, _vp]),
    "sparse_attn_fwd_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "sparse_attn_fwd": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp, _sz, _vp]),
    "sparse_attn_fwd_noalloc": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp]),
    "sparse_attn_fwd_lists": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp]),
    "sparse_attn_fwd_lists_window": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp]),
    "sparse_attn_row_order": (_i, [_vp, _i, _i, _i, _vp, _vp]),
    "sparse_attn_fwd_lists_ordered": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp]),
    "sparse_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "sparse_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp, _vp, _sz,
                             _vp]),
    "sparse_attn_pattern_mask": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "sparse_attn_window_transpose": (_i, [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "sparse_attn_squad_fwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _d, _vp, _vp, _vp]),
    "sparse_attn_probe_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "sparse_attn_probe_correct": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _d, _i, _d, _i, _vp, _vp, _vp,
                                       _sz, _vp]),
    "sparse_attn_kmeans_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "sparse_attn_kmeans": (_i, [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sparse_attn_cluster_select": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _d, _d, _vp, _vp, _vp]),
    "sparse_attn_permute_rows": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp]),
    "sparse_attn_cluster_fwd_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "sparse_attn_cluster_fwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _i, _d, _vp,
                                     _vp, _vp, _sz, _vp]),
    "sparse_attn_topk_count": (_i, [_d, _i]),
    "sparse_attn_error_string": (ctypes.c_char_p, [_i]),
    "sparse_attn_last_error": (ctypes.c_char_p, []),
}

_LIB = None


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"sparse_attn error {code}: {message}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback path)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_query_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(rc: int) -> None:
    if rc != SA_OK:
        msg = lib().sparse_attn_last_error().decode(errors="replace")
        raise SparseAttnError(rc, msg or lib().sparse_attn_error_string(rc).decode())
