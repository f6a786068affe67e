"""ctypes loader for libdsa.so (the C ABI declared in include/dsa.h).

Argument marshalling only: no computation happens here.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsa.so")

c_int, c_float, c_size_t, c_void_p, c_char_p = (ctypes.c_int, ctypes.c_float, ctypes.c_size_t,
                                               ctypes.c_void_p, ctypes.c_char_p)

# name -> (restype, argtypes); mirrors include/dsa.h
SIGNATURES = {
    "dsa_status_string": (c_char_p, [c_int]),
    "dsa_abi_version": (c_int, []),
    "dsa_kpool_compress": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dsa_kpool_append": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dsa_index_scores": (c_int, [c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                 c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                 c_void_p, c_void_p]),
    "dsa_topk_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "dsa_topk_workspace_init": (c_int, [c_void_p, c_size_t, c_void_p]),
    "dsa_topk_pools": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_size_t,
                               c_void_p]),
    "dsa_expand_selection": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_int,
                                     c_int, c_void_p, c_int, c_void_p]),
    "dsa_topk_pools_expand": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                      c_int, c_int, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "dsa_sparse_mla_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "dsa_sparse_mla_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_float, c_int, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
    "dsa_sparse_mla_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                              c_int, c_int, c_int, c_float, c_int, c_void_p, c_void_p, c_void_p]),
    "dsa_index_topk_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "dsa_index_topk_pools_expand": (c_int, [c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                            c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                            c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "dsa_sparse_mla_paged_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "dsa_sparse_mla_decode_paged": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                            c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_float,
                                            c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
}

DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP, DSA_ERR_TOO_LARGE = (
    0, -1, -2, -3, -4, -5, -6)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_MAX_KPOOL = 8
DSA_MAX_SELECT_K = 2048
DSA_TOPK_COUNTER_BYTES = 262144
DSA_MLA_SCRATCH_BYTES = 33554432

_lib = None


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load(build_if_missing: bool = False) -> ctypes.CDLL:
    """Load libdsa.so; raise (never fall back) if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python dsa_decode_amd/build_lib.py")
        from . import build_lib
        build_lib.build()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != DSA_OK:
        text = load().dsa_status_string(status).decode()
        raise DsaError(fn, status, text)
