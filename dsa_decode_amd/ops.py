"""Thin PyTorch binding of libdsa.so: same names as the C ABI (include/dsa.h).

Each function checks that the tensors are contiguous device tensors of the
right dtype, passes their device pointers and the current HIP stream, and
raises DsaError on a non-zero status.  Outputs may be passed in or are
allocated with torch.empty (every stage writes its whole output).  All
arithmetic runs in the library's kernels; there is no fallback.
"""
from __future__ import annotations

import threading

import torch

from . import _lib
from .layout import pool_cache_pools
from ._lib import (DSA_BF16, DSA_F32, DSA_FP8_E4M3, DSA_MLA_SCRATCH_BYTES, DSA_TOPK_COUNTER_BYTES,  # noqa: F401
                   DsaError, check)

_ACT = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16}


# tensors referenced by the call being bound (see _bind); None outside a bind
_binding = threading.local()


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    keep = getattr(_binding, "keep", None)
    if keep is not None:
        keep.append(t)
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _act_code(t: torch.Tensor) -> int:
    if t.dtype not in _ACT:
        raise ValueError(f"activation dtype {t.dtype} not supported")
    return _ACT[t.dtype]


def dsa_kpool_compress(k, gate, valid, ape, seq_len, kpool: int, P_max: int, out=None):
    """-> dict(k_pool [B, pool_cache_pools(P_max), D] tile-interleaved, pool_start,
    pool_valid [B,P_max], n_pools, first_valid [B])."""
    B, T_max, D = k.shape
    if out is None:
        dev = k.device
        out = dict(k_pool=torch.empty((B, pool_cache_pools(P_max), D), dtype=k.dtype, device=dev),
                   pool_start=torch.empty((B, P_max), dtype=torch.int32, device=dev),
                   pool_valid=torch.empty((B, P_max), dtype=torch.uint8, device=dev),
                   n_pools=torch.empty((B,), dtype=torch.int32, device=dev),
                   first_valid=torch.empty((B,), dtype=torch.int32, device=dev))
    st = _lib.load().dsa_kpool_compress(
        _dev(k, "k", k.dtype), _dev(gate, "gate", k.dtype), _dev(valid, "valid", torch.uint8),
        _dev(ape, "ape", torch.float32), _dev(seq_len, "seq_len", torch.int32),
        B, T_max, D, kpool, P_max, _act_code(k),
        _dev(out["k_pool"], "k_pool", k.dtype), _dev(out["pool_start"], "pool_start", torch.int32),
        _dev(out["pool_valid"], "pool_valid", torch.uint8), _dev(out["n_pools"], "n_pools", torch.int32),
        _dev(out["first_valid"], "first_valid", torch.int32), _stream())
    check("dsa_kpool_compress", st)
    return out


def dsa_kpool_append(k, gate, valid, ape, seq_len, kpool: int, state, max_new_pools: int = 1):
    """Advance the indexer state `state` (the dict dsa_kpool_compress returns:
    k_pool, pool_start, pool_valid, n_pools, first_valid) in place to the new
    lengths seq_len; forms at most max_new_pools pools per sequence."""
    B, T_max, D = k.shape
    P_max = state["pool_start"].shape[1]
    _check_pool_cache(state["k_pool"], B, P_max, D)
    st = _lib.load().dsa_kpool_append(
        _dev(k, "k", k.dtype), _dev(gate, "gate", k.dtype), _dev(valid, "valid", torch.uint8),
        _dev(ape, "ape", torch.float32), _dev(seq_len, "seq_len", torch.int32),
        B, T_max, D, kpool, P_max, int(max_new_pools), _act_code(k),
        _dev(state["k_pool"], "k_pool", k.dtype), _dev(state["pool_start"], "pool_start", torch.int32),
        _dev(state["pool_valid"], "pool_valid", torch.uint8), _dev(state["n_pools"], "n_pools", torch.int32),
        _dev(state["first_valid"], "first_valid", torch.int32), _stream())
    check("dsa_kpool_append", st)
    return state


def dsa_index_scores(q, w, scale: float, k_pool, pool_start, pool_valid, ln_gamma, ln_beta,
                     ln_eps: float, row_seq, row_pos, kpool: int, scores=None):
    """-> scores [Q, P_max] fp32 (-inf = not a candidate); k_pool is the
    tile-interleaved pool cache [B, pool_cache_pools(P_max), D]."""
    Q, H, D = q.shape
    B, P_max = pool_start.shape
    _check_pool_cache(k_pool, B, P_max, D)
    if scores is None:
        scores = torch.empty((Q, P_max), dtype=torch.float32, device=q.device)
    st = _lib.load().dsa_index_scores(
        _dev(q, "q", k_pool.dtype), _dev(w, "w", torch.float32), float(scale),
        _dev(k_pool, "k_pool"), _dev(pool_start, "pool_start", torch.int32),
        _dev(pool_valid, "pool_valid", torch.uint8), _dev(ln_gamma, "ln_gamma", torch.float32),
        _dev(ln_beta, "ln_beta", torch.float32), float(ln_eps), _dev(row_seq, "row_seq", torch.int32),
        _dev(row_pos, "row_pos", torch.int32), Q, H, D, B, P_max, kpool, _act_code(k_pool),
        _dev(scores, "scores", torch.float32), _stream())
    check("dsa_index_scores", st)
    return scores


def _check_pool_cache(k_pool, B: int, P_max: int, D: int) -> None:
    if tuple(k_pool.shape) != (B, pool_cache_pools(P_max), D):
        raise ValueError(f"k_pool has shape {tuple(k_pool.shape)}, expected the pool cache "
                         f"{(B, pool_cache_pools(P_max), D)}")


def dsa_topk_workspace_bytes(Q: int, P: int, K: int) -> int:
    return int(_lib.load().dsa_topk_workspace_bytes(Q, P, K))


def dsa_topk_workspace_init(workspace) -> None:
    """Zero the counter block of a top-k workspace on the current stream (a
    fill kernel); marks the tensor as a top-k workspace for the calls below."""
    st = _lib.load().dsa_topk_workspace_init(_dev(workspace, "workspace"),
                                             workspace.numel() * workspace.element_size(), _stream())
    check("dsa_topk_workspace_init", st)
    workspace._dsa_topk_ready = True


def topk_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A top-k workspace of nbytes (at least 1) with its counter block zeroed."""
    ws = torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)
    dsa_topk_workspace_init(ws)
    return ws


def _topk_ws(workspace, need: int, device):
    """The workspace for a top-k call: a new zeroed one when none is given;
    one passed in must come from topk_workspace / dsa_topk_workspace_init
    (its counter block starts at zero) and be large enough."""
    if workspace is None:
        return topk_workspace(need, device) if need else None
    if not getattr(workspace, "_dsa_topk_ready", False):
        raise ValueError("a top-k workspace must be made by ops.topk_workspace or passed through "
                         "ops.dsa_topk_workspace_init first (its counter block must start at zero)")
    return workspace


def dsa_topk_pools(scores, K: int, pool_ids=None, workspace=None):
    """-> pool_ids [Q, K] int32, (score desc, index asc), -1 padded."""
    Q, P = scores.shape
    if pool_ids is None:
        pool_ids = torch.empty((Q, K), dtype=torch.int32, device=scores.device)
    workspace = _topk_ws(workspace, dsa_topk_workspace_bytes(Q, P, K), scores.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dsa_topk_pools(_dev(scores, "scores", torch.float32), Q, P, K,
                                    _dev(pool_ids, "pool_ids", torch.int32), ws_ptr, ws_bytes, _stream())
    check("dsa_topk_pools", st)
    return pool_ids


def dsa_topk_pools_expand(scores, K: int, row_seq, pool_start, kpool: int, W: int, pool_ids=None,
                          token_ids=None, workspace=None):
    """dsa_topk_pools then dsa_expand_selection in one launch -> (pool_ids [Q, K],
    token_ids [Q, W])."""
    Q, P = scores.shape
    B, P_max = pool_start.shape
    if pool_ids is None:
        pool_ids = torch.empty((Q, K), dtype=torch.int32, device=scores.device)
    if token_ids is None:
        token_ids = torch.empty((Q, W), dtype=torch.int32, device=scores.device)
    workspace = _topk_ws(workspace, dsa_topk_workspace_bytes(Q, P, K), scores.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dsa_topk_pools_expand(
        _dev(scores, "scores", torch.float32), Q, P, K, _dev(pool_ids, "pool_ids", torch.int32),
        _dev(row_seq, "row_seq", torch.int32), _dev(pool_start, "pool_start", torch.int32), B, P_max, kpool,
        _dev(token_ids, "token_ids", torch.int32), W, ws_ptr, ws_bytes, _stream())
    check("dsa_topk_pools_expand", st)
    return pool_ids, token_ids


def dsa_index_topk_workspace_bytes(Q: int, P_max: int, K: int) -> int:
    return int(_lib.load().dsa_index_topk_workspace_bytes(Q, P_max, K))


def dsa_index_topk_pools_expand(q, w, scale: float, k_pool, pool_start, pool_valid, ln_gamma, ln_beta,
                                ln_eps: float, row_seq, row_pos, kpool: int, K: int, W: int, pool_ids=None,
                                token_ids=None, workspace=None):
    """dsa_index_scores then dsa_topk_pools_expand without the [Q, P_max] score
    tensor -> (pool_ids [Q, K], token_ids [Q, W]), bit-identical to the two
    calls: on the many-row score kernel's shapes the kernel keeps per-row
    candidate lists instead of scores, elsewhere the rows run in blocks of at
    most 64 MiB of scores.  A workspace passed in must come from
    topk_workspace (the top-k counters at its start must be zero)."""
    Q, H, D = q.shape
    B, P_max = pool_start.shape
    _check_pool_cache(k_pool, B, P_max, D)
    if pool_ids is None:
        pool_ids = torch.empty((Q, K), dtype=torch.int32, device=q.device)
    if token_ids is None:
        token_ids = torch.empty((Q, W), dtype=torch.int32, device=q.device)
    workspace = _topk_ws(workspace, dsa_index_topk_workspace_bytes(Q, P_max, K), q.device)
    st = _lib.load().dsa_index_topk_pools_expand(
        _dev(q, "q", k_pool.dtype), _dev(w, "w", torch.float32), float(scale), _dev(k_pool, "k_pool"),
        _dev(pool_start, "pool_start", torch.int32), _dev(pool_valid, "pool_valid", torch.uint8),
        _dev(ln_gamma, "ln_gamma", torch.float32), _dev(ln_beta, "ln_beta", torch.float32), float(ln_eps),
        _dev(row_seq, "row_seq", torch.int32), _dev(row_pos, "row_pos", torch.int32), Q, H, D, B, P_max, kpool,
        _act_code(k_pool), K, _dev(pool_ids, "pool_ids", torch.int32), _dev(token_ids, "token_ids", torch.int32),
        W, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    check("dsa_index_topk_pools_expand", st)
    return pool_ids, token_ids


def dsa_expand_selection(pool_ids, row_seq, pool_start, kpool: int, W: int, token_ids=None):
    """-> token_ids [Q, W] int32 (-1 = invalid, every column written)."""
    Q, K = pool_ids.shape
    B, P_max = pool_start.shape
    if token_ids is None:
        token_ids = torch.empty((Q, W), dtype=torch.int32, device=pool_ids.device)
    st = _lib.load().dsa_expand_selection(
        _dev(pool_ids, "pool_ids", torch.int32), Q, K, _dev(row_seq, "row_seq", torch.int32),
        _dev(pool_start, "pool_start", torch.int32), B, P_max, kpool,
        _dev(token_ids, "token_ids", torch.int32), W, _stream())
    check("dsa_expand_selection", st)
    return token_ids


def dsa_sparse_mla_workspace_bytes(Q: int, Hm: int, Dl: int, W: int, dtype: int) -> int:
    return int(_lib.load().dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W, dtype))


def dsa_sparse_mla_decode(q_lat, kv, row_seq, token_ids, sm_scale: float, out=None, lse=None,
                          workspace=None, want_lse: bool = True):
    """-> (out [Q, Hm, Dl] act, lse [Q, Hm] fp32 or None)."""
    Q, Hm, Dl = q_lat.shape
    B, T_max, Dl2 = kv.shape
    if Dl2 != Dl:
        raise ValueError("q_lat and kv disagree on Dl")
    W = token_ids.shape[1]
    code = _act_code(kv)
    if out is None:
        out = torch.empty((Q, Hm, Dl), dtype=kv.dtype, device=kv.device)
    if lse is None and want_lse:
        lse = torch.empty((Q, Hm), dtype=torch.float32, device=kv.device)
    need = dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W, code)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=kv.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dsa_sparse_mla_decode(
        _dev(q_lat, "q_lat", kv.dtype), _dev(kv, "kv"), _dev(row_seq, "row_seq", torch.int32),
        _dev(token_ids, "token_ids", torch.int32), Q, Hm, Dl, B, T_max, W, float(sm_scale), code,
        _dev(out, "out", kv.dtype), _dev(lse, "lse", torch.float32) if lse is not None else None,
        ws_ptr, ws_bytes, _stream())
    check("dsa_sparse_mla_decode", st)
    return out, lse


def dsa_sparse_mla_decode_noalloc(q_lat, kv, row_seq, token_ids, sm_scale: float, out, lse=None):
    """dsa_sparse_mla_decode with the split partials in the library's fixed
    per-GPU buffer (no workspace; the caller passes out and lse)."""
    Q, Hm, Dl = q_lat.shape
    B, T_max, Dl2 = kv.shape
    if Dl2 != Dl:
        raise ValueError("q_lat and kv disagree on Dl")
    st = _lib.load().dsa_sparse_mla_decode_noalloc(
        _dev(q_lat, "q_lat", kv.dtype), _dev(kv, "kv"), _dev(row_seq, "row_seq", torch.int32),
        _dev(token_ids, "token_ids", torch.int32), Q, Hm, Dl, B, T_max, token_ids.shape[1], float(sm_scale),
        _act_code(kv), _dev(out, "out", kv.dtype), _dev(lse, "lse", torch.float32) if lse is not None else None,
        _stream())
    check("dsa_sparse_mla_decode_noalloc", st)
    return out, lse


def dsa_sparse_mla_paged_workspace_bytes(Q: int, Hm: int, Dl: int, W: int) -> int:
    return int(_lib.load().dsa_sparse_mla_paged_workspace_bytes(Q, Hm, Dl, W))


def dsa_sparse_mla_decode_paged(q_lat, kv_pages, kv_scale, block_table, page_size: int, row_seq, token_ids,
                                sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Sparse MLA over a paged latent cache: kv_pages [num_pages, page_size, Dl]
    bf16, or uint8 OCP FP8 E4M3 codes with kv_scale [num_pages, page_size] fp32;
    block_table [B, max_pages] int32.  -> (out [Q, Hm, Dl] bf16, lse [Q, Hm])."""
    Q, Hm, Dl = q_lat.shape
    num_pages, ps, Dl2 = kv_pages.shape
    if Dl2 != Dl or ps != page_size:
        raise ValueError("kv_pages disagrees with q_lat / page_size")
    B, max_pages = block_table.shape
    W = token_ids.shape[1]
    if kv_pages.dtype == torch.bfloat16:
        code, sc_ptr = DSA_BF16, None
    elif kv_pages.dtype == torch.uint8:
        if kv_scale is None or tuple(kv_scale.shape) != (num_pages, page_size):
            raise ValueError("fp8 pages need kv_scale [num_pages, page_size]")
        code, sc_ptr = DSA_FP8_E4M3, _dev(kv_scale, "kv_scale", torch.float32)
    else:
        raise ValueError(f"kv_pages dtype {kv_pages.dtype} not supported")
    if out is None:
        out = torch.empty((Q, Hm, Dl), dtype=torch.bfloat16, device=q_lat.device)
    if lse is None and want_lse:
        lse = torch.empty((Q, Hm), dtype=torch.float32, device=q_lat.device)
    need = dsa_sparse_mla_paged_workspace_bytes(Q, Hm, Dl, W)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.load().dsa_sparse_mla_decode_paged(
        _dev(q_lat, "q_lat", torch.bfloat16), _dev(kv_pages, "kv_pages"), sc_ptr,
        _dev(block_table, "block_table", torch.int32), max_pages, page_size, num_pages,
        _dev(row_seq, "row_seq", torch.int32), _dev(token_ids, "token_ids", torch.int32), Q, Hm, Dl, B, W,
        float(sm_scale), code, _dev(out, "out", torch.bfloat16),
        _dev(lse, "lse", torch.float32) if lse is not None else None, ws_ptr, ws_bytes, _stream())
    check("dsa_sparse_mla_decode_paged", st)
    return out, lse


# ----------------------------------------------------------------------------
# Pre-bound calls: the same entry points with their argument tuple marshalled
# once, for loops that launch the same stage many times (benchmarks, serving
# steps).  Calling the result launches on the stream captured at bind time.
class BoundCall:
    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name: str, args: tuple, keep: tuple = ()):
        self.name = name
        self.fn = getattr(_lib.load(), name)
        self.args = args
        self.keep = keep  # the tensors behind the pointers in args, alive as long as the call

    def __call__(self) -> None:
        st = self.fn(*self.args)
        if st:
            check(self.name, st)


def _bind(name: str, build) -> BoundCall:
    """A BoundCall whose argument tuple build() marshals; every tensor that
    build() turns into a pointer is kept with the call, so that no buffer it
    launches on can be freed while the call exists."""
    _binding.keep = []
    try:
        args = build()
        keep = tuple(_binding.keep)
    finally:
        _binding.keep = None
    return BoundCall(name, args, keep)


def bind_index_scores(q, w, scale, k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq,
                      row_pos, kpool, scores) -> BoundCall:
    Q, H, D = q.shape
    B, P_max = pool_start.shape
    _check_pool_cache(k_pool, B, P_max, D)
    return _bind("dsa_index_scores", lambda: (
        _dev(q, "q", k_pool.dtype), _dev(w, "w", torch.float32), float(scale), _dev(k_pool, "k_pool"),
        _dev(pool_start, "pool_start", torch.int32), _dev(pool_valid, "pool_valid", torch.uint8),
        _dev(ln_gamma, "ln_gamma", torch.float32), _dev(ln_beta, "ln_beta", torch.float32), float(ln_eps),
        _dev(row_seq, "row_seq", torch.int32), _dev(row_pos, "row_pos", torch.int32), Q, H, D, B, P_max,
        kpool, _act_code(k_pool), _dev(scores, "scores", torch.float32), _stream()))


def bind_topk_pools(scores, K, pool_ids, workspace) -> BoundCall:
    Q, P = scores.shape
    workspace = _topk_ws(workspace, max(1, dsa_topk_workspace_bytes(Q, P, K)), scores.device)
    return _bind("dsa_topk_pools", lambda: (
        _dev(scores, "scores", torch.float32), Q, P, K, _dev(pool_ids, "pool_ids", torch.int32),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))


def bind_topk_pools_expand(scores, K, pool_ids, row_seq, pool_start, kpool, token_ids, workspace) -> BoundCall:
    Q, P = scores.shape
    workspace = _topk_ws(workspace, max(1, dsa_topk_workspace_bytes(Q, P, K)), scores.device)
    B, P_max = pool_start.shape
    return _bind("dsa_topk_pools_expand", lambda: (
        _dev(scores, "scores", torch.float32), Q, P, K, _dev(pool_ids, "pool_ids", torch.int32),
        _dev(row_seq, "row_seq", torch.int32), _dev(pool_start, "pool_start", torch.int32), B, P_max, kpool,
        _dev(token_ids, "token_ids", torch.int32), token_ids.shape[1],
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))


def bind_expand_selection(pool_ids, row_seq, pool_start, kpool, token_ids) -> BoundCall:
    Q, K = pool_ids.shape
    B, P_max = pool_start.shape
    return _bind("dsa_expand_selection", lambda: (
        _dev(pool_ids, "pool_ids", torch.int32), Q, K, _dev(row_seq, "row_seq", torch.int32),
        _dev(pool_start, "pool_start", torch.int32), B, P_max, kpool, _dev(token_ids, "token_ids", torch.int32),
        token_ids.shape[1], _stream()))


def bind_sparse_mla_decode(q_lat, kv, row_seq, token_ids, sm_scale, out, lse, workspace) -> BoundCall:
    Q, Hm, Dl = q_lat.shape
    B, T_max, _ = kv.shape
    return _bind("dsa_sparse_mla_decode", lambda: (
        _dev(q_lat, "q_lat", kv.dtype), _dev(kv, "kv"), _dev(row_seq, "row_seq", torch.int32),
        _dev(token_ids, "token_ids", torch.int32), Q, Hm, Dl, B, T_max, token_ids.shape[1], float(sm_scale),
        _act_code(kv), _dev(out, "out", kv.dtype), _dev(lse, "lse", torch.float32) if lse is not None else None,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))


def bind_sparse_mla_decode_paged(q_lat, kv_pages, kv_scale, block_table, page_size, row_seq, token_ids, sm_scale,
                                 out, lse, workspace) -> BoundCall:
    Q, Hm, Dl = q_lat.shape
    num_pages, ps, Dl2 = kv_pages.shape
    if Dl2 != Dl or ps != page_size:
        raise ValueError("kv_pages disagrees with q_lat / page_size")
    B, max_pages = block_table.shape
    if kv_pages.dtype == torch.bfloat16:
        code, sc_ptr = DSA_BF16, None
    elif kv_pages.dtype == torch.uint8:
        if kv_scale is None or tuple(kv_scale.shape) != (num_pages, page_size):
            raise ValueError("fp8 pages need kv_scale [num_pages, page_size]")
        code, sc_ptr = DSA_FP8_E4M3, _dev(kv_scale, "kv_scale", torch.float32)
    else:
        raise ValueError(f"kv_pages dtype {kv_pages.dtype} not supported")
    return _bind("dsa_sparse_mla_decode_paged", lambda: (
        _dev(q_lat, "q_lat", torch.bfloat16), _dev(kv_pages, "kv_pages"), sc_ptr,
        _dev(block_table, "block_table", torch.int32), max_pages, page_size, num_pages,
        _dev(row_seq, "row_seq", torch.int32), _dev(token_ids, "token_ids", torch.int32), Q, Hm, Dl, B,
        token_ids.shape[1], float(sm_scale), code, _dev(out, "out", torch.bfloat16),
        _dev(lse, "lse", torch.float32) if lse is not None else None,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))


def bind_kpool_append(k, gate, valid, ape, seq_len, kpool, state, max_new_pools=1) -> BoundCall:
    B, T_max, D = k.shape
    P_max = state["pool_start"].shape[1]
    _check_pool_cache(state["k_pool"], B, P_max, D)
    return _bind("dsa_kpool_append", lambda: (
        _dev(k, "k", k.dtype), _dev(gate, "gate", k.dtype), _dev(valid, "valid", torch.uint8),
        _dev(ape, "ape", torch.float32), _dev(seq_len, "seq_len", torch.int32),
        B, T_max, D, kpool, P_max, int(max_new_pools), _act_code(k),
        _dev(state["k_pool"], "k_pool", k.dtype), _dev(state["pool_start"], "pool_start", torch.int32),
        _dev(state["pool_valid"], "pool_valid", torch.uint8), _dev(state["n_pools"], "n_pools", torch.int32),
        _dev(state["first_valid"], "first_valid", torch.int32), _stream()))


def bind_index_topk_pools_expand(q, w, scale, k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq,
                                 row_pos, kpool, K, pool_ids, token_ids, workspace) -> BoundCall:
    Q, H, D = q.shape
    B, P_max = pool_start.shape
    _check_pool_cache(k_pool, B, P_max, D)
    workspace = _topk_ws(workspace, max(1, dsa_index_topk_workspace_bytes(Q, P_max, K)), q.device)
    return _bind("dsa_index_topk_pools_expand", lambda: (
        _dev(q, "q", k_pool.dtype), _dev(w, "w", torch.float32), float(scale), _dev(k_pool, "k_pool"),
        _dev(pool_start, "pool_start", torch.int32), _dev(pool_valid, "pool_valid", torch.uint8),
        _dev(ln_gamma, "ln_gamma", torch.float32), _dev(ln_beta, "ln_beta", torch.float32), float(ln_eps),
        _dev(row_seq, "row_seq", torch.int32), _dev(row_pos, "row_pos", torch.int32), Q, H, D, B, P_max, kpool,
        _act_code(k_pool), K, _dev(pool_ids, "pool_ids", torch.int32), _dev(token_ids, "token_ids", torch.int32),
        token_ids.shape[1], _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))
