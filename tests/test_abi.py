"""The C-ABI library: it loads, exports every entry point include/dsa.h
declares, and its host-side argument checks refuse bad calls before any
launch (no GPU work happens in these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
FAKE = ctypes.c_void_p(256)  # a non-NULL pointer that is never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"dsa_kpool_compress", "dsa_index_scores", "dsa_topk_pools", "dsa_expand_selection",
            "dsa_sparse_mla_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_cover_header(lib):
    from dsa_decode_amd import _lib
    assert set(_declared()) == set(_lib.SIGNATURES)


def test_status_strings_and_version(lib):
    assert lib.dsa_abi_version() == 2
    texts = [lib.dsa_status_string(code) for code in range(0, -7, -1)]
    assert all(texts) and len(set(texts)) == len(texts)
    assert lib.dsa_status_string(0) == b"ok"


def test_topk_workspace_init_checks(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_OK
    assert lib.dsa_topk_workspace_init(None, 1024, None) == DSA_ERR_NULL
    assert lib.dsa_topk_workspace_init(FAKE, 0, None) == DSA_OK      # nothing to clear: no launch


def test_binding_constants_match_header():
    # every plain numeric #define of the header has the same value in the binding
    from dsa_decode_amd import _lib
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    defs = dict(re.findall(r"#define\s+(DSA_\w+)\s+(-?\d+)\s*$", text, flags=re.M))
    assert {"DSA_TOPK_COUNTER_BYTES", "DSA_MAX_SELECT_K"} <= set(defs)
    for name, value in defs.items():
        if name in ("DSA_ABI_VERSION",):
            continue
        assert getattr(_lib, name) == int(value), name


def test_split_workspace_sizes(lib):
    from dsa_decode_amd._lib import DSA_TOPK_COUNTER_BYTES
    assert lib.dsa_topk_workspace_bytes(4, 65536, 512) > DSA_TOPK_COUNTER_BYTES
    assert lib.dsa_topk_workspace_bytes(1, 1000, 8) == 0                 # one chunk: no workspace
    assert lib.dsa_sparse_mla_workspace_bytes(4, 64, 512, 2048, 1) > 0
    assert lib.dsa_sparse_mla_workspace_bytes(4, 64, 512, 64, 1) == 0      # one slice: no workspace


def _compress(lib, **kw):
    a = dict(k=FAKE, gate=FAKE, valid=FAKE, ape=FAKE, seq_len=FAKE, B=1, T_max=64, D=32, kpool=4,
             P_max=16, dtype=0, k_pool=FAKE, pool_start=FAKE, pool_valid=FAKE, n_pools=FAKE,
             first_valid=FAKE, stream=None)
    a.update(kw)
    return lib.dsa_kpool_compress(*a.values())


def test_compress_refuses_bad_arguments(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED
    assert _compress(lib, k=None) == DSA_ERR_NULL
    assert _compress(lib, first_valid=None) == DSA_ERR_NULL
    assert _compress(lib, B=0) == DSA_ERR_SHAPE
    assert _compress(lib, P_max=15) == DSA_ERR_SHAPE          # P_max < T_max / kpool
    # kpool above the pages' limit of 8 slots is refused, never truncated
    assert _compress(lib, kpool=9, P_max=64) == DSA_ERR_UNSUPPORTED
    assert _compress(lib, D=36) == DSA_ERR_UNSUPPORTED
    assert _compress(lib, dtype=7) == DSA_ERR_UNSUPPORTED


def _append(lib, **kw):
    a = dict(k=FAKE, gate=FAKE, valid=FAKE, ape=FAKE, seq_len=FAKE, B=1, T_max=64, D=32, kpool=4,
             P_max=16, max_new=1, dtype=0, k_pool=FAKE, pool_start=FAKE, pool_valid=FAKE, n_pools=FAKE,
             first_valid=FAKE, stream=None)
    a.update(kw)
    return lib.dsa_kpool_append(*a.values())


def test_append_refuses_bad_arguments(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED
    assert _append(lib, gate=None) == DSA_ERR_NULL
    assert _append(lib, n_pools=None) == DSA_ERR_NULL
    assert _append(lib, max_new=0) == DSA_ERR_SHAPE
    assert _append(lib, T_max=0) == DSA_ERR_SHAPE
    assert _append(lib, P_max=15) == DSA_ERR_SHAPE
    assert _append(lib, kpool=9, P_max=64) == DSA_ERR_UNSUPPORTED
    assert _append(lib, D=12) == DSA_ERR_UNSUPPORTED
    assert _append(lib, dtype=3) == DSA_ERR_UNSUPPORTED


def _scores(lib, **kw):
    a = dict(q=FAKE, w=FAKE, scale=0.1, k_pool=FAKE, pool_start=FAKE, pool_valid=FAKE, g=FAKE, b=FAKE,
             eps=1e-5, row_seq=FAKE, row_pos=FAKE, Q=1, H=4, D=32, B=1, P_max=16, kpool=4, dtype=0,
             scores=FAKE, stream=None)
    a.update(kw)
    return lib.dsa_index_scores(*a.values())


def test_scores_refuse_bad_arguments(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED
    assert _scores(lib, scores=None) == DSA_ERR_NULL
    assert _scores(lib, Q=0) == DSA_ERR_SHAPE
    assert _scores(lib, D=48) == DSA_ERR_UNSUPPORTED
    assert _scores(lib, H=65) == DSA_ERR_UNSUPPORTED
    assert _scores(lib, kpool=9) == DSA_ERR_UNSUPPORTED


def test_topk_refuses_bad_arguments_and_sizes_workspace(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE
    assert lib.dsa_topk_pools(None, 1, 64, 8, FAKE, None, 0, None) == DSA_ERR_NULL
    assert lib.dsa_topk_pools(FAKE, 1, 64, 0, FAKE, None, 0, None) == DSA_ERR_SHAPE
    assert lib.dsa_topk_pools(FAKE, 1, 64, 2049, FAKE, None, 0, None) == DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_pools(FAKE, 1, 16 * 32768 + 1, 8, FAKE, None, 0, None) == DSA_ERR_UNSUPPORTED
    # a long row is split and needs a workspace
    need = lib.dsa_topk_workspace_bytes(4, 65536, 512)
    assert need >= 4 * 512 * 8
    assert lib.dsa_topk_pools(FAKE, 4, 65536, 512, FAKE, None, 0, None) == DSA_ERR_WORKSPACE
    assert lib.dsa_topk_pools(FAKE, 4, 65536, 512, FAKE, FAKE, need - 1, None) == DSA_ERR_WORKSPACE
    assert lib.dsa_topk_workspace_bytes(4096, 32768, 512) == 0


def test_expand_refuses_bad_arguments(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED
    assert lib.dsa_expand_selection(None, 1, 8, FAKE, FAKE, 1, 64, 4, FAKE, 32, None) == DSA_ERR_NULL
    assert lib.dsa_expand_selection(FAKE, 1, 8, FAKE, FAKE, 1, 64, 4, FAKE, 31, None) == DSA_ERR_SHAPE
    assert lib.dsa_expand_selection(FAKE, 1, 8, FAKE, FAKE, 1, 64, 9, FAKE, 72, None) == DSA_ERR_UNSUPPORTED


def test_topk_expand_refuses_bad_arguments(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE
    call = lambda **kw: lib.dsa_topk_pools_expand(*dict(dict(
        s=FAKE, Q=4, P=65536, K=512, ids=FAKE, rs=FAKE, ps=FAKE, B=4, P_max=65536, kp=4, tok=FAKE,
        W=2048, ws=None, wsb=0, stream=None), **kw).values())
    assert call(tok=None) == DSA_ERR_NULL
    assert call(ps=None) == DSA_ERR_NULL
    assert call(s=None) == DSA_ERR_NULL
    assert call(W=2047) == DSA_ERR_SHAPE            # W < K * kpool
    assert call(kp=9, W=8 * 512 * 2) == DSA_ERR_UNSUPPORTED
    assert call(K=4096, W=4096 * 4) == DSA_ERR_UNSUPPORTED
    assert call() == DSA_ERR_WORKSPACE              # split rows need the workspace


def test_mla_refuses_bad_arguments_and_sizes_workspace(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE
    call = lambda **kw: lib.dsa_sparse_mla_decode(*dict(dict(
        q=FAKE, kv=FAKE, rs=FAKE, ids=FAKE, Q=4, Hm=64, Dl=512, B=4, T=1024, W=2048, sc=0.04, dt=1,
        out=FAKE, lse=None, ws=None, wsb=0, stream=None), **kw).values())
    assert call(out=None) == DSA_ERR_NULL
    assert call(W=0) == DSA_ERR_SHAPE
    assert call(Dl=96) == DSA_ERR_UNSUPPORTED
    assert call(Hm=129) == DSA_ERR_UNSUPPORTED
    need = lib.dsa_sparse_mla_workspace_bytes(4, 64, 512, 2048, 1)
    assert need > 0
    assert call() == DSA_ERR_WORKSPACE
    assert call(ws=FAKE, wsb=need - 1) == DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_mla_workspace_bytes(1, 4, 64, 32, 0) == 0   # fp32 path: no split


def _paged(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, scale=FAKE, bt=FAKE, max_pages=4, page_size=64, num_pages=8, row_seq=FAKE,
             tok=FAKE, Q=2, Hm=64, Dl=512, B=2, W=256, sm=0.04, dtype=2, out=FAKE, lse=None, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dsa_sparse_mla_decode_paged(*a.values())


def test_paged_mla_refuses_bad_arguments_and_sizes_workspace(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE
    assert _paged(lib, bt=None) == DSA_ERR_NULL
    assert _paged(lib, scale=None) == DSA_ERR_NULL            # fp8 pages need their scales
    assert _paged(lib, page_size=0) == DSA_ERR_SHAPE
    assert _paged(lib, num_pages=0) == DSA_ERR_SHAPE
    assert _paged(lib, dtype=0) == DSA_ERR_UNSUPPORTED        # fp32 pages are not a paged format
    assert _paged(lib, Dl=256) == DSA_ERR_UNSUPPORTED
    assert _paged(lib, Hm=24) == DSA_ERR_UNSUPPORTED
    assert _paged(lib, ws=None) == DSA_ERR_WORKSPACE
    assert _paged(lib, ws_bytes=16) == DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_mla_paged_workspace_bytes(2, 64, 512, 256) > 0
    assert lib.dsa_sparse_mla_paged_workspace_bytes(2, 64, 512, 128) == 0   # one id slice of 128
    # the paged entry splits the ids for any row count (no many-rows path)
    assert lib.dsa_sparse_mla_paged_workspace_bytes(4096, 64, 512, 2048) > 0


def _streamed(lib, **kw):
    a = dict(q=FAKE, w=FAKE, scale=0.1, k_pool=FAKE, ps=FAKE, pv=FAKE, g=FAKE, b=FAKE, eps=1e-5, rs=FAKE, rp=FAKE,
             Q=4096, H=32, D=128, B=1, P_max=32768, kpool=4, dtype=1, K=512, ids=FAKE, tok=FAKE, W=2048, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.dsa_index_topk_pools_expand(*a.values())


def test_streamed_index_topk_refuses_bad_arguments_and_sizes_workspace(lib):
    from dsa_decode_amd._lib import DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE
    assert _streamed(lib, tok=None) == DSA_ERR_NULL
    assert _streamed(lib, W=2047) == DSA_ERR_SHAPE          # W < K * kpool
    assert _streamed(lib, K=0) == DSA_ERR_SHAPE
    assert _streamed(lib, K=4096, W=4 * 4096) == DSA_ERR_UNSUPPORTED
    assert _streamed(lib, D=96) == DSA_ERR_UNSUPPORTED
    assert _streamed(lib, kpool=9, W=9 * 512) == DSA_ERR_UNSUPPORTED
    assert _streamed(lib, ws=None) == DSA_ERR_WORKSPACE
    assert _streamed(lib, ws_bytes=1 << 20) == DSA_ERR_WORKSPACE
    # the prefill chunk: the larger of the filtered path's layout (the top-k
    # counter block, one list of 2048 8-byte keys per row, the 4096 list
    # lengths) and the row-blocked path's (blocks of 512 rows, 64 MiB of
    # scores, no top-k split)
    from dsa_decode_amd._lib import DSA_TOPK_COUNTER_BYTES
    filtered = DSA_TOPK_COUNTER_BYTES + 4096 * 2048 * 8 + 4096 * 4
    assert filtered > 512 * 32768 * 4
    assert lib.dsa_index_topk_workspace_bytes(4096, 32768, 512) == filtered
    # larger select_k: lists of 4096 keys (K = 1024; 1024 rows -> 4 pool ranges
    # per row) and of 8192 keys (K = 2048; 2048 rows -> 2 ranges, 256 MiB of
    # lists, the most the filtered path takes)
    assert lib.dsa_index_topk_workspace_bytes(1024, 32768, 1024) == \
        DSA_TOPK_COUNTER_BYTES + 1024 * 4 * 4096 * 8 + 1024 * 4 * 4
    assert lib.dsa_index_topk_workspace_bytes(2048, 32768, 2048) == \
        DSA_TOPK_COUNTER_BYTES + 2048 * 2 * 8192 * 8 + 2048 * 2 * 4
    # 8192 rows at K = 2048 would take 512 MiB of lists: the row-blocked layout
    assert lib.dsa_index_topk_workspace_bytes(8192, 32768, 2048) == 512 * 32768 * 4
    # few rows: one block, the split top-k's workspace (counter block first) plus the scores
    n = lib.dsa_index_topk_workspace_bytes(4, 65536, 512)
    assert n >= lib.dsa_topk_workspace_bytes(4, 65536, 512) + 4 * 65536 * 4


def test_streamed_workspace_covers_a_ragged_last_block(lib):
    # 1000 rows x 20000 pools: blocks of 832 rows (64 MiB / 80000 B, a multiple of 8)
    # and a last block of 168 rows, whose top-k splits the rows and needs the
    # counter block; the workspace holds the larger of that layout (the larger
    # of the two top-k needs, aligned to 256 B, and one block of scores) and
    # the filtered path's (125 workgroup rows give each row 5 pool ranges of
    # 256 tiles: 5 lists of 2048 keys per row, 10240 slots <= 20000 pools)
    from dsa_decode_amd._lib import DSA_TOPK_COUNTER_BYTES
    R, rem, P, K = 832, 168, 20000, 512
    tk = max(lib.dsa_topk_workspace_bytes(R, P, K), lib.dsa_topk_workspace_bytes(rem, P, K))
    assert lib.dsa_topk_workspace_bytes(rem, P, K) > 0
    blocked = ((tk + 255) // 256) * 256 + R * P * 4
    filtered = DSA_TOPK_COUNTER_BYTES + 1000 * 5 * 2048 * 8 + 1000 * 5 * 4
    assert lib.dsa_index_topk_workspace_bytes(1000, P, K) == max(blocked, filtered)
    # 100 rows: the score kernel gives each row 40 pool ranges, whose lists
    # (40 x 2048 slots) would outgrow the row's 20000 scores, so only the
    # row-blocked layout counts: all rows in one block
    assert lib.dsa_index_topk_workspace_bytes(100, P, K) == \
        ((lib.dsa_topk_workspace_bytes(100, P, K) + 255) // 256) * 256 + 100 * P * 4
